"""GPU parity of decode over a key/value cache (attn_kv_append, attn_decode)
against the float64 oracle's decode step (itself pinned to the forward's row
pos), plus exact special cases."""

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    import oracle
    from tests.gpu_util import TOL, errors


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load()


DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def inputs(B, H, L, D, dtype, seed, qk=("normal", 1.0)):
    """q, k, v [B, H, L, D] in the 16-bit dtype (CPU); the decode query at
    position pos is q[:, :, pos]."""
    q, k, v, _ = workloads.draw((B, H, L, D), qk=qk, seed=seed)
    return tuple(torch.from_numpy(a).to(DT[dtype]) for a in (q, k, v))


def run_decode(q, k, v, pos, Tmax, dtype, fill=None):
    """Prefill cache rows 0 .. pos in one append, then one decode step at pos."""
    B, H, L, D = k.shape
    cache = attn.KVCache(B, H, Tmax, D, DT[dtype], DEV)
    if fill is not None:
        cache.buf.fill_(fill)
    cache.append(k[:, :, :pos + 1].to(DEV), v[:, :, :pos + 1].to(DEV), 0)
    o, lse = cache.decode(q[:, :, pos].contiguous().to(DEV), pos)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, q, k, v, pos, dtype, label):
    f = lambda t: workloads.as_float64(t)
    ro, rl = oracle.attention_decode(f(q)[:, :, pos], f(k), f(v), pos)
    mx, rel = errors(f(o), ro)
    assert np.all(np.isfinite(f(o))), label
    assert mx <= TOL[dtype]["max_abs"], f"{label}: o max-abs {mx:.3e}"
    assert rel <= TOL[dtype]["rel_l2"], f"{label}: o rel-l2 {rel:.3e}"
    # lse is diagnostic, with the forward's bound: the fp16 score operands carry
    # a relative error ~2^-11, so the bound grows with the logit magnitude
    lmx, _ = errors(lse.numpy().astype(np.float64), rl)
    lse_tol = 1e-2 + 1e-3 * float(np.max(np.abs(rl)))
    assert lmx <= lse_tol, f"{label}: lse max-abs {lmx:.3e} > {lse_tol:.3e}"


# positions at and around the 64-key slice boundaries, and the cache's last row
CASES = [(1, 1, 1, 0), (2, 3, 100, 63), (2, 3, 100, 64), (1, 2, 300, 257), (2, 2, 130, 129),
         (1, 1, 64, 63), (3, 1, 200, 199)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,Tmax,pos", CASES)
def test_decode_small(B, H, Tmax, pos, D, dtype):
    q, k, v = inputs(B, H, Tmax, D, dtype, seed=pos + D)
    o, lse = run_decode(q, k, v, pos, Tmax, dtype)
    check(o, lse, q, k, v, pos, dtype, f"{dtype} B{B} H{H} Tmax{Tmax} pos{pos} D{D}")


@pytest.mark.parametrize("pos", [0, 511, 1023])
def test_decode_full_layer(pos):
    """The decode workload's shape, every head checked."""
    w = workloads.WORKLOADS["decode_bf16_b8h12t1024d64"]
    q, k, v = inputs(w.B, w.H, w.T, w.D, w.dtype, seed=0)
    o, lse = run_decode(q, k, v, pos, w.T, w.dtype)
    check(o, lse, q, k, v, pos, w.dtype, f"{w.name} pos {pos}")


def test_decode_peaky_logits():
    q, k, v = inputs(2, 3, 300, 64, "bf16", seed=7, qk=("normal", 3.0))
    o, lse = run_decode(q, k, v, 299, 300, "bf16")
    check(o, lse, q, k, v, 299, "bf16", "peaky")


def test_position_zero_is_v_zero_bitwise():
    q, k, v = inputs(2, 3, 16, 64, "bf16", seed=3)
    o, _ = run_decode(q, k, v, 0, 16, "bf16")
    assert torch.equal(o, v[:, :, 0])


def test_rows_past_pos_are_not_read():
    """Cache bytes past row pos hold NaN patterns; the step must not see them."""
    q, k, v = inputs(2, 2, 200, 64, "bf16", seed=11)
    o1, l1 = run_decode(q, k, v, 150, 200, "bf16", fill=255)
    o2, l2 = run_decode(q, k, v, 150, 200, "bf16", fill=0)
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_token_by_token_generation_matches_the_forward():
    """Append one token per step and decode it: step t equals row t of the
    oracle forward over positions 0 .. t (and of the GPU forward within the
    same tolerance)."""
    B, H, T, D = 2, 3, 70, 64
    q, k, v = inputs(B, H, T, D, "bf16", seed=21)
    cache = attn.KVCache(B, H, T, D, torch.bfloat16, DEV)
    outs = []
    for t in range(T):
        cache.append(k[:, :, t:t + 1].to(DEV), v[:, :, t:t + 1].to(DEV), t)
        o, _ = cache.decode(q[:, :, t].contiguous().to(DEV), t)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    got = np.stack([workloads.as_float64(o) for o in outs], axis=2)      # [B, H, T, D]
    f = lambda t: workloads.as_float64(t)
    ro, _ = oracle.attention_forward(f(q), f(k), f(v))
    mx, rel = errors(got, ro)
    assert mx <= TOL["bf16"]["max_abs"] and rel <= TOL["bf16"]["rel_l2"], (mx, rel)
    g = {n: t.to(DEV) for n, t in dict(q=q, k=k, v=v).items()}
    go, _, _ = attn.forward(g["q"], g["k"], g["v"])
    mx2, _ = errors(got, workloads.as_float64(go.cpu()))
    assert mx2 <= 2 * TOL["bf16"]["max_abs"], mx2


def test_append_writes_rotated_keys_and_values():
    """Cache rows are R_u k_u (fp16, within its rounding) and the values as given;
    rows outside the appended range keep their previous bytes."""
    B, H, Tmax, D, pos0, n = 2, 3, 50, 64, 7, 20
    q, k, v = inputs(B, H, Tmax, D, "bf16", seed=31)
    cache = attn.KVCache(B, H, Tmax, D, torch.bfloat16, DEV)
    cache.buf.fill_(0x7E)
    cache.append(k[:, :, pos0:pos0 + n].to(DEV), v[:, :, pos0:pos0 + n].to(DEV), pos0)
    torch.cuda.synchronize()
    nk = B * H * Tmax * D
    kc = cache.buf[:2 * nk].view(torch.float16).view(B, H, Tmax, D).cpu()
    vc = cache.buf[2 * nk:4 * nk].view(torch.bfloat16).view(B, H, Tmax, D).cpu()
    ref = oracle.rope(workloads.as_float64(k))[:, :, pos0:pos0 + n]
    got = workloads.as_float64(kc[:, :, pos0:pos0 + n])
    assert np.allclose(got, ref, rtol=2.0 ** -10, atol=1e-6)
    assert torch.equal(vc[:, :, pos0:pos0 + n], v[:, :, pos0:pos0 + n])
    untouched = torch.cat([cache.buf[:2 * nk].view(B, H, Tmax, 2 * D)[:, :, :pos0].flatten(),
                           cache.buf[:2 * nk].view(B, H, Tmax, 2 * D)[:, :, pos0 + n:].flatten()])
    assert torch.all(untouched == 0x7E)


def test_steps_at_different_positions_share_a_workspace():
    """Decode steps at different positions reuse one workspace; repeating a
    step reproduces it exactly."""
    B, H, Tmax, D = 2, 3, 300, 64
    q, k, v = inputs(B, H, Tmax, D, "bf16", seed=41)
    cache = attn.KVCache(B, H, Tmax, D, torch.bfloat16, DEV)
    cache.append(k.to(DEV), v.to(DEV), 0)
    first = {}
    for pos in (299, 5, 64, 299, 130, 5):
        o, lse = cache.decode(q[:, :, pos].contiguous().to(DEV), pos)
        torch.cuda.synchronize()
        if pos in first:
            assert torch.equal(o, first[pos][0]) and torch.equal(lse, first[pos][1])
        else:
            first[pos] = (o.clone(), lse.clone())
            check(o.cpu(), lse.cpu(), q, k, v, pos, "bf16", f"shared workspace pos {pos}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_fused_step_equals_append_then_decode(D, dtype):
    """attn_decode_step (append + decode in one launch) gives bitwise the outputs
    and cache contents of attn_kv_append followed by attn_decode, token by token,
    across slice boundaries, and matches the oracle."""
    B, H, T = 2, 3, 140
    q, k, v = inputs(B, H, T, D, dtype, seed=51 + D)
    a = attn.KVCache(B, H, T, D, DT[dtype], DEV)
    b = attn.KVCache(B, H, T, D, DT[dtype], DEV)
    for t in range(T):
        qt, kt, vt = (x[:, :, t].contiguous().to(DEV) for x in (q, k, v))
        a.append(kt[:, :, None], vt[:, :, None], t)
        oa, la = a.decode(qt, t)
        ob, lb = b.step(qt, kt, vt, t)
        if t in (0, 1, 63, 64, 65, 127, 128, 139):
            torch.cuda.synchronize()
            assert torch.equal(oa, ob) and torch.equal(la, lb), t
            check(ob.cpu(), lb.cpu(), q, k, v, t, dtype, f"fused step {dtype} D{D} pos {t}")
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)


# 64 heads or more take one workgroup per head (its waves merge the slices in
# LDS); Tmax spans more 64-key slices than that workgroup has waves (16 at D 64,
# 8 at D 128), so waves also carry a running maximum over several slices
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D,Tmax", [(64, 1100), (128, 600)])
def test_decode_many_heads(D, Tmax, dtype):
    B, H = 4, 16
    q, k, v = inputs(B, H, Tmax, D, dtype, seed=61 + D)
    cache = attn.KVCache(B, H, Tmax, D, DT[dtype], DEV)
    cache.append(k.to(DEV), v.to(DEV), 0)
    for pos in (0, 63, 64, 511, 520, Tmax - 1):
        o, lse = cache.decode(q[:, :, pos].contiguous().to(DEV), pos)
        torch.cuda.synchronize()
        check(o.cpu(), lse.cpu(), q, k, v, pos, dtype, f"many heads {dtype} D{D} pos {pos}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D,Tmax", [(64, 1100), (128, 600)])
def test_fused_step_many_heads(D, Tmax, dtype):
    """attn_decode_step with one workgroup per head: bitwise append + decode, and
    the oracle, at positions on and around slice boundaries and past 16 (8) slices."""
    B, H = 4, 16
    q, k, v = inputs(B, H, Tmax, D, dtype, seed=71 + D)
    a = attn.KVCache(B, H, Tmax, D, DT[dtype], DEV)
    b = attn.KVCache(B, H, Tmax, D, DT[dtype], DEV)
    positions = (0, 1, 64, 511, 512, Tmax - 1)
    prev = 0
    for pos in positions:
        if pos > prev:  # rows prev .. pos-1 through the plain append on both caches
            kk, vv = k[:, :, prev:pos].to(DEV), v[:, :, prev:pos].to(DEV)
            a.append(kk, vv, prev)
            b.append(kk, vv, prev)
        qt, kt, vt = (x[:, :, pos].contiguous().to(DEV) for x in (q, k, v))
        a.append(kt[:, :, None], vt[:, :, None], pos)
        oa, la = a.decode(qt, pos)
        ob, lb = b.step(qt, kt, vt, pos)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(la, lb), pos
        check(ob.cpu(), lb.cpu(), q, k, v, pos, dtype, f"fused step many heads {dtype} D{D} pos {pos}")
        prev = pos + 1
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)


def test_decode_maximum_size():
    """The largest cache the decode calls accept: one head short of 2^31 elements
    per [B, H, Tmax, D] half at Tmax = 8192 (B1 H4095 D64, bf16; 17 GB of cache).
    All 8192 positions are appended in one call; decode at the last position is
    checked against the oracle on three heads (first, middle, last), and the
    fused step at that position (the first 8191 rows appended into a second
    cache) gives bitwise the same o, lse and cache rows. Inputs are drawn on the
    GPU from a seeded generator."""
    B, H, Tmax, D = 1, 4095, 8192, 64
    assert B * H * Tmax * D < 2 ** 31 <= B * (H + 1) * Tmax * D
    pos = Tmax - 1
    g = torch.Generator(device=DEV)
    g.manual_seed(4095)
    k = torch.randn((B, H, Tmax, D), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((B, H, Tmax, D), generator=g, device=DEV, dtype=torch.bfloat16)
    q = torch.randn((B, H, D), generator=g, device=DEV, dtype=torch.bfloat16)
    print("decode maximum size: inputs drawn", flush=True)
    a = attn.KVCache(B, H, Tmax, D, torch.bfloat16, DEV)
    a.append(k, v, 0)
    oa, la = a.decode(q, pos)
    torch.cuda.synchronize()
    print("decode maximum size: append and decode done", flush=True)
    b = attn.KVCache(B, H, Tmax, D, torch.bfloat16, DEV)
    b.append(k[:, :, :pos].contiguous(), v[:, :, :pos].contiguous(), 0)
    ob, lb = b.step(q, k[:, :, pos].contiguous(), v[:, :, pos].contiguous(), pos)
    torch.cuda.synchronize()
    print("decode maximum size: fused step done", flush=True)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(a.buf, b.buf)
    del b
    assert bool(torch.isfinite(oa).all()) and bool(torch.isfinite(la).all())
    heads = [0, H // 2, H - 1]
    f = lambda t: workloads.as_float64(t[:, heads].cpu())
    ro, rl = oracle.attention_decode(f(q), f(k), f(v), pos)
    o3, l3 = f(oa), la[:, heads].cpu().numpy().astype(np.float64)
    mx, rel = errors(o3, ro)
    assert mx <= TOL["bf16"]["max_abs"] and rel <= TOL["bf16"]["rel_l2"], (mx, rel)
    lmx, _ = errors(l3, rl)
    assert lmx <= 1e-2 + 1e-3 * float(np.max(np.abs(rl))), lmx
