"""GPU parity of the model-native layouts (attn_fwd_packed / attn_bwd_packed):
q, k, v read from the packed [B, T, 3, H, D] projection output, o and dO in
[B, T, H, D], gradients written back packed. Checked against the float64
oracle, bitwise against the [B, H, T, D] entry points (same kernels, only the
addressing differs), and for writes outside the output tensors."""

import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    from tests.gpu_util import assert_close, gpu_run, gpu_run_packed, oracle_run, select_heads
    from tests.gpu_util import to_packed


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load()


HALF = {"bf16": workloads.HEADLINE, "f16": "gpt2s_f16_b8h12t1024d64"}
SHAPES = [(1, 1, 1), (2, 1, 65), (1, 3, 127), (1, 2, 200), (2, 2, 333)]


@pytest.mark.parametrize("save", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,T", SHAPES)
def test_packed_small_shapes(B, H, T, D, dtype, save):
    """With a saved buffer, and without one (the backward rotates q, k itself)."""
    x = workloads.make(workloads.WORKLOADS[HALF[dtype]], seed=T + D + 1, shape=(B, H, T, D))
    got = gpu_run_packed(x, save=save)
    assert_close(got, oracle_run(x), dtype, f"packed {dtype} B{B} H{H} T{T} D{D}")
    ref = gpu_run(x)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(got[n], ref[n]), f"packed {n} differs from the [B,H,T,D] path"


@pytest.mark.parametrize("name", ["gpt2s_bf16_b8h12t1024d64", "gpt2s_f16_b8h12t1024d64"])
def test_packed_full_size(name):
    """The benchmark's shape: bitwise equal to the [B, H, T, D] path everywhere,
    and within tolerance of the oracle on sampled heads."""
    w = workloads.WORKLOADS[name]
    x = workloads.make(w)
    got = gpu_run_packed(x)
    ref = gpu_run(x)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(got[n], ref[n]), f"packed {n} differs from the [B,H,T,D] path"
    heads = [(0, 0), (5, 11)]
    assert_close(select_heads(got, heads), oracle_run(x, heads=heads), w.dtype, name)


def test_packed_writes_nothing_outside_its_outputs():
    """o and dqkv are placed inside larger buffers filled with a sentinel; the
    bytes before and after each output stay untouched."""
    B, H, T, D = 2, 3, 200, 64
    x = workloads.make(workloads.WORKLOADS[workloads.HEADLINE], seed=5, shape=(B, H, T, D))
    dev = torch.device("cuda", 0)
    qkv, do = to_packed(x, dev)
    dt = attn.ATTN_BF16
    cs, sn = attn.rope_tables(T, D, 10000.0, dev)
    pad = 4096
    n_o, n_g = B * T * H * D, 3 * B * T * H * D
    obuf = torch.full((n_o + 2 * pad,), -7.0, dtype=torch.bfloat16, device=dev)
    gbuf = torch.full((n_g + 2 * pad,), -7.0, dtype=torch.bfloat16, device=dev)
    o = obuf[pad:pad + n_o]
    dqkv = gbuf[pad:pad + n_g]
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ns = attn.attn_saved_bytes(B, H, T, D, dt)
    saved = torch.empty(ns, dtype=torch.uint8, device=dev)
    nw = attn.attn_bwd_workspace_bytes(B, H, T, D, dt)
    ws = torch.empty(nw, dtype=torch.uint8, device=dev)
    attn.attn_fwd_packed(qkv, cs, sn, o, lse, saved, ns, B, H, T, D, dt)
    attn.attn_bwd_packed(qkv, o, do, lse, cs, sn, saved, ns, dqkv, ws, nw, B, H, T, D, dt)
    torch.cuda.synchronize()
    for buf, n in ((obuf, n_o), (gbuf, n_g)):
        assert torch.all(buf[:pad] == -7.0) and torch.all(buf[pad + n:] == -7.0)
        assert torch.isfinite(buf[pad:pad + n].float()).all()
    ref = gpu_run(x)
    assert torch.equal(o.view(B, T, H, D).permute(0, 2, 1, 3).cpu(), ref["o"])


@pytest.mark.parametrize("H,D", [(1365, 64), (682, 128)])
def test_packed_maximum_size(H, D):
    """The largest packed tensor the packed entry points accept: one head short of
    2^31 elements in [B, T, 3, H, D] at T = 8192 (H1365 at D = 64, H682 at D = 128),
    bf16. Every output is bitwise that of the [B, H, T, D] entry points on the same
    values, three heads are checked against the oracle, and o's first row is v's.
    Inputs are drawn on the GPU from a seeded generator."""
    B, T = 1, 8192
    assert 3 * B * H * T * D < 2 ** 31 <= 3 * B * (H + 1) * T * D
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(H + D)
    qkv = torch.randn((B, T, 3, H, D), generator=g, device=dev, dtype=torch.bfloat16)
    do = (torch.randn((B, T, H, D), generator=g, device=dev, dtype=torch.float32) * 0.1).to(
        torch.bfloat16)
    print(f"packed maximum size H{H} D{D}: inputs drawn", flush=True)
    o, lse, saved = attn.forward_packed(qkv, save=True)
    dqkv = attn.backward_packed(qkv, o, do, lse, saved)
    torch.cuda.synchronize()
    del saved
    print("packed maximum size: packed forward and backward done", flush=True)
    bhtd = lambda t: t.permute(0, 2, 1, 3).contiguous()
    q, k, v, dob = bhtd(qkv[:, :, 0]), bhtd(qkv[:, :, 1]), bhtd(qkv[:, :, 2]), bhtd(do)
    o2, lse2, saved2 = attn.forward(q, k, v, save=True)
    dq2, dk2, dv2 = attn.backward(q, k, v, o2, dob, lse2, saved2)
    torch.cuda.synchronize()
    del saved2
    print("packed maximum size: [B, H, T, D] forward and backward done", flush=True)
    assert torch.equal(bhtd(o), o2) and torch.equal(lse, lse2)
    for s, (n, ref) in enumerate(zip(("dq", "dk", "dv"), (dq2, dk2, dv2))):
        assert torch.equal(bhtd(dqkv[:, :, s]), ref), n
    for n, t in dict(o=o2, lse=lse2, dq=dq2, dk=dk2, dv=dv2).items():
        assert bool(torch.isfinite(t).all()), f"{n} has non-finite values"
    assert torch.equal(o2[:, :, 0], v[:, :, 0])
    heads = [(0, 0), (0, H // 2), (0, H - 1)]
    pick = lambda t: torch.stack([t[b, h] for b, h in heads])[None].cpu()
    x = {n: pick(t) for n, t in dict(q=q, k=k, v=v, do=dob).items()}
    got = {n: pick(t) for n, t in dict(o=o2, lse=lse2, dq=dq2, dk=dk2, dv=dv2).items()}
    del qkv, do, o, lse, dqkv, q, k, v, dob, o2, lse2, dq2, dk2, dv2
    torch.cuda.empty_cache()
    print("packed maximum size: oracle on 3 heads", flush=True)
    assert_close(got, oracle_run(x), "bf16", f"packed maximum size B1 H{H} T8192 D{D}, heads {heads}")
