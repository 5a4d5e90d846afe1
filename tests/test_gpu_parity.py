"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded inputs, plus exact special cases and invariants."""

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    from tests.gpu_util import assert_close, gpu_run, oracle_run


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_attn_amd as attn
    attn.load()


def test_tiny_f32_workload():
    w = workloads.WORKLOADS[workloads.TINY]
    x = workloads.make(w)
    assert_close(gpu_run(x), oracle_run(x), "f32", w.name)


# shapes that cross tile boundaries and leave ragged tails (tiles are 32/64/128 rows)
SMALL = [(1, 1, 1), (1, 1, 3), (1, 2, 63), (1, 1, 64), (2, 1, 65), (1, 3, 127), (1, 1, 128),
         (1, 2, 200), (1, 1, 257), (2, 2, 333)]


HALF = {"bf16": workloads.HEADLINE, "f16": "gpt2s_f16_b8h12t1024d64"}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,T", SMALL)
def test_16bit_small_shapes(B, H, T, D, dtype):
    w = workloads.WORKLOADS[HALF[dtype]]
    x = workloads.make(w, seed=T + D, shape=(B, H, T, D))
    assert_close(gpu_run(x), oracle_run(x), dtype, f"{dtype} B{B} H{H} T{T} D{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 2, 65), (1, 1, 200), (2, 1, 129)])
def test_f32_small_shapes(B, H, T, D):
    w = workloads.WORKLOADS[workloads.TINY]
    x = workloads.make(w, seed=T + D, shape=(B, H, T, D))
    assert_close(gpu_run(x), oracle_run(x), "f32", f"f32 B{B} H{H} T{T} D{D}")


def test_peaky_logits_small():
    w = workloads.WORKLOADS["peaky_bf16_b16h12t2048d64"]
    x = workloads.make(w, shape=(1, 2, 300, 64))
    assert_close(gpu_run(x), oracle_run(x), "bf16", "peaky small")


FULL = ["gpt2s_bf16_b8h12t1024d64", "gpt2s_f16_b8h12t1024d64", "longctx_bf16_b2h12t4096d64",
        "peaky_bf16_b16h12t2048d64", "wide_bf16_b1h6t8192d128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads_all_heads(name):
    """Full-size launch in the benchmark's configuration (the saved path), every
    output element of every head against the oracle."""
    w = workloads.WORKLOADS[name]
    x = workloads.make(w)
    got = gpu_run(x)
    print(f"{name}: GPU done, oracle on all {w.B * w.H} heads", flush=True)
    assert_close(got, oracle_run(x), w.dtype, name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 2, 63), (2, 1, 65), (1, 3, 127), (1, 2, 200),
                                   (2, 2, 333)])
def test_paths_agree_bitwise(B, H, T, D, dtype):
    """attn_fwd + attn_bwd (q, k rotated by the backward itself), attn_fwd_save +
    attn_bwd_saved, the rotation pass + attn_fwd_rotated, and the four stages one
    by one give bitwise the same outputs; the forward's saved buffer is bitwise the
    rotation pass's output."""
    x = workloads.make(workloads.WORKLOADS[HALF[dtype]], seed=T + D + 3, shape=(B, H, T, D))
    runs = {p: gpu_run(x, path=p) for p in ("saved", "plain", "rotated", "stages")}
    for p in ("plain", "rotated", "stages"):
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(runs[p][n], runs["saved"][n]), (p, n)
    n = B * H * T * D * 2  # bytes of rotated q, then of rotated k
    for p in ("rotated", "stages"):
        for part in (slice(0, n), slice(n, 2 * n)):
            assert torch.equal(runs[p]["saved"][part], runs["saved"]["saved"][part]), p


def test_backward_reads_its_own_q_and_k():
    """attn_bwd rotates the q, k it is given; attn_bwd_saved trusts its buffer:
    handed the rotated values of other inputs, it gives other gradients."""
    w = workloads.WORKLOADS[workloads.HEADLINE]
    x = workloads.make(w, seed=21, shape=(1, 2, 150, 64))
    y = workloads.make(w, seed=22, shape=(1, 2, 150, 64))
    ref = oracle_run(x)
    dev = torch.device("cuda", 0)
    g = {n: t.to(dev) for n, t in x.items()}
    o, lse, _ = attn.forward(g["q"], g["k"], g["v"], save=False)
    _, _, stale = attn.forward(y["q"].to(dev), y["k"].to(dev), y["v"].to(dev))
    dq, dk, dv = attn.backward(g["q"], g["k"], g["v"], o, g["do"], lse, None)
    got = dict(o=o.cpu(), lse=lse.cpu(), dq=dq.cpu(), dk=dk.cpu(), dv=dv.cpu())
    assert_close(got, ref, "bf16", "attn_bwd from its own q, k")
    dq2, _, _ = attn.backward(g["q"], g["k"], g["v"], o, g["do"], lse, stale)
    assert not torch.equal(dq2.cpu(), got["dq"])


@pytest.mark.parametrize("dtype,H,D", [("bf16", 4095, 64), ("bf16", 2047, 128), ("f16", 4095, 64)])
def test_maximum_size_sampled_heads(dtype, H, D):
    """The largest [B, H, T, D] tensors the entry points accept (one head short of
    2^31 elements at T = 8192: H4095 at D = 64, H2047 at D = 128; bf16, and fp16
    storage at D = 64; about 45 GB on the GPU with the outputs, the saved buffer
    and the workspace) through the training pair. Three heads (first, middle, last) are checked against the oracle
    element by element; every head is checked for finite outputs and for o's first
    row being exactly v's first row (the first query attends to key 0 alone). Inputs
    are drawn on the GPU from a seeded generator, with the headline workload's
    distributions."""
    B, T = 1, 8192
    assert B * H * T * D < 2 ** 31 <= B * (H + 1) * T * D
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(H + (dtype == "f16"))
    shape = (B, H, T, D)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    q = torch.randn(shape, generator=g, device=dev, dtype=dt)
    k = torch.randn(shape, generator=g, device=dev, dtype=dt)
    v = torch.randn(shape, generator=g, device=dev, dtype=dt)
    do = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * 0.1).to(dt)
    print("maximum size: inputs drawn", flush=True)
    o, lse, saved = attn.forward(q, k, v, save=True)
    dq, dk, dv = attn.backward(q, k, v, o, do, lse, saved)
    torch.cuda.synchronize()
    print("maximum size: GPU forward and backward done", flush=True)
    for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items():
        assert bool(torch.isfinite(t).all()), f"{n} has non-finite values"
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    del saved
    heads = [(0, 0), (0, H // 2), (0, H - 1)]
    x = {n: torch.stack([t[b, h] for b, h in heads])[None].cpu() for n, t in
         dict(q=q, k=k, v=v, do=do).items()}
    got = {n: torch.stack([t[b, h] for b, h in heads])[None].cpu() for n, t in
           dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    print("maximum size: oracle on 3 heads", flush=True)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()  # the 45 GB go back before the next test
    assert_close(got, oracle_run(x), dtype, f"maximum size {dtype} B1 H{H} T8192 D{D}, heads {heads}")


def test_row_zero_is_v_zero_bitwise():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    for D in (64, 128):
        x = workloads.make(w, seed=5, shape=(2, 3, 150, D))
        got = gpu_run(x)
        assert torch.equal(got["o"][:, :, 0], x["v"][:, :, 0])
        # exactly 0 in exact arithmetic; on the GPU dP (MFMA) and delta (VALU)
        # sum the same products in different orders, leaving fp32 rounding noise
        assert float(got["dq"][:, :, 0].abs().max()) < 1e-5


def test_zero_queries_uniform_attention():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    for D in (64, 128):
        x = workloads.make(w, seed=6, shape=(1, 2, 190, D))
        x["q"] = torch.zeros_like(x["q"])
        got = gpu_run(x)
        v = workloads.as_float64(x["v"])
        n = np.arange(1, 191, dtype=np.float64)
        np.testing.assert_allclose(workloads.as_float64(got["o"]),
                                   np.cumsum(v, axis=2) / n[:, None], atol=2e-2)
        np.testing.assert_allclose(workloads.as_float64(got["lse"]),
                                   np.broadcast_to(np.log(n), (1, 2, 190)), atol=1e-5)
        assert float(np.max(np.abs(workloads.as_float64(got["dk"])))) < 1e-3


def test_causal_invariance_bitwise():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    for dtype_w, D in ((w, 64), (w, 128), (workloads.WORKLOADS[workloads.TINY], 64)):
        x = workloads.make(dtype_w, seed=7, shape=(1, 2, 260, D))
        base = gpu_run(x)
        for t in (0, 31, 64, 129, 258):
            y = {n: v.clone() for n, v in x.items()}
            noise = workloads.make(dtype_w, seed=100 + t, shape=(1, 2, 260, D))
            for n in y:
                y[n][:, :, t + 1:] = noise[n][:, :, t + 1:]
            got = gpu_run(y)
            for n in ("o", "lse", "dq"):
                assert torch.equal(got[n][:, :, :t + 1], base[n][:, :, :t + 1]), (D, t, n)


def test_deterministic():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    x = workloads.make(w, seed=8, shape=(2, 3, 700, 64))
    a, b = gpu_run(x), gpu_run(x)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_rope_table_kernel():
    import causal_attention_attn_amd as attn
    for T, D in ((1, 64), (1024, 64), (8192, 128)):
        cs, sn = attn.rope_tables(T, D, 10000.0, "cuda:0")
        t = np.arange(T, dtype=np.float64)[:, None]
        ang = t * 10000.0 ** (-np.arange(0, D, 2, dtype=np.float64) / D)
        np.testing.assert_allclose(cs.cpu().double().numpy(), np.cos(ang), rtol=0, atol=1e-7)
        np.testing.assert_allclose(sn.cpu().double().numpy(), np.sin(ang), rtol=0, atol=1e-7)


def test_binding_rejects_before_any_launch():
    """The Python helpers check what the C ABI cannot see (tensor devices, a saved
    buffer's real size, lse's dtype and device) and raise ValueError before they
    allocate outputs or launch anything."""
    dev = torch.device("cuda", 0)
    q = torch.randn((1, 2, 40, 64), device=dev).to(torch.bfloat16)
    o, lse, saved = attn.forward(q, q, q)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):  # a saved buffer shorter than these inputs need
        attn.backward(q, q, q, o, q, lse, saved[:-256])
    with pytest.raises(ValueError):  # saved on the host
        attn.backward(q, q, q, o, q, lse, saved.cpu())
    with pytest.raises(ValueError):  # lse on the host
        attn.backward(q, q, q, o, q, lse.cpu(), saved)
    with pytest.raises(ValueError):  # lse of another dtype
        attn.backward(q, q, q, o, q, lse.double(), saved)
    cache = attn.KVCache(1, 2, 64, 64, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 2, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host k, v
        cache.append(kv, kv, 0)
    with pytest.raises(ValueError):  # host q
        cache.decode(torch.zeros((1, 2, 64), dtype=torch.bfloat16), 3)
    with pytest.raises(ValueError):  # host q, k, v for a fused step
        x = torch.zeros((1, 2, 64), dtype=torch.bfloat16)
        cache.step(x, x, x, 3)


def test_abi_errors_on_gpu():
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    cs, sn = attn.rope_tables(8, 64, 10000.0, "cuda:0")
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 8), dtype=torch.float32, device="cuda")
    ns = attn.attn_saved_bytes(1, 1, 8, 64, attn.ATTN_BF16)
    saved = torch.empty(ns, dtype=torch.uint8, device="cuda")
    with pytest.raises(attn.AttnError):
        attn.attn_fwd(q, q, q, cs, sn, o, lse, 1, 1, 8, 96, attn.ATTN_BF16)
    with pytest.raises(attn.AttnError):
        attn.attn_fwd(q, q, q, cs, sn, q, lse, 1, 1, 8, 64, attn.ATTN_BF16)
    with pytest.raises(attn.AttnError):
        attn.attn_fwd_save(q, q, q, cs, sn, o, lse, saved, ns - 256, 1, 1, 8, 64, attn.ATTN_BF16)
    with pytest.raises(ValueError):  # the binding checks lse before any launch
        attn.backward(q, q, q, o, q, lse[:, :, :4], saved)
    attn.attn_fwd(q, q, q, cs, sn, o, lse, 1, 1, 8, 64, attn.ATTN_BF16)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
