"""GPU parity of the per-layer kernels next to attention (residual add +
RMSNorm, SwiGLU; forward and backward) against the float64 oracle.

Tolerances, from the arithmetic: outputs are computed in fp32 and rounded once
to bf16 or fp16, whose half-ulp is 2^-8 or 2^-11 of the value, so each output
element must lie within 2^-7 (bf16) or 2^-10 (fp16) of the oracle value relative
to the larger of its magnitude and the tensor's root mean square (outputs that
cancel to near zero get the tensor's scale). dg is fp32 throughout: relative
L2 error <= 1e-4. The residual stream h is x + r rounded to the dtype; the
oracle normalises that stored h (the reading stated with the oracle), and h
itself must equal the rounded sum bitwise."""

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import causal_attention_attn_amd as attn
    import oracle

DEV = "cuda:0"
REL = {"bf16": 2.0 ** -7, "f16": 2.0 ** -10}
CODE = {"bf16": 0, "f16": 2}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load()


f64 = workloads.as_float64


def close(got, ref, dtype, label):
    got = f64(got)
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref)) + 1e-30)
    bad = np.abs(got - ref) > REL[dtype] * scale
    assert np.all(np.isfinite(got)), label
    assert not bad.any(), f"{label}: {bad.sum()} elements off, worst {np.max(np.abs(got - ref) / scale):.3e}"


def run_norm(x, r, g, dy, dres, dtype, eps=1e-5):
    N, C = x.shape
    d = {n: (t.to(DEV) if t is not None else None) for n, t in dict(x=x, r=r, g=g, dy=dy, dres=dres).items()}
    h = torch.empty_like(d["x"]); y = torch.empty_like(d["x"])
    rstd = torch.empty(N, dtype=torch.float32, device=DEV)
    attn.attn_rmsnorm_fwd(d["x"], d["r"], d["g"], eps, h if r is not None else None, y, rstd, N,
                          C, CODE[dtype])
    hin = h if r is not None else d["x"]
    dh = torch.empty_like(d["x"]); dg = torch.empty(C, dtype=torch.float32, device=DEV)
    nw = attn.attn_rmsnorm_bwd_workspace_bytes(N, C, CODE[dtype])
    ws = torch.empty(nw, dtype=torch.uint8, device=DEV)
    attn.attn_rmsnorm_bwd(hin, d["g"], rstd, d["dy"], d["dres"], dh, dg, ws, nw, N, C,
                          CODE[dtype])
    torch.cuda.synchronize()
    return h.cpu(), y.cpu(), rstd.cpu(), dh.cpu(), dg.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,C", [(1, 256), (3, 768), (37, 512), (130, 1024), (9, 4096), (20001, 512)])
@pytest.mark.parametrize("residual", [True, False])
def test_rmsnorm(N, C, dtype, residual):
    x = workloads.layer_inputs("rmsnorm", N, C, dtype, seed=N + C)
    r = x["r"] if residual else None
    dres = x["dres"] if residual else None
    h, y, rstd, dh, dg = run_norm(x["x"], r, x["g"], x["dy"], dres, dtype)
    hs = (x["x"].float() + x["r"].float()).to(x["x"].dtype) if residual else x["x"]
    if residual:
        assert torch.equal(h, hs)
    _, ry, rr = oracle.rmsnorm_forward(f64(hs), f64(x["g"]))
    rdh, rdg = oracle.rmsnorm_backward(f64(hs), f64(x["g"]), f64(x["dy"]),
                                       dres=f64(dres) if residual else None)
    label = f"rmsnorm {dtype} N{N} C{C} res{residual}"
    close(y, ry, dtype, label + " y")
    np.testing.assert_allclose(f64(rstd), rr, rtol=1e-5)
    close(dh, rdh, dtype, label + " dh")
    rel = np.linalg.norm(f64(dg) - rdg) / np.linalg.norm(rdg)
    assert rel <= 1e-4, (label, rel)


def test_rmsnorm_full_workload():
    kind, N, C, dtype = workloads.LAYER_WORKLOADS["rmsnorm_bf16_n8192c768"]
    x = workloads.layer_inputs(kind, N, C, dtype)
    h, y, _, dh, dg = run_norm(x["x"], x["r"], x["g"], x["dy"], x["dres"], dtype)
    hs = (x["x"].float() + x["r"].float()).to(torch.bfloat16)
    assert torch.equal(h, hs)
    _, ry, _ = oracle.rmsnorm_forward(f64(hs), f64(x["g"]))
    rdh, rdg = oracle.rmsnorm_backward(f64(hs), f64(x["g"]), f64(x["dy"]), dres=f64(x["dres"]))
    close(y, ry, dtype, "rmsnorm full y")
    close(dh, rdh, dtype, "rmsnorm full dh")
    assert np.linalg.norm(f64(dg) - rdg) / np.linalg.norm(rdg) <= 1e-4


def run_swiglu(u, dout, dtype):
    N, F2 = u.shape
    F = F2 // 2
    du_, dd = u.to(DEV), dout.to(DEV)
    out = torch.empty((N, F), dtype=u.dtype, device=DEV)
    du = torch.empty_like(du_)
    attn.attn_swiglu_fwd(du_, out, N, F, CODE[dtype])
    attn.attn_swiglu_bwd(du_, dd, du, N, F, CODE[dtype])
    torch.cuda.synchronize()
    return out.cpu(), du.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,F", [(1, 8), (3, 24), (17, 2048), (64, 1000)])
def test_swiglu(N, F, dtype):
    x = workloads.layer_inputs("swiglu", N, F, dtype, seed=N + F)
    out, du = run_swiglu(x["u"], x["dout"], dtype)
    close(out, oracle.swiglu_forward(f64(x["u"])), dtype, f"swiglu {dtype} N{N} F{F} out")
    close(du, oracle.swiglu_backward(f64(x["u"]), f64(x["dout"])), dtype,
          f"swiglu {dtype} N{N} F{F} du")


def test_swiglu_full_workload_and_extremes():
    kind, N, F, dtype = workloads.LAYER_WORKLOADS["swiglu_bf16_n8192f2048"]
    x = workloads.layer_inputs(kind, N, F, dtype)
    out, du = run_swiglu(x["u"], x["dout"], dtype)
    close(out, oracle.swiglu_forward(f64(x["u"])), dtype, "swiglu full out")
    close(du, oracle.swiglu_backward(f64(x["u"]), f64(x["dout"])), dtype, "swiglu full du")
    # large gates: sigmoid saturates to 0 and 1 without overflow or NaN
    u = torch.zeros((1, 16), dtype=torch.bfloat16)
    u[0, :8] = torch.tensor([-200., -60., -20., -1., 1., 20., 60., 200.])
    u[0, 8:] = 1.0
    out, du = run_swiglu(u, torch.ones((1, 8), dtype=torch.bfloat16), "bf16")
    close(out, oracle.swiglu_forward(f64(u)), "bf16", "swiglu extremes out")
    close(du, oracle.swiglu_backward(f64(u), np.ones((1, 8))), "bf16", "swiglu extremes du")


def test_layers_maximum_size():
    """The largest tensors the per-layer calls accept: N*C one row short of 2^31
    elements for RMSNorm (N 524287, C 4096, with the residual) and 2*N*F for
    SwiGLU (N 262143, F 4096), bf16. Rows are independent in both forwards, in
    the RMSNorm dh and in SwiGLU's du, so the first, middle and last rows are
    checked against the oracle; h must be the rounded x + r bitwise everywhere,
    and every output finite. Inputs are drawn on the GPU from a seeded generator."""
    dt, code = torch.bfloat16, CODE["bf16"]
    g_ = torch.Generator(device=DEV)
    g_.manual_seed(2 ** 31 - 1)
    rnd = lambda *s: torch.randn(s, generator=g_, device=DEV, dtype=torch.float32)
    N, C = 524287, 4096
    assert N * C < 2 ** 31 <= (N + 1) * C
    x, r = rnd(N, C).to(dt), rnd(N, C).to(dt)
    dy, dres = (rnd(N, C) * 0.1).to(dt), (rnd(N, C) * 0.1).to(dt)
    gain = (1.0 + 0.1 * rnd(C)).to(dt)
    h, y, dh = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    rstd = torch.empty(N, dtype=torch.float32, device=DEV)
    dg = torch.empty(C, dtype=torch.float32, device=DEV)
    attn.attn_rmsnorm_fwd(x, r, gain, 1e-5, h, y, rstd, N, C, code)
    nw = attn.attn_rmsnorm_bwd_workspace_bytes(N, C, code)
    ws = torch.empty(nw, dtype=torch.uint8, device=DEV)
    attn.attn_rmsnorm_bwd(h, gain, rstd, dy, dres, dh, dg, ws, nw, N, C, code)
    torch.cuda.synchronize()
    print("layers maximum size: RMSNorm done", flush=True)
    assert torch.equal(h, (x.float() + r.float()).to(dt))
    for n, t in dict(y=y, rstd=rstd, dh=dh, dg=dg).items():
        assert bool(torch.isfinite(t).all()), f"rmsnorm {n} has non-finite values"
    rows = [0, 1, N // 2, N - 2, N - 1]
    pick = lambda t: t[rows].cpu()
    hs, gs = f64(pick(h)), f64(gain.cpu())
    _, ry, rr = oracle.rmsnorm_forward(hs, gs)
    rdh, _ = oracle.rmsnorm_backward(hs, gs, f64(pick(dy)), dres=f64(pick(dres)))
    close(pick(y), ry, "bf16", "rmsnorm maximum size y")
    np.testing.assert_allclose(f64(pick(rstd)), rr, rtol=1e-5)
    close(pick(dh), rdh, "bf16", "rmsnorm maximum size dh")
    del x, r, dy, dres, h, y, dh, ws
    torch.cuda.empty_cache()

    N, F = 262143, 4096
    assert 2 * N * F < 2 ** 31 <= 2 * (N + 1) * F
    u = rnd(N, 2 * F).to(dt)
    dout = (rnd(N, F) * 0.1).to(dt)
    out, du = torch.empty((N, F), dtype=dt, device=DEV), torch.empty_like(u)
    attn.attn_swiglu_fwd(u, out, N, F, code)
    attn.attn_swiglu_bwd(u, dout, du, N, F, code)
    torch.cuda.synchronize()
    print("layers maximum size: SwiGLU done", flush=True)
    for n, t in dict(out=out, du=du).items():
        assert bool(torch.isfinite(t).all()), f"swiglu {n} has non-finite values"
    rows = [0, 1, N // 2, N - 2, N - 1]
    us = f64(u[rows].cpu())
    close(out[rows].cpu(), oracle.swiglu_forward(us), "bf16", "swiglu maximum size out")
    close(du[rows].cpu(), oracle.swiglu_backward(us, f64(dout[rows].cpu())), "bf16",
          "swiglu maximum size du")


@pytest.mark.parametrize("residual", [True, False])
def test_rmsnorm_autograd(residual):
    """attn.rmsnorm as a differentiable op: y (and h), and the gradients of x, res
    and g for L = sum(y * dy) + sum(h * dres), bitwise those of the direct calls
    (g's gradient rounded from the fp32 dg)."""
    N, C = 300, 768
    x = workloads.layer_inputs("rmsnorm", N, C, "bf16", seed=77)
    d = {n: t.to(DEV) for n, t in x.items()}
    xg = d["x"].clone().requires_grad_()
    gg = d["g"].clone().requires_grad_()
    if residual:
        rg = d["r"].clone().requires_grad_()
        y, h = attn.rmsnorm(xg, gg, rg)
        ((y.float() * d["dy"].float()).sum() + (h.float() * d["dres"].float()).sum()).backward()
    else:
        y = attn.rmsnorm(xg, gg)
        (y.float() * d["dy"].float()).sum().backward()
    rh, ry, _, rdh, rdg = run_norm(x["x"], x["r"] if residual else None, x["g"], x["dy"],
                                   x["dres"] if residual else None, "bf16")
    assert torch.equal(y.detach().cpu(), ry)
    if residual:
        assert torch.equal(h.detach().cpu(), rh)
        assert torch.equal(rg.grad.cpu(), rdh)
    assert torch.equal(xg.grad.cpu(), rdh)
    assert torch.equal(gg.grad.cpu(), rdg.to(torch.bfloat16))


def test_swiglu_autograd():
    N, F = 64, 1000
    x = workloads.layer_inputs("swiglu", N, F, "bf16", seed=78)
    u = x["u"].to(DEV).requires_grad_()
    out = attn.swiglu(u)
    out.backward(x["dout"].to(DEV))
    rout, rdu = run_swiglu(x["u"], x["dout"], "bf16")
    assert torch.equal(out.detach().cpu(), rout)
    assert torch.equal(u.grad.cpu(), rdu)
