"""Pins for the float64 RMSNorm and SwiGLU oracle (CPU only): closed forms,
invariances, centred finite differences in double precision (the pages' own
gradient check, "Show HN: NanoEuler" paragraph 2) and torch's float64
rms_norm / silu with autograd as library routines."""

import math

import numpy as np
import pytest

import oracle


def rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------- RMSNorm ----------

def test_rmsnorm_constant_row():
    # a row of equal values c: mean square c^2, so y = g * c / sqrt(c^2 + eps)
    C, c = 16, 3.0
    x = np.full((1, C), c)
    g = rand((C,), 1)
    h, y, rstd = oracle.rmsnorm_forward(x, g)
    np.testing.assert_allclose(y[0], g * c / math.sqrt(c * c + 1e-5), rtol=1e-14)
    np.testing.assert_allclose(rstd, 1 / math.sqrt(c * c + 1e-5), rtol=1e-14)


def test_rmsnorm_residual_add_and_unit_rms():
    x, r = rand((5, 32), 2), rand((5, 32), 3)
    h, y, _ = oracle.rmsnorm_forward(x, np.ones(32), r=r, eps=0.0)
    np.testing.assert_array_equal(h, x + r)
    # with g = 1 and eps = 0 every output row has root mean square exactly 1
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    # scale invariance: y(alpha h) = y(h) when eps = 0
    _, y2, _ = oracle.rmsnorm_forward(7.5 * h, np.ones(32), eps=0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13)


def test_rmsnorm_matches_torch_float64():
    torch = pytest.importorskip("torch")
    N, C = 6, 48
    h, g, dy = rand((N, C), 4), rand((C,), 5), rand((N, C), 6)
    th = torch.tensor(h, requires_grad=True)
    tg = torch.tensor(g, requires_grad=True)
    ty = torch.nn.functional.rms_norm(th, (C,), tg, eps=1e-5)
    (ty * torch.tensor(dy)).sum().backward()
    _, y, _ = oracle.rmsnorm_forward(h, g)
    dh, dg = oracle.rmsnorm_backward(h, g, dy)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_rmsnorm_gradients_match_centred_differences():
    N, C, eps, step = 3, 8, 1e-5, 1e-6
    h, g, dy, dres = rand((N, C), 7), rand((C,), 8), rand((N, C), 9), rand((N, C), 10)
    loss = lambda hh, gg: np.sum(oracle.rmsnorm_forward(hh, gg, eps=eps)[1] * dy) + np.sum(hh * dres)
    dh, dg = oracle.rmsnorm_backward(h, g, dy, dres=dres, eps=eps)
    for idx in np.ndindex(N, C):
        e = np.zeros((N, C)); e[idx] = step
        fd = (loss(h + e, g) - loss(h - e, g)) / (2 * step)
        assert abs(fd - dh[idx]) <= 1e-6 * max(1.0, abs(fd)), idx
    for c in range(C):
        e = np.zeros(C); e[c] = step
        fd = (loss(h, g + e) - loss(h, g - e)) / (2 * step)
        assert abs(fd - dg[c]) <= 1e-6 * max(1.0, abs(fd)), c


def test_rmsnorm_gradient_is_orthogonal_to_the_row():
    # y is invariant to scaling h (eps = 0), so <dh, h> = 0 for every row when dres = 0
    h, g, dy = rand((4, 24), 11), rand((24,), 12), rand((4, 24), 13)
    dh, _ = oracle.rmsnorm_backward(h, g, dy, eps=0.0)
    np.testing.assert_allclose(np.sum(dh * h, axis=1), 0.0, atol=1e-12)


# -------------------------------------------------------------- SwiGLU ----------

def test_swiglu_closed_forms():
    F = 8
    b = rand((2, F), 20)
    u = np.concatenate([np.zeros((2, F)), b], axis=1)        # a = 0
    np.testing.assert_array_equal(oracle.swiglu_forward(u), 0.0)
    dout = rand((2, F), 21)
    du = oracle.swiglu_backward(u, dout)
    # silu'(0) = sigmoid(0) = 1/2, silu(0) = 0
    np.testing.assert_allclose(du[:, :F], dout * b / 2, rtol=1e-15)
    np.testing.assert_array_equal(du[:, F:], 0.0)
    # a = 1: silu(1) = 1 / (1 + 1/e)
    u1 = np.concatenate([np.ones((1, F)), np.ones((1, F))], axis=1)
    np.testing.assert_allclose(oracle.swiglu_forward(u1), 1 / (1 + math.exp(-1)), rtol=1e-15)


def test_swiglu_matches_torch_float64():
    torch = pytest.importorskip("torch")
    N, F = 5, 12
    u, dout = rand((N, 2 * F), 22, 3.0), rand((N, F), 23)
    tu = torch.tensor(u, requires_grad=True)
    a, b = tu[:, :F], tu[:, F:]
    out = torch.nn.functional.silu(a) * b
    (out * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(oracle.swiglu_forward(u), out.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(oracle.swiglu_backward(u, dout), tu.grad.numpy(), rtol=1e-12,
                               atol=1e-14)


def test_swiglu_gradients_match_centred_differences():
    N, F, step = 2, 5, 1e-6
    u, dout = rand((N, 2 * F), 24, 2.0), rand((N, F), 25)
    du = oracle.swiglu_backward(u, dout)
    for idx in np.ndindex(N, 2 * F):
        e = np.zeros((N, 2 * F)); e[idx] = step
        fd = (np.sum(oracle.swiglu_forward(u + e) * dout)
              - np.sum(oracle.swiglu_forward(u - e) * dout)) / (2 * step)
        assert abs(fd - du[idx]) <= 1e-7 * max(1.0, abs(fd)), idx


def test_layer_pins_catch_planted_mistakes(monkeypatch):
    """A dropped term in either backward fails the finite-difference pins."""
    import oracle.layers as Lm
    u, dout = rand((1, 6), 30), rand((1, 3), 31)
    real = Lm.swiglu_backward

    def dropped(uu, dd):       # silu'(a) taken as sigmoid(a), the a*s*(1-s) term dropped
        uu = np.asarray(uu, float); F = uu.shape[1] // 2
        a, b = uu[:, :F], uu[:, F:]
        s = 1 / (1 + np.exp(-a))
        return np.concatenate([dd * b * s, dd * a * s], axis=1)
    fd = (np.sum(Lm.swiglu_forward(u + np.eye(6)[0] * 1e-6) * dout)
          - np.sum(Lm.swiglu_forward(u - np.eye(6)[0] * 1e-6) * dout)) / 2e-6
    assert abs(real(u, dout)[0, 0] - fd) < 1e-7
    assert abs(dropped(u, dout)[0, 0] - fd) > 1e-3
    h, g, dy = rand((2, 6), 32), rand((6,), 33), rand((2, 6), 34)

    def no_mean_term(hh, gg, d, dres=None, eps=1e-5):
        rstd = 1 / np.sqrt(np.mean(hh * hh, axis=1) + eps)
        return rstd[:, None] * gg[None, :] * d, np.sum(d * hh * rstd[:, None], axis=0)
    monkeypatch.setattr(Lm, "rmsnorm_backward", no_mean_term)
    e = np.zeros((2, 6)); e[0, 0] = 1e-6
    loss = lambda hh: np.sum(Lm.rmsnorm_forward(hh, g)[1] * dy)
    fd = (loss(h + e) - loss(h - e)) / 2e-6
    assert abs(Lm.rmsnorm_backward(h, g, dy)[0][0, 0] - fd) > 1e-4
