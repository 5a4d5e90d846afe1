"""Plain float64 CPU oracle for the two per-layer kernels next to attention:
RMSNorm (with the residual add that precedes it) and the SwiGLU activation.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark may import or run this module. The GPU library
never calls it, and it shares no code, table or constant with the GPU path.

The pages list RMSNorm and SwiGLU among the hand-written CUDA kernels of the
engine ("Show HN: NanoEuler", paragraph 2) and describe each layer as causal
attention plus a feed-forward network of two linear transforms with a Swish
activation, both wrapped in residual connections ("Tiny Hackable CUDA",
section 3). They give no formulas; the readings taken here:

* Residual add + RMSNorm over the model width C of each token row:
  h = x + r (r optional), stored in the tensors' dtype (the residual stream);
  y = h * rstd * g with rstd = 1 / sqrt(mean_c(h^2) + eps), eps = 1e-5, g the
  per-feature gain. The norm is taken of h as stored.
  Backward, with h_hat = h * rstd and upstream gradients dy (of y) and dres
  (of h, from the residual stream; optional):
  dh = rstd * (g*dy - h_hat * mean_c(h_hat * g * dy)) + dres, which is also the
  gradient of x and of r; dg = sum over rows of dy * h_hat.
* SwiGLU: the fused gate/up projection gives u = [a | b] of width 2F per row;
  out = silu(a) * b with silu(a) = a * sigmoid(a) (Swish with beta = 1).
  Backward: da = dout * b * sigmoid(a) * (1 + a * (1 - sigmoid(a))),
  db = dout * silu(a), returned packed as du = [da | db].
"""

import numpy as np

DEFAULT_EPS = 1e-5


def rmsnorm_forward(x, g, r=None, eps=DEFAULT_EPS):
    """x, r [N, C], g [C]. Returns (h, y, rstd [N]) in float64."""
    x = np.asarray(x, dtype=np.float64)
    h = x if r is None else x + np.asarray(r, dtype=np.float64)
    rstd = 1.0 / np.sqrt(np.mean(h * h, axis=1) + eps)
    y = h * rstd[:, None] * np.asarray(g, dtype=np.float64)[None, :]
    return h, y, rstd


def rmsnorm_backward(h, g, dy, dres=None, eps=DEFAULT_EPS):
    """Gradients of L = sum(y * dy) + sum(h * dres) for y = RMSNorm(h) * g.
    Returns (dh [N, C], dg [C]); dh is also the gradient of x and of r."""
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    C = h.shape[1]
    rstd = 1.0 / np.sqrt(np.mean(h * h, axis=1) + eps)
    hh = h * rstd[:, None]
    gdy = g[None, :] * dy
    dh = rstd[:, None] * (gdy - hh * (np.sum(hh * gdy, axis=1) / C)[:, None])
    if dres is not None:
        dh = dh + np.asarray(dres, dtype=np.float64)
    dg = np.sum(dy * hh, axis=0)
    return dh, dg


def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def swiglu_forward(u):
    """u [N, 2F] = [a | b]. Returns silu(a) * b, [N, F], float64."""
    u = np.asarray(u, dtype=np.float64)
    F = u.shape[1] // 2
    a, b = u[:, :F], u[:, F:]
    return a * _sigmoid(a) * b


def swiglu_backward(u, dout):
    """Gradient of L = sum(out * dout) with respect to u = [a | b]: [N, 2F]."""
    u = np.asarray(u, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    F = u.shape[1] // 2
    a, b = u[:, :F], u[:, F:]
    s = _sigmoid(a)
    return np.concatenate([dout * b * s * (1.0 + a * (1.0 - s)), dout * a * s], axis=1)
