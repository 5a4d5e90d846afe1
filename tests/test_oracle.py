"""Pins for the float64 oracle (CPU only).

None of these re-types the oracle's formulas. They check it against what the
mathematics fixes: the softmax and causal invariants, closed forms (T = 1,
all-zero queries, a hand-worked T = 2 case, explicit rotation angles), the
relative-position property of RoPE, gradient identities, centred finite
differences in double precision (the pages' own gradient check, "Show HN:
NanoEuler" paragraph 2), a pure-Python brute force, and torch's
scaled_dot_product_attention + autograd in float64 on the CPU.
"""

import math

import numpy as np
import pytest

import oracle
from tests import brute_force


def rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- RoPE --------

def test_rope_frequency_closed_forms():
    # D = 2: a single pair with theta_0 = base**0 = 1, so position t turns by t radians.
    x = np.zeros((5, 2))
    x[:, 0] = 1.0
    r = oracle.rope(x, base=10000.0)
    t = np.arange(5)
    np.testing.assert_allclose(r[:, 0], np.cos(t), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r[:, 1], np.sin(t), rtol=0, atol=1e-15)   # +t: counter-clockwise
    # D = 4, base 10000: theta_1 = 10000**(-1/2) = 0.01; position 100 turns pair 1 by 1 rad.
    x = np.zeros((101, 4))
    x[:, 2] = 1.0
    r = oracle.rope(x, base=10000.0)
    assert abs(r[100, 2] - math.cos(1.0)) < 1e-14 and abs(r[100, 3] - math.sin(1.0)) < 1e-14
    assert np.all(r[:, :2] == 0.0)
    # D = 64: the last pair turns by 10000**(-62/64) per position.
    assert abs(oracle.rope_frequencies(64)[31] - 10000.0 ** (-62.0 / 64.0)) < 1e-18


def test_rope_is_rotation():
    x = rand((3, 40, 64), 1)
    r = oracle.rope(x)
    # R_0 = I
    np.testing.assert_array_equal(r[:, 0], x[:, 0])
    # each pair keeps its length
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)
    # the inverse undoes it
    np.testing.assert_allclose(oracle.rope(r, inverse=True), x, rtol=0, atol=1e-12)
    # <R_t a, b> = <a, R_t^T b>
    a, b = rand((40, 64), 2), rand((40, 64), 3)
    lhs = np.sum(oracle.rope(a) * b, axis=1)
    rhs = np.sum(a * oracle.rope(b, inverse=True), axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_rope_relative_position_toeplitz():
    # same q at every position, same k at every position: the score depends on t - u only
    T, D = 24, 16
    q = np.tile(rand((1, D), 4), (T, 1))[None, None]
    k = np.tile(rand((1, D), 5), (T, 1))[None, None]
    qr, kr = oracle.rope(q)[0, 0], oracle.rope(k)[0, 0]
    S = qr @ kr.T
    for off in range(-T + 1, T):
        d = np.diagonal(S, offset=off)
        np.testing.assert_allclose(d, d[0], rtol=0, atol=1e-12)


# ------------------------------------------------------- softmax / mask ---------

def test_rows_sum_to_one_and_mask_is_exact():
    q, k = rand((2, 3, 33, 16), 6), rand((2, 3, 33, 16), 7)
    P = oracle.attention_probabilities(q, k)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    upper = np.triu(np.ones((33, 33), bool), 1)
    assert np.all(P[..., upper] == 0.0)
    assert np.all(P[..., ~upper] > 0.0)


def test_causal_invariance_bitwise():
    B, H, T, D = 1, 2, 40, 32
    q, k, v, do = (rand((B, H, T, D), s) for s in range(10, 14))
    o, lse = oracle.attention_forward(q, k, v)
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    for t in (0, 7, 25, 38):
        q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
        for i, x in enumerate((q2, k2, v2, do2)):
            x[:, :, t + 1:] = rand(x[:, :, t + 1:].shape, 100 + i, 5.0)
        o2, lse2 = oracle.attention_forward(q2, k2, v2)
        dq2, _, _ = oracle.attention_backward(q2, k2, v2, do2)
        assert np.array_equal(o[:, :, :t + 1], o2[:, :, :t + 1])
        assert np.array_equal(lse[:, :, :t + 1], lse2[:, :, :t + 1])
        assert np.array_equal(dq[:, :, :t + 1], dq2[:, :, :t + 1])
        assert not np.array_equal(o[:, :, t + 1:], o2[:, :, t + 1:])


# ---------------------------------------------------------- closed forms ---------

def test_single_position():
    q, k, v, do = (rand((2, 3, 1, 8), s) for s in range(20, 24))
    o, lse = oracle.attention_forward(q, k, v)
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse[..., 0], (q * k).sum(-1)[..., 0] / math.sqrt(8), rtol=1e-14)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, do)


def test_row_zero_is_v_zero():
    q, k, v, do = (rand((1, 2, 17, 16), s) for s in range(24, 28))
    o, lse = oracle.attention_forward(q, k, v)
    dq, _, _ = oracle.attention_backward(q, k, v, do)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], (q[:, :, 0] * k[:, :, 0]).sum(-1) / 4.0, rtol=1e-14)
    assert np.all(dq[:, :, 0] == 0)


def test_zero_queries_give_uniform_attention():
    B, H, T, D = 1, 2, 30, 16
    q = np.zeros((B, H, T, D))
    k, v, do = (rand((B, H, T, D), s) for s in range(30, 33))
    o, lse = oracle.attention_forward(q, k, v)
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    n = np.arange(1, T + 1, dtype=np.float64)
    np.testing.assert_allclose(o, np.cumsum(v, axis=2) / n[:, None], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(n), lse.shape), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    suffix = np.cumsum((do / n[:, None])[:, :, ::-1], axis=2)[:, :, ::-1]
    np.testing.assert_allclose(dv, suffix, rtol=1e-12, atol=1e-13)


def test_hand_worked_two_positions():
    # D = 2 (theta_0 = 1, so position 1 turns by 1 rad), T = 2.
    # q0 = (1,0), q1 = (0,1), k0 = k1 = (1,0), v0 = (1,2), v1 = (3,-1).
    # Rotated: q1r = (-sin 1, cos 1), k1r = (cos 1, sin 1); so
    # S10 = s*<q1r,k0> = -s sin 1 and S11 = s*<q1r,k1r> = 0, with s = 1/sqrt 2.
    q = np.array([[1.0, 0.0], [0.0, 1.0]])[None, None]
    k = np.array([[1.0, 0.0], [1.0, 0.0]])[None, None]
    v = np.array([[1.0, 2.0], [3.0, -1.0]])[None, None]
    s = 1.0 / math.sqrt(2.0)
    e = math.exp(-s * math.sin(1.0))
    p10, p11 = e / (e + 1.0), 1.0 / (e + 1.0)
    o, lse = oracle.attention_forward(q, k, v)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 2.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], [p10 * 1 + p11 * 3, p10 * 2 - p11 * 1], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [s * 1.0, math.log(e + 1.0)], rtol=1e-14)


# ---------------------------------------------------------- gradients ---------

def _loss(q, k, v, do):
    o, _ = oracle.attention_forward(q, k, v)
    return float(np.sum(o * do))


@pytest.mark.parametrize("T,D", [(1, 2), (2, 4), (5, 8), (8, 2), (8, 8), (5, 4)])
def test_gradients_match_centred_differences(T, D):
    """The pages' own check: analytic gradients against centred differences in
    double precision, RoPE included ("Show HN: NanoEuler", paragraph 2)."""
    q, k, v, do = (rand((1, 1, T, D), 40 + s) for s in range(4))
    grads = oracle.attention_backward(q, k, v, do)
    h = 1e-6
    for x, g in zip((q, k, v), grads):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(q, k, v, do)
            x[idx] = keep - h
            lm = _loss(q, k, v, do)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_gradient_identities():
    B, H, T, D = 2, 2, 37, 16
    q, k, v, do = (rand((B, H, T, D), 50 + s) for s in range(4))
    o, _ = oracle.attention_forward(q, k, v)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, return_delta=True)
    # scaling q by a and k by 1/a leaves the loss unchanged
    np.testing.assert_allclose((q * dq).sum((2, 3)), (k * dk).sum((2, 3)), rtol=1e-10, atol=1e-12)
    # the loss is linear in v
    np.testing.assert_allclose((v * dv).sum((2, 3)), (o * do).sum((2, 3)), rtol=1e-12)
    # delta from the softmax Jacobian equals sum_d O * dO
    np.testing.assert_allclose(delta, (o * do).sum(-1), rtol=1e-11, atol=1e-13)
    # rows of dS sum to zero, so the rotated dk sum to zero over keys
    np.testing.assert_allclose(oracle.rope(dk).sum(2), 0.0, atol=1e-12)


def test_row_chunking_changes_nothing():
    q, k, v, do = (rand((1, 2, 50, 8), 60 + s) for s in range(4))
    o1, l1 = oracle.attention_forward(q, k, v, row_chunk=1024)
    o2, l2 = oracle.attention_forward(q, k, v, row_chunk=7)
    g1 = oracle.attention_backward(q, k, v, do, row_chunk=1024)
    g2 = oracle.attention_backward(q, k, v, do, row_chunk=7)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------- independent routes ---------

@pytest.mark.parametrize("T,D", [(1, 4), (3, 2), (6, 4), (8, 8)])
def test_brute_force(T, D):
    q, k, v, do = (rand((1, 1, T, D), 70 + s) for s in range(4))
    o, lse = oracle.attention_forward(q, k, v)
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    L = lambda a: a[0, 0].tolist()
    bo, blse, _ = brute_force.head_forward(L(q), L(k), L(v))
    bdq, bdk, bdv = brute_force.head_backward(L(q), L(k), L(v), L(do))
    np.testing.assert_allclose(o[0, 0], bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], blse, rtol=1e-13)
    for a, b in ((dq, bdq), (dk, bdk), (dv, bdv)):
        np.testing.assert_allclose(a[0, 0], b, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("T,D", [(1, 2), (3, 4), (5, 8), (8, 8)])
def test_probabilities_match_brute_force(T, D):
    """The full probability matrix against the scalar implementation's P (its own
    rotation, scale and key-by-key softmax), masked entries included."""
    q, k = rand((2, 1, T, D), 110 + T), rand((2, 1, T, D), 111 + T)
    P = oracle.attention_probabilities(q, k)
    for b in range(2):
        _, _, bP = brute_force.head_forward(q[b, 0].tolist(), k[b, 0].tolist(),
                                            k[b, 0].tolist())
        np.testing.assert_allclose(P[b, 0], np.array(bP), rtol=1e-12, atol=1e-15)


def test_probabilities_times_values_is_the_forward():
    """P V equals the forward's output (the forward does not go through
    attention_probabilities), and exp(S - lse) rebuilds P from the forward's lse."""
    q, k, v = (rand((1, 2, 11, 8), 120 + s) for s in range(3))
    P = oracle.attention_probabilities(q, k)
    o, lse = oracle.attention_forward(q, k, v)
    np.testing.assert_allclose(P @ v, o, rtol=1e-12, atol=1e-13)
    qr, kr = oracle.rope(q), oracle.rope(k)
    S = (qr @ np.swapaxes(kr, -1, -2)) / np.sqrt(8.0)
    mask = np.triu(np.ones((11, 11), bool), 1)
    rebuilt = np.where(mask, 0.0, np.exp(S - lse[..., None]))
    np.testing.assert_allclose(P, rebuilt, rtol=1e-12, atol=1e-15)


def test_torch_sdpa_float64_cross_check():
    torch = pytest.importorskip("torch")
    B, H, T, D = 2, 3, 45, 16
    q, k, v, do = (rand((B, H, T, D), 80 + s) for s in range(4))

    def rope_real(x):
        # written as a real 2x2 rotation with torch ops, independently of the oracle
        pos = torch.arange(T, dtype=torch.float64)[:, None]
        inv = 10000.0 ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        c, s = torch.cos(pos * inv), torch.sin(pos * inv)
        x0, x1 = x[..., 0::2], x[..., 1::2]
        return torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1).flatten(-2)

    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        rope_real(tq), rope_real(tk), tv, is_causal=True)
    (out * torch.tensor(do)).sum().backward()
    o, _ = oracle.attention_forward(q, k, v)
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- decode ---------

@pytest.mark.parametrize("pos,L,D", [(0, 1, 8), (5, 9, 8), (33, 34, 16), (63, 100, 64)])
def test_decode_is_a_row_of_the_forward(pos, L, D):
    """A generation step at position pos sees exactly what row pos of the causal
    forward over positions 0 .. pos sees (the other query rows are arbitrary)."""
    B, H = 2, 3
    q = rand((B, H, D), 300 + pos)
    k, v = rand((B, H, L, D), 301 + pos), rand((B, H, L, D), 302 + pos)
    o, lse = oracle.attention_decode(q, k, v, pos)
    qf = rand((B, H, pos + 1, D), 303)
    qf[:, :, pos] = q
    of, lf = oracle.attention_forward(qf, k[:, :, :pos + 1], v[:, :, :pos + 1])
    np.testing.assert_allclose(o, of[:, :, pos], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lf[:, :, pos], rtol=1e-13, atol=1e-13)


def test_decode_closed_forms():
    B, H, L, D = 2, 2, 40, 16
    k, v = rand((B, H, L, D), 310), rand((B, H, L, D), 311)
    q = rand((B, H, D), 312)
    # position 0: the only key is the query's own position and R_0 = I
    o, lse = oracle.attention_decode(q, k, v, 0)
    np.testing.assert_array_equal(o, v[:, :, 0])
    np.testing.assert_allclose(lse, (q * k[:, :, 0]).sum(-1) / 4.0, rtol=1e-14)
    # an all-zero query weighs positions 0 .. pos equally
    for pos in (1, 17, 39):
        o, lse = oracle.attention_decode(np.zeros((B, H, D)), k, v, pos)
        np.testing.assert_allclose(o, v[:, :, :pos + 1].mean(axis=2), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, math.log(pos + 1), rtol=1e-14)


def test_decode_reads_nothing_past_pos():
    B, H, L, D = 1, 2, 30, 8
    q, k, v = rand((B, H, D), 320), rand((B, H, L, D), 321), rand((B, H, L, D), 322)
    pos = 11
    o, lse = oracle.attention_decode(q, k, v, pos)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, pos + 1:] = rand((B, H, L - pos - 1, D), 323)
    v2[:, :, pos + 1:] = np.nan
    o2, lse2 = oracle.attention_decode(q, k2, v2, pos)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# ------------------------------------------------------ planted mistakes ---------

def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the oracle fails at least one independent pin."""
    import oracle.attention as A
    q, k, v, do = (rand((1, 1, 6, 4), 90 + s) for s in range(4))
    L = lambda a: a[0, 0].tolist()
    bo, _, _ = brute_force.head_forward(L(q), L(k), L(v))
    bdq, bdk, bdv = brute_force.head_backward(L(q), L(k), L(v), L(do))

    def fwd_ok():
        o, _ = A.attention_forward(q, k, v)
        return np.allclose(o[0, 0], bo, rtol=1e-10, atol=1e-12)

    def bwd_ok():
        g = A.attention_backward(q, k, v, do)
        return all(np.allclose(a[0, 0], b, rtol=1e-8, atol=1e-10) for a, b in zip(g, (bdq, bdk, bdv)))

    assert fwd_ok() and bwd_ok()
    real_rope = A.rope
    # wrong rotation sign
    monkeypatch.setattr(A, "rope", lambda x, base=10000.0, inverse=False: real_rope(x, base, not inverse))
    assert not fwd_ok()
    monkeypatch.setattr(A, "rope", real_rope)
    # strict mask u < t instead of u <= t: row 0 would be empty, so check row 1 onwards
    real_scores = A._scores

    def strict(qr_rows, kr, row0, scale):
        S = real_scores(qr_rows, kr, row0, scale)
        t = np.arange(row0, row0 + qr_rows.shape[0])
        for i, tt in enumerate(t):
            if tt > 0:
                S[i, tt] = -np.inf
        return S
    monkeypatch.setattr(A, "_scores", strict)
    assert not fwd_ok()
    monkeypatch.setattr(A, "_scores", real_scores)
    # gradient taken with respect to the rotated inputs (RoPE backward dropped)
    monkeypatch.setattr(A, "rope", lambda x, base=10000.0, inverse=False:
                        np.asarray(x, float).copy() if inverse else real_rope(x, base))
    assert fwd_ok() and not bwd_ok()
    monkeypatch.setattr(A, "rope", real_rope)
    # a decode query rotated at position 0 instead of its own position
    qd, kd, vd = rand((1, 1, 4), 95), rand((1, 1, 6, 4), 96), rand((1, 1, 6, 4), 97)
    bo = brute_force.head_forward(L(np.concatenate([kd[:, :, :5], qd[:, :, None]], 2)),
                                  L(kd), L(vd))[0]
    assert np.allclose(A.attention_decode(qd, kd, vd, 5)[0][0, 0], bo[5], rtol=1e-10)
    monkeypatch.setattr(A, "rope", lambda x, base=10000.0, inverse=False, positions=None:
                        real_rope(x, base, inverse, None if positions is None else [0]))
    assert not np.allclose(A.attention_decode(qd, kd, vd, 5)[0][0, 0], bo[5], rtol=1e-6)
