"""Scalar pure-Python causal RoPE attention for T <= 8: a third implementation
used only to pin the float64 oracle.

It is written independently of the oracle: the rotation uses the real 2x2 form
with math.cos/math.sin (the oracle multiplies by complex exponentials), the
softmax is accumulated key by key, and the backward goes through the full
softmax Jacobian dS[t,u] = sum_w dP[t,w] * P[t,w] * ([w == u] - P[t,u])
instead of the oracle's delta form.
"""

import math


def _rotate(vec, t, base, sign):
    D = len(vec)
    out = [0.0] * D
    for i in range(D // 2):
        ang = sign * t * base ** (-2.0 * i / D)
        c, s = math.cos(ang), math.sin(ang)
        x0, x1 = vec[2 * i], vec[2 * i + 1]
        out[2 * i] = x0 * c - x1 * s
        out[2 * i + 1] = x0 * s + x1 * c
    return out


def head_forward(q, k, v, base=10000.0):
    """q, k, v: lists of T rows of D floats. Returns (o, lse, P)."""
    T, D = len(q), len(q[0])
    s = 1.0 / math.sqrt(D)
    qr = [_rotate(q[t], t, base, +1) for t in range(T)]
    kr = [_rotate(k[u], u, base, +1) for u in range(T)]
    o, lse, P = [], [], []
    for t in range(T):
        sc = [s * sum(qr[t][d] * kr[u][d] for d in range(D)) for u in range(t + 1)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = sum(w)
        p = [x / z for x in w] + [0.0] * (T - t - 1)
        P.append(p)
        lse.append(m + math.log(z))
        o.append([sum(p[u] * v[u][d] for u in range(T)) for d in range(D)])
    return o, lse, P


def head_backward(q, k, v, do, base=10000.0):
    """Gradients of sum(O * dO) with respect to q, k, v (lists of rows)."""
    T, D = len(q), len(q[0])
    s = 1.0 / math.sqrt(D)
    qr = [_rotate(q[t], t, base, +1) for t in range(T)]
    kr = [_rotate(k[u], u, base, +1) for u in range(T)]
    _, _, P = head_forward(q, k, v, base)
    dP = [[sum(do[t][d] * v[u][d] for d in range(D)) for u in range(T)] for t in range(T)]
    dS = [[sum(dP[t][w] * P[t][w] * ((1.0 if w == u else 0.0) - P[t][u]) for w in range(T))
           for u in range(T)] for t in range(T)]
    dv = [[sum(P[t][u] * do[t][d] for t in range(T)) for d in range(D)] for u in range(T)]
    dqr = [[s * sum(dS[t][u] * kr[u][d] for u in range(T)) for d in range(D)] for t in range(T)]
    dkr = [[s * sum(dS[t][u] * qr[t][d] for t in range(T)) for d in range(D)] for u in range(T)]
    dq = [_rotate(dqr[t], t, base, -1) for t in range(T)]
    dk = [_rotate(dkr[u], u, base, -1) for u in range(T)]
    return dq, dk, dv
