"""Plain float64 CPU oracle: causal self-attention with rotary position embedding,
forward and analytic backward.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark may import or run this module. The GPU library
never calls it, and it shares no code, table or constant with the GPU path.

What is computed, per (batch, head) and entirely in float64:

* RoPE. The pages name rotary position embedding on the query/key projections,
  used so that attention scores depend on relative position ("Tiny Hackable
  CUDA", section 3, causal attention paragraph; "Show HN: NanoEuler", paragraph
  2, lists RoPE among the hand-written CUDA components). The pages give no
  formula, so the reading taken here is: feature pairs (2i, 2i+1) form the
  complex number z = x[2i] + j*x[2i+1], which at position t is multiplied by
  exp(+j*t*theta_i) with theta_i = base**(-2i/D), D the head dimension,
  positions counted from 0, base 10000. V is not rotated.
* Causal softmax attention. Scores S = (1/sqrt(D)) * Q^r K^r^T; a query at
  position t sees keys u <= t only (the pages: a prediction may depend only on
  earlier positions; the diagonal is kept, since an autoregressive model's
  position t reads itself). P = softmax over each row, O = P V, and
  lse_t = m_t + ln(sum_u exp(S[t,u] - m_t)), the natural log-sum-exp of the
  scaled, masked scores of row t.
* Backward. The pages' engine trains without autograd and checks every analytic
  gradient against a centred difference in double precision, RoPE included
  ("Show HN: NanoEuler", paragraph 2). With loss L = sum(O * dO):
  dV = P^T dO, dP = dO V^T, delta_t = sum_u P[t,u] dP[t,u] (the softmax
  Jacobian written out), dS = P * (dP - delta), dQ^r = s dS K^r,
  dK^r = s dS^T Q^r, and the gradients with respect to the un-rotated inputs
  are dq = R_t^T dQ^r, dk = R_u^T dK^r (multiplication by exp(-j*t*theta_i)).

* Decode. One generation step at position pos: the new query, rotated by its
  own position, against cached keys and values of positions 0 .. pos; by
  definition row pos of the causal forward over those positions.

FlashAttention is exact attention evaluated in tiles; the oracle is the plain
full-matrix definition instead, with no tiling. For long sequences the rows are
processed in groups (each row's softmax always spans all T keys), which changes
nothing but peak memory.
"""

import numpy as np

DEFAULT_BASE = 10000.0


def rope_frequencies(D, base=DEFAULT_BASE):
    """theta_i = base**(-2i/D) for i = 0 .. D/2-1 (D = head dimension)."""
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope(x, base=DEFAULT_BASE, inverse=False, positions=None):
    """Rotate each adjacent feature pair of x[..., T, D] by its position's angle.

    The pair (x[2i], x[2i+1]) at position t is read as the complex number
    x[2i] + j*x[2i+1] and multiplied by exp(+j*t*theta_i); inverse=True
    multiplies by exp(-j*t*theta_i), which is the transpose of the rotation
    and therefore carries a gradient back through RoPE. Row r of x sits at
    position r, or at positions[r] when positions (T integers) is given.
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape[-2], x.shape[-1]
    theta = rope_frequencies(D, base)
    pos = np.arange(T) if positions is None else np.asarray(positions)
    if pos.shape != (T,):
        raise ValueError("one position per row")
    angle = pos.astype(np.float64)[:, None] * theta[None, :]
    phase = np.exp((-1j if inverse else 1j) * angle)          # [T, D/2]
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * phase
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def _scores(qr_rows, kr, row0, scale):
    """Scaled scores of query rows row0.. against every key, with the causal
    mask (key u > query t) set to -inf."""
    S = scale * (qr_rows @ kr.T)
    t = np.arange(row0, row0 + qr_rows.shape[0])[:, None]
    u = np.arange(kr.shape[0])[None, :]
    S[u > t] = -np.inf
    return S


def _softmax_rows(S):
    """Row softmax and natural log-sum-exp of each row."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    denom = E.sum(axis=1, keepdims=True)
    return E / denom, m[:, 0] + np.log(denom[:, 0])


def _check(*xs):
    shape = xs[0].shape
    if len(shape) != 4:
        raise ValueError("expected [B, H, T, D] arrays")
    for x in xs:
        if x.shape != shape:
            raise ValueError("all tensors must share one [B, H, T, D] shape")
    return shape


def attention_probabilities(q, k, base=DEFAULT_BASE):
    """Full causal softmax matrix P[b, h, t, u] (for small T in tests)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, T, D = _check(q, k)
    scale = 1.0 / np.sqrt(D)
    qr, kr = rope(q, base), rope(k, base)
    P = np.empty((B, H, T, T))
    for b in range(B):
        for h in range(H):
            P[b, h], _ = _softmax_rows(_scores(qr[b, h], kr[b, h], 0, scale))
    return P


def attention_forward(q, k, v, base=DEFAULT_BASE, row_chunk=1024):
    """Causal RoPE attention forward. Returns (o [B,H,T,D], lse [B,H,T]), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, D = _check(q, k, v)
    scale = 1.0 / np.sqrt(D)
    o = np.empty((B, H, T, D))
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            qr, kr = rope(q[b, h], base), rope(k[b, h], base)
            for r0 in range(0, T, row_chunk):
                r1 = min(T, r0 + row_chunk)
                P, lse[b, h, r0:r1] = _softmax_rows(_scores(qr[r0:r1], kr, r0, scale))
                o[b, h, r0:r1] = P @ v[b, h]
    return o, lse


def attention_backward(q, k, v, do, base=DEFAULT_BASE, row_chunk=1024,
                       return_delta=False):
    """Gradients of L = sum(O * dO) with respect to the un-rotated q, k and v.

    Returns (dq, dk, dv), each [B,H,T,D] float64, and delta [B,H,T] as a fourth
    value when return_delta is set. delta is formed from the softmax Jacobian,
    sum_u P*dP, not from sum_d O*dO.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, T, D = _check(q, k, v, do)
    scale = 1.0 / np.sqrt(D)
    dq = np.empty((B, H, T, D))
    dk = np.empty((B, H, T, D))
    dv = np.empty((B, H, T, D))
    delta = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            qr, kr = rope(q[b, h], base), rope(k[b, h], base)
            dqr = np.empty((T, D))
            dkr = np.zeros((T, D))
            dvh = np.zeros((T, D))
            for r0 in range(0, T, row_chunk):
                r1 = min(T, r0 + row_chunk)
                P, _ = _softmax_rows(_scores(qr[r0:r1], kr, r0, scale))
                dO = do[b, h, r0:r1]
                dvh += P.T @ dO
                dP = dO @ v[b, h].T
                dlt = (P * dP).sum(axis=1)
                dS = P * (dP - dlt[:, None])
                dqr[r0:r1] = scale * (dS @ kr)
                dkr += scale * (dS.T @ qr[r0:r1])
                delta[b, h, r0:r1] = dlt
            dq[b, h] = rope(dqr, base, inverse=True)
            dk[b, h] = rope(dkr, base, inverse=True)
            dv[b, h] = dvh
    if return_delta:
        return dq, dk, dv, delta
    return dq, dk, dv



def attention_decode(q, k_cache, v_cache, pos, base=DEFAULT_BASE):
    """One generation step over a key/value cache.

    The pages' model generates text one token at a time, and each new position
    may attend only to itself and earlier positions ("Tiny Hackable CUDA",
    section 3, causal attention paragraph). At position `pos` the new query q
    ([B, H, D], pre-RoPE) is rotated by its own position and scored against the
    cached keys of positions 0 .. pos (k_cache [B, H, L, D], pre-RoPE, L > pos,
    each rotated by its own position); v_cache [B, H, L, D] holds the values.
    Rows of the cache past `pos` are not read. Returns (o [B, H, D],
    lse [B, H]) in float64: softmax(S) v and the natural log-sum-exp of the
    scaled scores S_u = (1/sqrt(D)) <R_pos q, R_u k_u>, u = 0 .. pos.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B, H, D] and k_cache, v_cache [B, H, L, D]")
    B, H, L, D = k_cache.shape
    if q.shape != (B, H, D) or not 0 <= pos < L:
        raise ValueError("q must be [B, H, D] and 0 <= pos < L")
    scale = 1.0 / np.sqrt(D)
    o = np.empty((B, H, D))
    lse = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            qr = rope(q[b, h][None, :], base, positions=[pos])[0]
            kr = rope(k_cache[b, h, :pos + 1], base)
            S = scale * (kr @ qr)                     # [pos + 1]
            m = S.max()
            w = np.exp(S - m)
            o[b, h] = (w @ v_cache[b, h, :pos + 1]) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return o, lse
