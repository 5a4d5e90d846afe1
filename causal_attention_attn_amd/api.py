"""Tensor-level helpers over the C ABI: they allocate outputs with torch on the
inputs' device and call the library on torch's current stream. Every step of
the computation runs in the library's HIP kernels."""

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.ATTN_BF16, torch.float16: _lib.ATTN_F16,
           torch.float32: _lib.ATTN_F32}
_tables = {}


def _dtype_code(t):
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")
    return _DTYPES[t.dtype]


def _shape(*ts):
    x = ts[0]
    if x.dim() != 4:
        raise ValueError("expected [B, H, T, D] tensors")
    for t in ts:
        if t.shape != x.shape or t.dtype != x.dtype or t.device != x.device:
            raise ValueError("tensors must share shape, dtype and device")
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, T, D]")
    return tuple(x.shape)


def _check_lse(lse, B, H, T, device):
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, T) or lse.device != device or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 [B, H, T] = {(B, H, T)} tensor on "
                         f"{device}")


def _saved_arg(saved, nsaved, device):
    """(pointer source, byte size) of a saved buffer after checking it; None when
    the dtype needs none."""
    if nsaved == 0:
        return None, 0
    if (not isinstance(saved, torch.Tensor) or saved.device != device
            or not saved.is_contiguous()):
        raise ValueError(f"saved must be the contiguous tensor forward() returned, on {device}")
    nbytes = saved.numel() * saved.element_size()
    if nbytes < nsaved:
        raise ValueError(f"saved holds {nbytes} bytes; these inputs need {nsaved}")
    return saved, nbytes


def rope_tables(T, D, base=10000.0, device=None):
    """fp32 cos/sin tables [T, D/2] built by the library's table kernel; cached
    per (device, T, D, base)."""
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    key = (dev, T, D, float(base))
    if key not in _tables:
        cs = torch.empty((T, D // 2), dtype=torch.float32, device=dev)
        sn = torch.empty_like(cs)
        _lib.attn_rope_tables(cs, sn, T, D, base)
        _tables[key] = (cs, sn)
    return _tables[key]


def forward(q, k, v, base=10000.0, save=True):
    """Causal RoPE attention forward; returns (o, lse, saved). With save=True (and
    a 16-bit dtype) `saved` is a uint8 tensor holding the rotated q and k the
    forward formed (attn_fwd_save), for backward(); otherwise it is None and the
    forward is attn_fwd."""
    B, H, T, D = _shape(q, k, v)
    dt = _dtype_code(q)
    cs, sn = rope_tables(T, D, base, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    nsaved = _lib.attn_saved_bytes(B, H, T, D, dt)
    if not save or nsaved == 0:
        _lib.attn_fwd(q, k, v, cs, sn, o, lse, B, H, T, D, dt)
        return o, lse, None
    saved = torch.empty(nsaved, dtype=torch.uint8, device=q.device)
    _lib.attn_fwd_save(q, k, v, cs, sn, o, lse, saved, nsaved, B, H, T, D, dt)
    return o, lse, saved


def backward(q, k, v, o, do, lse, saved=None, base=10000.0):
    """Gradients of sum(o * do) w.r.t. the pre-RoPE q, k and v; returns (dq, dk, dv).
    `saved`: the third value forward() returned for these q and k (attn_bwd_saved),
    or None (attn_bwd, which rotates q and k again)."""
    B, H, T, D = _shape(q, k, v, o, do)
    dt = _dtype_code(q)
    _check_lse(lse, B, H, T, q.device)
    nsaved = _lib.attn_saved_bytes(B, H, T, D, dt)
    use_saved = saved is not None and nsaved != 0
    sv, nsv = _saved_arg(saved, nsaved, q.device) if use_saved else (None, 0)
    # every argument is checked; only now is anything allocated or launched
    cs, sn = rope_tables(T, D, base, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = _lib.attn_bwd_workspace_bytes(B, H, T, D, dt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if use_saved:
        _lib.attn_bwd_saved(q, k, v, o, do, lse, cs, sn, sv, nsv, dq, dk, dv, ws, nbytes,
                            B, H, T, D, dt)
    else:
        _lib.attn_bwd(q, k, v, o, do, lse, cs, sn, dq, dk, dv, ws, nbytes, B, H, T, D, dt)
    return dq, dk, dv


def _packed_shape(qkv):
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError("expected a packed [B, T, 3, H, D] tensor")
    if not qkv.is_cuda or not qkv.is_contiguous():
        raise ValueError("the packed tensor must be a contiguous GPU tensor")
    B, T, _, H, D = qkv.shape
    return B, H, T, D


def forward_packed(qkv, base=10000.0, save=True):
    """Forward from the QKV projection's packed [B, T, 3, H, D] output; returns
    (o, lse, saved) with o as [B, T, H, D] (= [B, T, H*D], the out-projection's
    input) and saved as in forward(). 16-bit dtypes only."""
    B, H, T, D = _packed_shape(qkv)
    dt = _dtype_code(qkv)
    cs, sn = rope_tables(T, D, base, qkv.device)
    o = torch.empty((B, T, H, D), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=qkv.device)
    nsaved = _lib.attn_saved_bytes(B, H, T, D, dt)
    saved = torch.empty(nsaved, dtype=torch.uint8, device=qkv.device) if save else None
    _lib.attn_fwd_packed(qkv, cs, sn, o, lse, saved, nsaved if save else 0, B, H, T, D, dt)
    return o, lse, saved


def backward_packed(qkv, o, do, lse, saved=None, base=10000.0):
    """Gradients of sum(o * do) w.r.t. the pre-RoPE q, k and v of a packed
    [B, T, 3, H, D] tensor, returned in that layout (o and do are [B, T, H, D]);
    `saved` as in backward()."""
    B, H, T, D = _packed_shape(qkv)
    for t in (o, do):
        if (tuple(t.shape) != (B, T, H, D) or t.dtype != qkv.dtype or not t.is_contiguous()
                or t.device != qkv.device):
            raise ValueError("o and do must be contiguous [B, T, H, D] of the packed dtype and "
                             "device")
    dt = _dtype_code(qkv)
    _check_lse(lse, B, H, T, qkv.device)
    nsaved = _lib.attn_saved_bytes(B, H, T, D, dt)
    sv, nsv = (None, 0) if saved is None else _saved_arg(saved, nsaved, qkv.device)
    # every argument is checked; only now is anything allocated or launched
    cs, sn = rope_tables(T, D, base, qkv.device)
    dqkv = torch.empty_like(qkv)
    nbytes = _lib.attn_bwd_workspace_bytes(B, H, T, D, dt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=qkv.device)
    _lib.attn_bwd_packed(qkv, o, do, lse, cs, sn, sv, nsv, dqkv, ws, nbytes, B, H, T, D, dt)
    return dqkv


class KVCache:
    """A key/value cache for generation: B sequences, H heads, up to Tmax
    positions, head dimension D, 16-bit dtype. append() writes pre-RoPE keys and
    values of new positions; decode() runs one generation step."""

    def __init__(self, B, H, Tmax, D, dtype=torch.bfloat16, device=None, base=10000.0):
        self.B, self.H, self.Tmax, self.D, self.base = B, H, Tmax, D, base
        self.dtype = dtype
        self.code = _DTYPES[dtype]
        dev = torch.device(device if device is not None else "cuda")
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.nbytes = _lib.attn_kv_cache_bytes(B, H, Tmax, D, self.code)
        if self.nbytes == 0:
            raise ValueError("unsupported cache shape or dtype")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self.ws_bytes = _lib.attn_decode_workspace_bytes(B, H, Tmax, D, self.code)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.cs, self.sn = rope_tables(Tmax, D, base, self.device)

    def _on_device(self, *ts):
        for t in ts:
            if t.device != self.device:
                raise ValueError(f"tensor on {t.device}; the cache lives on {self.device}")

    def append(self, k, v, pos0):
        """k, v: [B, H, n, D] pre-RoPE keys and values of positions pos0 .. pos0+n-1."""
        B, H, n, D = k.shape
        if v.shape != k.shape or (B, H, D) != (self.B, self.H, self.D):
            raise ValueError("k and v must be [B, H, n, D] of the cache's B, H and D")
        if k.dtype != self.dtype or v.dtype != self.dtype:
            raise ValueError("k and v must have the cache's dtype")
        self._on_device(k, v)
        _lib.attn_kv_append(k.contiguous(), v.contiguous(), self.cs, self.sn, self.buf,
                            self.nbytes, pos0, n, B, H, self.Tmax, D, self.code)

    def decode(self, q, pos):
        """q: [B, H, D] pre-RoPE query at position pos; returns (o [B, H, D], lse [B, H])."""
        if tuple(q.shape) != (self.B, self.H, self.D) or q.dtype != self.dtype:
            raise ValueError("q must be [B, H, D] of the cache's dtype")
        self._on_device(q)
        o = torch.empty_like(q)
        lse = torch.empty((self.B, self.H), dtype=torch.float32, device=q.device)
        _lib.attn_decode(q.contiguous(), self.buf, self.nbytes, self.cs, self.sn, o, lse,
                         self.ws, self.ws_bytes, pos, self.B, self.H, self.Tmax, self.D,
                         self.code)
        return o, lse

    def step(self, q, k_new, v_new, pos):
        """One generation step in one launch: append the new token's pre-RoPE key
        and value ([B, H, D]) at position pos and decode its query there."""
        for t in (q, k_new, v_new):
            if tuple(t.shape) != (self.B, self.H, self.D) or t.dtype != self.dtype:
                raise ValueError("q, k_new and v_new must be [B, H, D] of the cache's dtype")
        self._on_device(q, k_new, v_new)
        o = torch.empty_like(q)
        lse = torch.empty((self.B, self.H), dtype=torch.float32, device=q.device)
        _lib.attn_decode_step(q.contiguous(), k_new.contiguous(), v_new.contiguous(), self.buf,
                              self.nbytes, self.cs, self.sn, o, lse, self.ws, self.ws_bytes, pos,
                              self.B, self.H, self.Tmax, self.D, self.code)
        return o, lse


class _Attention(torch.autograd.Function):
    """forward() and backward() as one autograd node: the forward keeps o, lse and
    the rotated q, k it formed, and the backward hands them to attn_bwd_saved."""

    @staticmethod
    def forward(ctx, q, k, v, base):
        o, lse, saved = forward(q, k, v, base=base, save=True)
        ctx.base = base
        ctx.has_saved = saved is not None
        ctx.save_for_backward(q, k, v, o, lse, *([saved] if saved is not None else []))
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, *rest = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, rest[0] if ctx.has_saved else None,
                              base=ctx.base)
        return dq, dk, dv, None


def attention(q, k, v, base=10000.0):
    """Causal RoPE attention of [B, H, T, D] q, k, v (bf16, fp16 or fp32, on the
    GPU) as a differentiable torch op: o = forward(...)[0], and o.backward() (or
    any autograd use) runs the library's backward."""
    return _Attention.apply(q, k, v, base)


class _AttentionPacked(torch.autograd.Function):
    """forward_packed() and backward_packed() as one autograd node."""

    @staticmethod
    def forward(ctx, qkv, base):
        o, lse, saved = forward_packed(qkv, base=base, save=True)
        ctx.base = base
        ctx.save_for_backward(qkv, o, lse, saved)
        return o

    @staticmethod
    def backward(ctx, do):
        qkv, o, lse, saved = ctx.saved_tensors
        return backward_packed(qkv, o, do.contiguous(), lse, saved, base=ctx.base), None


def attention_packed(qkv, base=10000.0):
    """attention() on the QKV projection's packed [B, T, 3, H, D] output (16-bit
    dtypes), returning o as [B, T, H, D]; differentiable with respect to qkv."""
    return _AttentionPacked.apply(qkv, base)


def _rows(t, what):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous GPU tensor")
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"{what}: bfloat16 or float16 expected")
    return t.reshape(-1, t.shape[-1])


class _RMSNorm(torch.autograd.Function):
    """Residual add + RMSNorm (attn_rmsnorm_fwd / attn_rmsnorm_bwd) as one node:
    outputs y and, with a residual, the stored sum h = x + res."""

    @staticmethod
    def forward(ctx, x, g, res, eps):
        x2 = _rows(x, "x")
        N, C = x2.shape
        if tuple(g.shape) != (C,) or g.dtype != x.dtype or g.device != x.device:
            raise ValueError("g must be [C] of x's dtype and device")
        if res is not None and (res.shape != x.shape or res.dtype != x.dtype
                                or res.device != x.device or not res.is_contiguous()):
            raise ValueError("res must match x")
        dt = _dtype_code(x)
        y = torch.empty_like(x)
        h = torch.empty_like(x) if res is not None else None
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
        _lib.attn_rmsnorm_fwd(x2, res, g, eps, h, y, rstd, N, C, dt)
        ctx.save_for_backward(h if res is not None else x, g, rstd)
        ctx.has_res = res is not None
        if res is None:
            return y
        return y, h

    @staticmethod
    def backward(ctx, dy, dh_out=None):
        h, g, rstd = ctx.saved_tensors
        N, C = h.reshape(-1, h.shape[-1]).shape
        dt = _dtype_code(h)
        dy = dy.contiguous() if dy is not None else torch.zeros_like(h)
        dres = dh_out.contiguous() if (ctx.has_res and dh_out is not None) else None
        dh = torch.empty_like(h)
        dg = torch.empty(C, dtype=torch.float32, device=h.device)
        nw = _lib.attn_rmsnorm_bwd_workspace_bytes(N, C, dt)
        ws = torch.empty(nw, dtype=torch.uint8, device=h.device)
        _lib.attn_rmsnorm_bwd(h, g, rstd, dy, dres, dh, dg, ws, nw, N, C, dt)
        return dh, dg.to(g.dtype), (dh if ctx.has_res else None), None


def rmsnorm(x, g, res=None, eps=1e-5):
    """y = RMSNorm(x [+ res]) * g over the last dimension (C a multiple of 256,
    up to 4096; bf16 or fp16 on the GPU), differentiable. With res, returns
    (y, h) where h = x + res is the stored residual stream. g's gradient is
    reduced in fp32 and rounded to g's dtype."""
    return _RMSNorm.apply(x, g, res, eps)


class _SwiGLU(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u):
        u2 = _rows(u, "u")
        N, F2 = u2.shape
        if F2 % 16:
            raise ValueError("the last dimension of u must be 2F with F a multiple of 8")
        out = torch.empty((*u.shape[:-1], F2 // 2), dtype=u.dtype, device=u.device)
        _lib.attn_swiglu_fwd(u2, out, N, F2 // 2, _dtype_code(u))
        ctx.save_for_backward(u)
        return out

    @staticmethod
    def backward(ctx, dout):
        (u,) = ctx.saved_tensors
        N, F2 = u.reshape(-1, u.shape[-1]).shape
        du = torch.empty_like(u)
        _lib.attn_swiglu_bwd(u, dout.contiguous(), du, N, F2 // 2, _dtype_code(u))
        return du


def swiglu(u):
    """silu(a) * b for u = [a | b] along the last dimension (the fused gate/up
    projection; bf16 or fp16 on the GPU), differentiable."""
    return _SwiGLU.apply(u)
