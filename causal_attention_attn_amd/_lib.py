"""ctypes binding of libattn.so: the C ABI of include/attn.h under the same names.

Argument marshalling only. Tensor arguments may be torch tensors (their
data_ptr() is passed) or plain integer device addresses; `stream` may be a
torch.cuda.Stream, an integer hipStream_t handle, or None for torch's current
stream on the current device. A non-zero status raises AttnError. There is no
fallback: if the library is missing, every call raises.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree one
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(_PKG, "libattn.so")

ATTN_BF16 = 0
ATTN_F32 = 1
ATTN_F16 = 2

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE",
    4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_ALIAS",
    8: "ATTN_ERR_VALUE", 9: "ATTN_ERR_SAVED", 10: "ATTN_ERR_SCRATCH",
}

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_SIGS = {
    "attn_rope_tables": (_I, [_P, _P, _I, _I, ctypes.c_double, _P]),
    "attn_saved_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "attn_rotate_qk": (_I, [_P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _P]),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "attn_fwd_save": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _P]),
    "attn_fwd_rotated": (_I, [_P, _Z, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "attn_bwd_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                      _I, _I, _I, _I, _I, _P]),
    "attn_bwd_saved": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _P, _P, _P, _Z,
                            _I, _I, _I, _I, _I, _P]),
    "attn_bwd_prep": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _P]),
    "attn_bwd_grads": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _P, _P, _P, _Z,
                            _I, _I, _I, _I, _I, _P]),
    "attn_fwd_packed": (_I, [_P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _P]),
    "attn_bwd_packed": (_I, [_P, _P, _P, _P, _P, _P, _P, _Z, _P, _P, _Z, _I, _I, _I, _I, _I,
                             _P]),
    "attn_kv_cache_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "attn_kv_append": (_I, [_P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _I, _I, _P]),
    "attn_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "attn_decode": (_I, [_P, _P, _Z, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _I, _P]),
    "attn_decode_step": (_I, [_P, _P, _P, _P, _Z, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I,
                              _I, _P]),
    "attn_rmsnorm_fwd": (_I, [_P, _P, _P, ctypes.c_float, _P, _P, _P, _I, _I, _I, _P]),
    "attn_rmsnorm_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "attn_rmsnorm_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _P]),
    "attn_swiglu_fwd": (_I, [_P, _P, _I, _I, _I, _P]),
    "attn_swiglu_bwd": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "attn_bwd_saved_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _P, _P,
                                    _I, _I, _I, _I, _I, _P]),
    "attn_noalloc_scratch_bytes": (_Z, []),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_hip_error": (_I, []),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        detail = ""
        if status == 6:
            detail = f" (hipError_t {load().attn_last_hip_error()})"
        name = STATUS.get(status, str(status))
        super().__init__(f"{fn} failed: {name}: "
                         f"{load().attn_status_string(status).decode()}{detail}")


def load(path=None):
    """Load libattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m causal_attention_attn_amd.build`"
                           " (the GPU path has no fallback)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != 0:
        raise AttnError(name, st)


def attn_rope_tables(cos_tab, sin_tab, T, D, base=10000.0, stream=None):
    _call("attn_rope_tables", _ptr(cos_tab), _ptr(sin_tab), T, D, float(base), _stream(stream))


def attn_saved_bytes(B, H, T, D, dtype):
    return int(load().attn_saved_bytes(B, H, T, D, dtype))


def attn_rotate_qk(q, k, cos_tab, sin_tab, saved, saved_bytes, B, H, T, D, dtype, stream=None):
    _call("attn_rotate_qk", _ptr(q), _ptr(k), _ptr(cos_tab), _ptr(sin_tab), _ptr(saved),
          int(saved_bytes), B, H, T, D, dtype, _stream(stream))


def attn_fwd(q, k, v, cos_tab, sin_tab, o, lse, B, H, T, D, dtype, stream=None):
    _call("attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(cos_tab), _ptr(sin_tab), _ptr(o),
          _ptr(lse), B, H, T, D, dtype, _stream(stream))


def attn_fwd_save(q, k, v, cos_tab, sin_tab, o, lse, saved, saved_bytes, B, H, T, D, dtype,
                  stream=None):
    _call("attn_fwd_save", _ptr(q), _ptr(k), _ptr(v), _ptr(cos_tab), _ptr(sin_tab), _ptr(o),
          _ptr(lse), _ptr(saved), int(saved_bytes), B, H, T, D, dtype, _stream(stream))


def attn_fwd_rotated(saved, saved_bytes, v, o, lse, B, H, T, D, dtype, stream=None):
    _call("attn_fwd_rotated", _ptr(saved), int(saved_bytes), _ptr(v), _ptr(o), _ptr(lse),
          B, H, T, D, dtype, _stream(stream))


def attn_bwd_workspace_bytes(B, H, T, D, dtype):
    return int(load().attn_bwd_workspace_bytes(B, H, T, D, dtype))


def attn_bwd(q, k, v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv, workspace, workspace_bytes,
             B, H, T, D, dtype, stream=None):
    _call("attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(cos_tab),
          _ptr(sin_tab), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace_bytes),
          B, H, T, D, dtype, _stream(stream))


def attn_bwd_saved(q, k, v, o, dO, lse, cos_tab, sin_tab, saved, saved_bytes, dq, dk, dv,
                   workspace, workspace_bytes, B, H, T, D, dtype, stream=None):
    _call("attn_bwd_saved", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
          _ptr(cos_tab), _ptr(sin_tab), _ptr(saved), int(saved_bytes), _ptr(dq), _ptr(dk),
          _ptr(dv), _ptr(workspace), int(workspace_bytes), B, H, T, D, dtype, _stream(stream))


def attn_bwd_prep(q, k, o, dO, lse, cos_tab, sin_tab, workspace, workspace_bytes, B, H, T, D,
                  dtype, stream=None):
    _call("attn_bwd_prep", _ptr(q), _ptr(k), _ptr(o), _ptr(dO), _ptr(lse), _ptr(cos_tab),
          _ptr(sin_tab), _ptr(workspace), int(workspace_bytes), B, H, T, D, dtype,
          _stream(stream))


def attn_bwd_grads(q, k, v, dO, lse, cos_tab, sin_tab, saved, saved_bytes, dq, dk, dv,
                   workspace, workspace_bytes, B, H, T, D, dtype, stream=None):
    _call("attn_bwd_grads", _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(cos_tab),
          _ptr(sin_tab), _ptr(saved), int(saved_bytes), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(workspace), int(workspace_bytes), B, H, T, D, dtype, _stream(stream))


def attn_fwd_packed(qkv, cos_tab, sin_tab, o, lse, saved, saved_bytes, B, H, T, D, dtype,
                    stream=None):
    _call("attn_fwd_packed", _ptr(qkv), _ptr(cos_tab), _ptr(sin_tab), _ptr(o), _ptr(lse),
          _ptr(saved), int(saved_bytes), B, H, T, D, dtype, _stream(stream))


def attn_bwd_packed(qkv, o, dO, lse, cos_tab, sin_tab, saved, saved_bytes, dqkv, workspace,
                    workspace_bytes, B, H, T, D, dtype, stream=None):
    _call("attn_bwd_packed", _ptr(qkv), _ptr(o), _ptr(dO), _ptr(lse), _ptr(cos_tab),
          _ptr(sin_tab), _ptr(saved), int(saved_bytes), _ptr(dqkv), _ptr(workspace),
          int(workspace_bytes), B, H, T, D, dtype, _stream(stream))


def attn_kv_cache_bytes(B, H, Tmax, D, dtype):
    return int(load().attn_kv_cache_bytes(B, H, Tmax, D, dtype))


def attn_kv_append(k, v, cos_tab, sin_tab, cache, cache_bytes, pos0, n, B, H, Tmax, D, dtype,
                   stream=None):
    _call("attn_kv_append", _ptr(k), _ptr(v), _ptr(cos_tab), _ptr(sin_tab), _ptr(cache),
          int(cache_bytes), pos0, n, B, H, Tmax, D, dtype, _stream(stream))


def attn_decode_workspace_bytes(B, H, Tmax, D, dtype):
    return int(load().attn_decode_workspace_bytes(B, H, Tmax, D, dtype))


def attn_decode(q, cache, cache_bytes, cos_tab, sin_tab, o, lse, workspace, workspace_bytes,
                pos, B, H, Tmax, D, dtype, stream=None):
    _call("attn_decode", _ptr(q), _ptr(cache), int(cache_bytes), _ptr(cos_tab), _ptr(sin_tab),
          _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes), pos, B, H, Tmax, D, dtype,
          _stream(stream))


def attn_decode_step(q, k_new, v_new, cache, cache_bytes, cos_tab, sin_tab, o, lse, workspace,
                     workspace_bytes, pos, B, H, Tmax, D, dtype, stream=None):
    _call("attn_decode_step", _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cache), int(cache_bytes),
          _ptr(cos_tab), _ptr(sin_tab), _ptr(o), _ptr(lse), _ptr(workspace),
          int(workspace_bytes), pos, B, H, Tmax, D, dtype, _stream(stream))


def attn_rmsnorm_fwd(x, res, g, eps, h, y, rstd, N, C, dtype, stream=None):
    _call("attn_rmsnorm_fwd", _ptr(x), _ptr(res), _ptr(g), float(eps), _ptr(h), _ptr(y),
          _ptr(rstd), N, C, dtype, _stream(stream))


def attn_rmsnorm_bwd_workspace_bytes(N, C, dtype):
    return int(load().attn_rmsnorm_bwd_workspace_bytes(N, C, dtype))


def attn_rmsnorm_bwd(h, g, rstd, dy, dres, dh, dg, workspace, workspace_bytes, N, C, dtype,
                     stream=None):
    _call("attn_rmsnorm_bwd", _ptr(h), _ptr(g), _ptr(rstd), _ptr(dy), _ptr(dres), _ptr(dh),
          _ptr(dg), _ptr(workspace), int(workspace_bytes), N, C, dtype, _stream(stream))


def attn_swiglu_fwd(u, out, N, F, dtype, stream=None):
    _call("attn_swiglu_fwd", _ptr(u), _ptr(out), N, F, dtype, _stream(stream))


def attn_swiglu_bwd(u, dout, du, N, F, dtype, stream=None):
    _call("attn_swiglu_bwd", _ptr(u), _ptr(dout), _ptr(du), N, F, dtype, _stream(stream))


def attn_bwd_saved_noalloc(q, k, v, o, dO, lse, cos_tab, sin_tab, saved, saved_bytes, dq, dk,
                           dv, B, H, T, D, dtype, stream=None):
    _call("attn_bwd_saved_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
          _ptr(cos_tab), _ptr(sin_tab), _ptr(saved), int(saved_bytes), _ptr(dq), _ptr(dk),
          _ptr(dv), B, H, T, D, dtype, _stream(stream))


def attn_noalloc_scratch_bytes():
    return int(load().attn_noalloc_scratch_bytes())


def attn_status_string(status):
    return load().attn_status_string(status).decode()


def attn_last_hip_error():
    return int(load().attn_last_hip_error())
