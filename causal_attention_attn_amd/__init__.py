"""MI355X (gfx950) causal self-attention with rotary position embedding.

The computation runs in libattn.so (hand-written HIP kernels behind a C ABI,
include/attn.h); this package is its Python binding. torch provides device
memory and streams only.
"""

from ._lib import (  # noqa: F401
    ATTN_BF16,
    ATTN_F16,
    ATTN_F32,
    LIB_PATH,
    AttnError,
    attn_bwd,
    attn_bwd_saved,
    attn_bwd_saved_noalloc,
    attn_bwd_grads,
    attn_bwd_packed,
    attn_bwd_prep,
    attn_bwd_workspace_bytes,
    attn_decode,
    attn_decode_step,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_packed,
    attn_fwd_save,
    attn_fwd_rotated,
    attn_kv_append,
    attn_kv_cache_bytes,
    attn_last_hip_error,
    attn_noalloc_scratch_bytes,
    attn_rmsnorm_bwd,
    attn_rmsnorm_bwd_workspace_bytes,
    attn_rmsnorm_fwd,
    attn_rope_tables,
    attn_rotate_qk,
    attn_saved_bytes,
    attn_status_string,
    attn_swiglu_bwd,
    attn_swiglu_fwd,
    load,
)
from .api import (  # noqa: F401
    KVCache,
    attention,
    attention_packed,
    backward,
    backward_packed,
    forward,
    forward_packed,
    rmsnorm,
    rope_tables,
    swiglu,
)
