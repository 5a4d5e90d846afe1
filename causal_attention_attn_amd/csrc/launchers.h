// Host-side launchers of the attention kernels. Arguments are validated by the
// C ABI layer before any of these is called; launchers only pick the template
// instance, size the grid and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Where element (b, h, t, d) of a [B, H, T, D]-indexed tensor sits, in elements
// from the tensor's base: b*sb + h*sh + t*st + d (the D features of a row are
// contiguous). Contiguous [B, H, T, D] has (H*T*D, T*D, D); a head's slice of
// token-major [B, T, H, D] has (T*H*D, D, H*D); a q, k or v slice of the packed
// [B, T, 3, H, D] projection output has (3*T*H*D, D, 3*H*D).
struct Layout {
    long long sb, sh;
    int st;
    __host__ __device__ long long head(int bh, int H) const {
        return (long long)(bh / H) * sb + (long long)(bh % H) * sh;
    }
    // bytes from a head's first element to the end of its row T-1
    __host__ __device__ unsigned int head_bytes(int T, int D) const {
        return (unsigned int)(((long long)(T - 1) * st + D) * 2);
    }
};

inline Layout layout_bhtd(int H, int T, int D) {
    return {(long long)H * T * D, (long long)T * D, D};
}
inline Layout layout_bthd(int H, int T, int D, int slots) {
    return {(long long)slots * T * H * D, D, slots * H * D};
}

struct FwdArgs {
    const void *q, *k, *v;
    const float *cs, *sn;
    const void* rot;  // 16-bit path, optional: rotated q * log2(e)/sqrt(D), then rotated k,
                      // [B, H, T, D] fp16 each (null: the forward rotates q and k on load)
    void* o;
    float* lse;
    Layout lqkv;  // q, k, v (the 16-bit path; fp32 takes [B, H, T, D] only)
    Layout lo;    // o
    int B, H, T, D;
    hipStream_t stream;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dO;
    const float *lse, *cs, *sn;
    const void* rot;  // 16-bit path: rotated q * log2(e)/sqrt(D), then rotated k, [B, H, T, D] fp16 each
    void *dq, *dk, *dv;
    float* ws;  // workspace (written by the pre-pass): 16-bit path [B, H, T] -lse*log2(e),
                // then [B, H, T] -delta; fp32 path [B, H, T] delta
    Layout lqkv;  // v, dq, dk, dv (q and k too, for fp32, which takes [B, H, T, D] only)
    Layout lo;    // o, dO
    int B, H, T, D;
    hipStream_t stream;
};

// Compute units of the current device (cached per device; 0 if HIP cannot say).
int device_cu_count();

hipError_t launch_rope_tables(float* cs, float* sn, int T, int D, double base, hipStream_t s);
// The 16-bit path (bf16 or, with f16_storage, fp16 tensors).
hipError_t launch_rotate_qk(const void* q, const void* k, Layout lqk, const float* cs,
                            const float* sn, void* out, int B, int H, int T, int D,
                            bool f16_storage, hipStream_t s);
hipError_t launch_fwd16(const FwdArgs& a, bool f16_storage);
// workspace entries; rot non-null: also the rotated q, k (from a.q, a.k) into rot
hipError_t launch_bwd_prep16(const BwdArgs& a, bool f16_storage, void* rot = nullptr);
hipError_t launch_bwd_grads16(const BwdArgs& a, bool f16_storage);  // dq, dk, dv in one launch

// Decode over a key/value cache (16-bit path): the cache is [B, H, Tmax, D] fp16
// rotated keys followed by [B, H, Tmax, D] values of the storage type.
int decode_slices(int pos);                                        // 64-key slices of 0..pos
size_t decode_workspace_floats(int B, int H, int Tmax, int D);     // partials for pos = Tmax-1
hipError_t launch_kv_append(const void* k, const void* v, const float* cs, const float* sn,
                            void* cache, int pos0, int n, int B, int H, int Tmax, int D,
                            bool f16_storage, hipStream_t s);
// knew, vnew: the new token's pre-RoPE key and value [B, H, D], written into cache
// row pos by the same launch; both null: row pos is already in the cache.
hipError_t launch_decode(const void* q, const void* knew, const void* vnew, const void* cache,
                         const float* cs, const float* sn, void* o, float* lse, float* ws, int pos,
                         int B, int H, int Tmax, int D, bool f16_storage, hipStream_t s);

// The per-layer kernels next to attention (16-bit path): residual add +
// RMSNorm and SwiGLU.
int rmsnorm_bwd_parts(int N, int C);  // workgroups of the backward = rows of its fp32 partial sums
hipError_t launch_rmsnorm_fwd(const void* x, const void* r, const void* g, float eps, void* h,
                              void* y, float* rstd, int N, int C, bool f16_storage,
                              hipStream_t s);
hipError_t launch_rmsnorm_bwd(const void* h, const void* g, const float* rstd, const void* dy,
                              const void* dres, void* dh, float* dg, float* part, int N, int C,
                              bool f16_storage, hipStream_t s);
hipError_t launch_swiglu(const void* u, const void* dout, void* out, int N, int F, bool backward,
                         bool f16_storage, hipStream_t s);

hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_prep_f32(const BwdArgs& a);    // workspace entries (delta)
hipError_t launch_bwd_dq_f32(const BwdArgs& a);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a);

}  // namespace attn
