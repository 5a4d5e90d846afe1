// C ABI of libattn.so (declared in include/attn.h): argument validation, status
// codes and dispatch to the gfx950 kernels. Nothing here allocates, frees or
// synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "attn.h"
#include "launchers.h"

namespace {

thread_local int g_last_hip_error = 0;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_shape(int B, int H, int T, int D, int dtype) {
    if (dtype != ATTN_BF16 && dtype != ATTN_F16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (D != 64 && D != 128) return ATTN_ERR_SHAPE;
    if (B < 1 || H < 1 || T < 1) return ATTN_ERR_SHAPE;
    const long long elems = (long long)B * H * T * D;
    if (elems >= (1ll << 31)) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return ATTN_ERR_NULL;
    for (const void* p : ps)
        if (misaligned(p)) return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

bool any_alias(std::initializer_list<const void*> outs, std::initializer_list<const void*> ins) {
    for (const void* a : outs) {
        for (const void* b : ins)
            if (a == b) return true;
    }
    for (const void* a : outs) {
        int n = 0;
        for (const void* b : outs) n += (a == b);
        if (n > 1) return true;
    }
    return false;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t saved_need(int B, int H, int T, int D, int dtype) {
    return dtype != ATTN_F32 ? round256((size_t)4 * B * H * T * D) : 0;
}

size_t workspace_need(int B, int H, int T, int dtype) {
    return round256((size_t)(dtype != ATTN_F32 ? 8 : 4) * B * H * T);
}

// the rotated q/k buffer an entry point reads: required for bf16 and fp16, unused for fp32
int check_saved(const void* saved, size_t saved_bytes, int B, int H, int T, int D, int dtype) {
    if (dtype == ATTN_F32) return ATTN_OK;
    if (saved == nullptr) return ATTN_ERR_NULL;
    if (misaligned(saved)) return ATTN_ERR_ALIGN;
    if (saved_bytes < saved_need(B, H, T, D, dtype)) return ATTN_ERR_SAVED;
    return ATTN_OK;
}

int check_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse,
              const float* cs, const float* sn, const void* saved, size_t saved_bytes,
              const void* ws, size_t ws_bytes, int B, int H, int T, int D, int dtype) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({q, k, v, dO, lse, cs, sn});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (ws == nullptr || ws_bytes < workspace_need(B, H, T, dtype)) return ATTN_ERR_WORKSPACE;
    if (misaligned(ws)) return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

attn::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, const float* cs, const float* sn,
                       const void* saved, void* dq, void* dk, void* dv, const void* ws, int B,
                       int H, int T, int D, void* stream) {
    attn::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO;
    a.lse = lse; a.cs = cs; a.sn = sn; a.rot = saved;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.ws = static_cast<float*>(const_cast<void*>(ws));
    a.lqkv = a.lo = attn::layout_bhtd(H, T, D);
    a.B = B; a.H = H; a.T = T; a.D = D;
    a.stream = static_cast<hipStream_t>(stream);
    return a;
}

// the packed entry points: the 16-bit path only; the packed [B, T, 3, H, D]
// tensor must hold fewer than 2^31 elements (all in-head byte offsets fit 32
// bits) and a token row fewer than 2^23 (the strided tile loads form a row's
// extra offset with a 24-bit multiply)
int check_packed(int B, int H, int T, int D, int dtype) {
    const int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return ATTN_ERR_DTYPE;
    if ((long long)3 * B * H * T * D >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if ((long long)3 * H * D >= (1ll << 23)) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

// the q, k and v slices of a packed [B, T, 3, H, D] tensor (16-bit elements)
const void* packed_slot(const void* qkv, int slot, int H, int D) {
    return static_cast<const char*>(qkv) + (size_t)slot * H * D * 2;
}

}  // namespace

namespace attn {

int device_cu_count() {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0 &&
        hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = 0;
    return cus[dev];
}

}  // namespace attn

extern "C" {

int attn_rope_tables(float* cos_tab, float* sin_tab, int T, int D, double base, void* stream) {
    if (cos_tab == nullptr || sin_tab == nullptr) return ATTN_ERR_NULL;
    if (T < 1 || D < 2 || D > 1024 || (D & 1)) return ATTN_ERR_SHAPE;
    if ((long long)T * (D / 2) >= (1ll << 31)) return ATTN_ERR_SHAPE;
    if (!(base > 1.0) || base != base) return ATTN_ERR_VALUE;
    if (cos_tab == sin_tab) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_rope_tables(cos_tab, sin_tab, T, D, base,
                                               static_cast<hipStream_t>(stream)));
}

size_t attn_saved_bytes(int B, int H, int T, int D, int dtype) {
    if (check_shape(B, H, T, D, dtype) != ATTN_OK) return 0;
    return saved_need(B, H, T, D, dtype);
}

int attn_rotate_qk(const void* q, const void* k, const float* cos_tab, const float* sin_tab,
                   void* saved, size_t saved_bytes, int B, int H, int T, int D, int dtype,
                   void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return ATTN_OK;  // the fp32 path rotates on load
    st = check_ptrs({q, k, cos_tab, sin_tab});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (any_alias({saved}, {q, k, cos_tab, sin_tab})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_rotate_qk(q, k, attn::layout_bhtd(H, T, D), cos_tab, sin_tab,
                                             saved, B, H, T, D, dtype == ATTN_F16,
                                             static_cast<hipStream_t>(stream)));
}

int attn_fwd_rotated(const void* saved, size_t saved_bytes, const void* v, void* o, float* lse,
                     int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return ATTN_ERR_DTYPE;
    st = check_ptrs({v, o, lse});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (any_alias({o, lse}, {v, saved})) return ATTN_ERR_ALIAS;
    attn::FwdArgs a = {};
    a.v = v; a.rot = saved; a.o = o; a.lse = lse;
    a.lqkv = a.lo = attn::layout_bhtd(H, T, D);
    a.B = B; a.H = H; a.T = T; a.D = D;
    a.stream = static_cast<hipStream_t>(stream);
    return hip_status(attn::launch_fwd16(a, dtype == ATTN_F16));
}

int attn_fwd(const void* q, const void* k, const void* v, const float* cos_tab,
             const float* sin_tab, void* o, float* lse, void* saved, size_t saved_bytes, int B,
             int H, int T, int D, int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({q, k, v, cos_tab, sin_tab, o, lse});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (any_alias({o, lse}, {q, k, v, cos_tab, sin_tab, saved})) return ATTN_ERR_ALIAS;
    if (dtype != ATTN_F32) {
        if (any_alias({saved}, {q, k, v, cos_tab, sin_tab})) return ATTN_ERR_ALIAS;
        st = attn_rotate_qk(q, k, cos_tab, sin_tab, saved, saved_bytes, B, H, T, D, dtype,
                            stream);
        if (st) return st;
        return attn_fwd_rotated(saved, saved_bytes, v, o, lse, B, H, T, D, dtype, stream);
    }
    attn::FwdArgs a = {};
    a.q = q; a.k = k; a.v = v; a.cs = cos_tab; a.sn = sin_tab; a.o = o; a.lse = lse;
    a.lqkv = a.lo = attn::layout_bhtd(H, T, D);
    a.B = B; a.H = H; a.T = T; a.D = D;
    a.stream = static_cast<hipStream_t>(stream);
    return hip_status(attn::launch_fwd_f32(a));
}

size_t attn_bwd_workspace_bytes(int B, int H, int T, int D, int dtype) {
    if (check_shape(B, H, T, D, dtype) != ATTN_OK) return 0;
    return workspace_need(B, H, T, dtype);
}

int attn_bwd_prep(const void* o, const void* dO, const float* lse, void* workspace,
                  size_t workspace_bytes, int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({o, dO, lse});
    if (st) return st;
    if (workspace == nullptr || workspace_bytes < workspace_need(B, H, T, dtype))
        return ATTN_ERR_WORKSPACE;
    if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    if (any_alias({workspace}, {o, dO, lse})) return ATTN_ERR_ALIAS;
    const attn::BwdArgs a = bwd_args(nullptr, nullptr, nullptr, o, dO, lse, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, workspace, B, H, T, D,
                                     stream);
    return hip_status(dtype == ATTN_F32 ? attn::launch_bwd_prep_f32(a)
                                        : attn::launch_bwd_prep16(a, dtype == ATTN_F16));
}

int attn_bwd_grads(const void* q, const void* k, const void* v, const void* dO,
                   const float* lse, const float* cos_tab, const float* sin_tab,
                   const void* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                   const void* workspace, size_t workspace_bytes, int B, int H, int T, int D,
                   int dtype, void* stream) {
    int st = check_bwd(q, k, v, dO, lse, cos_tab, sin_tab, saved, saved_bytes, workspace,
                       workspace_bytes, B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({dq, dk, dv});
    if (st) return st;
    if (any_alias({dq, dk, dv}, {q, k, v, dO, lse, cos_tab, sin_tab, saved, workspace}))
        return ATTN_ERR_ALIAS;
    const attn::BwdArgs a = bwd_args(q, k, v, nullptr, dO, lse, cos_tab, sin_tab, saved, dq, dk,
                                     dv, workspace, B, H, T, D, stream);
    if (dtype != ATTN_F32) return hip_status(attn::launch_bwd_grads16(a, dtype == ATTN_F16));
    st = hip_status(attn::launch_bwd_dq_f32(a));
    if (st) return st;
    return hip_status(attn::launch_bwd_dkdv_f32(a));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, const float* cos_tab, const float* sin_tab, const void* saved,
             size_t saved_bytes, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_bwd(q, k, v, dO, lse, cos_tab, sin_tab, saved, saved_bytes, workspace,
                       workspace_bytes, B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({o, dq, dk, dv});
    if (st) return st;
    if (any_alias({dq, dk, dv, workspace}, {q, k, v, o, dO, lse, cos_tab, sin_tab, saved}))
        return ATTN_ERR_ALIAS;
    st = attn_bwd_prep(o, dO, lse, workspace, workspace_bytes, B, H, T, D, dtype, stream);
    if (st) return st;
    return attn_bwd_grads(q, k, v, dO, lse, cos_tab, sin_tab, saved, saved_bytes, dq, dk, dv,
                          workspace, workspace_bytes, B, H, T, D, dtype, stream);
}

int attn_fwd_packed(const void* qkv, const float* cos_tab, const float* sin_tab, void* o,
                    float* lse, void* saved, size_t saved_bytes, int B, int H, int T, int D,
                    int dtype, void* stream) {
    int st = check_packed(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({qkv, cos_tab, sin_tab, o, lse});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (any_alias({o, lse, saved}, {qkv, cos_tab, sin_tab})) return ATTN_ERR_ALIAS;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const attn::Layout lqkv = attn::layout_bthd(H, T, D, 3);
    st = hip_status(attn::launch_rotate_qk(packed_slot(qkv, 0, H, D), packed_slot(qkv, 1, H, D),
                                           lqkv, cos_tab, sin_tab, saved, B, H, T, D,
                                           dtype == ATTN_F16, s));
    if (st) return st;
    attn::FwdArgs a = {};
    a.v = packed_slot(qkv, 2, H, D); a.rot = saved; a.o = o; a.lse = lse;
    a.lqkv = lqkv;
    a.lo = attn::layout_bthd(H, T, D, 1);
    a.B = B; a.H = H; a.T = T; a.D = D;
    a.stream = s;
    return hip_status(attn::launch_fwd16(a, dtype == ATTN_F16));
}

int attn_bwd_packed(const void* qkv, const void* o, const void* dO, const float* lse,
                    const float* cos_tab, const float* sin_tab, const void* saved,
                    size_t saved_bytes, void* dqkv, void* workspace, size_t workspace_bytes,
                    int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_packed(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({qkv, o, dO, lse, cos_tab, sin_tab, dqkv});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (workspace == nullptr || workspace_bytes < workspace_need(B, H, T, dtype))
        return ATTN_ERR_WORKSPACE;
    if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    if (any_alias({dqkv, workspace}, {qkv, o, dO, lse, cos_tab, sin_tab, saved}))
        return ATTN_ERR_ALIAS;
    char* g = static_cast<char*>(dqkv);
    attn::BwdArgs a = bwd_args(nullptr, nullptr, packed_slot(qkv, 2, H, D), o, dO, lse, cos_tab,
                               sin_tab, saved, g, g + (size_t)H * D * 2, g + (size_t)2 * H * D * 2,
                               workspace, B, H, T, D, stream);
    a.lqkv = attn::layout_bthd(H, T, D, 3);
    a.lo = attn::layout_bthd(H, T, D, 1);
    st = hip_status(attn::launch_bwd_prep16(a, dtype == ATTN_F16));
    if (st) return st;
    return hip_status(attn::launch_bwd_grads16(a, dtype == ATTN_F16));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "null pointer";
        case ATTN_ERR_SHAPE: return "unsupported shape";
        case ATTN_ERR_DTYPE: return "unsupported dtype";
        case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_HIP: return "HIP launch failed";
        case ATTN_ERR_ALIAS: return "output aliases an input";
        case ATTN_ERR_VALUE: return "invalid scalar argument";
        case ATTN_ERR_SAVED: return "saved rotated q/k buffer too small";
        default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

// ---- decode over a key/value cache (16-bit path) ----

namespace {

int check_cache_shape(int B, int H, int Tmax, int D, int dtype) {
    const int st = check_shape(B, H, Tmax, D, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return ATTN_ERR_DTYPE;
    return ATTN_OK;
}

size_t cache_need(int B, int H, int Tmax, int D) { return round256((size_t)4 * B * H * Tmax * D); }

size_t decode_ws_need(int B, int H, int Tmax, int D) {
    return round256(attn::decode_workspace_floats(B, H, Tmax, D) * sizeof(float));
}

}  // namespace

extern "C" {

size_t attn_kv_cache_bytes(int B, int H, int Tmax, int D, int dtype) {
    if (check_cache_shape(B, H, Tmax, D, dtype) != ATTN_OK) return 0;
    return cache_need(B, H, Tmax, D);
}

size_t attn_decode_workspace_bytes(int B, int H, int Tmax, int D, int dtype) {
    if (check_cache_shape(B, H, Tmax, D, dtype) != ATTN_OK) return 0;
    return decode_ws_need(B, H, Tmax, D);
}

int attn_kv_append(const void* k, const void* v, const float* cos_tab, const float* sin_tab,
                   void* cache, size_t cache_bytes, int pos0, int n, int B, int H, int Tmax,
                   int D, int dtype, void* stream) {
    int st = check_cache_shape(B, H, Tmax, D, dtype);
    if (st) return st;
    if (n < 1 || pos0 < 0 || (long long)pos0 + n > Tmax) return ATTN_ERR_SHAPE;
    st = check_ptrs({k, v, cos_tab, sin_tab, cache});
    if (st) return st;
    if (cache_bytes < cache_need(B, H, Tmax, D)) return ATTN_ERR_WORKSPACE;
    if (any_alias({cache}, {k, v, cos_tab, sin_tab})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_kv_append(k, v, cos_tab, sin_tab, cache, pos0, n, B, H, Tmax,
                                             D, dtype == ATTN_F16,
                                             static_cast<hipStream_t>(stream)));
}

int attn_decode(const void* q, const void* cache, size_t cache_bytes, const float* cos_tab,
                const float* sin_tab, void* o, float* lse, void* workspace,
                size_t workspace_bytes, int pos, int B, int H, int Tmax, int D, int dtype,
                void* stream) {
    int st = check_cache_shape(B, H, Tmax, D, dtype);
    if (st) return st;
    if (pos < 0 || pos >= Tmax) return ATTN_ERR_SHAPE;
    st = check_ptrs({q, cache, cos_tab, sin_tab, o, lse});
    if (st) return st;
    if (cache_bytes < cache_need(B, H, Tmax, D)) return ATTN_ERR_WORKSPACE;
    if (workspace == nullptr || workspace_bytes < decode_ws_need(B, H, Tmax, D))
        return ATTN_ERR_WORKSPACE;
    if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    if (any_alias({o, lse, workspace}, {q, cache, cos_tab, sin_tab})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_decode(q, nullptr, nullptr, cache, cos_tab, sin_tab, o, lse,
                                          static_cast<float*>(workspace), pos, B, H, Tmax, D,
                                          dtype == ATTN_F16, static_cast<hipStream_t>(stream)));
}

int attn_decode_step(const void* q, const void* k_new, const void* v_new, void* cache,
                     size_t cache_bytes, const float* cos_tab, const float* sin_tab, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, int pos, int B, int H,
                     int Tmax, int D, int dtype, void* stream) {
    int st = check_cache_shape(B, H, Tmax, D, dtype);
    if (st) return st;
    if (pos < 0 || pos >= Tmax) return ATTN_ERR_SHAPE;
    st = check_ptrs({q, k_new, v_new, cache, cos_tab, sin_tab, o, lse});
    if (st) return st;
    if (cache_bytes < cache_need(B, H, Tmax, D)) return ATTN_ERR_WORKSPACE;
    if (workspace == nullptr || workspace_bytes < decode_ws_need(B, H, Tmax, D))
        return ATTN_ERR_WORKSPACE;
    if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    if (any_alias({o, lse, workspace, cache}, {q, k_new, v_new, cos_tab, sin_tab}) ||
        any_alias({o, lse, workspace}, {cache}))
        return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_decode(q, k_new, v_new, cache, cos_tab, sin_tab, o, lse,
                                          static_cast<float*>(workspace), pos, B, H, Tmax, D,
                                          dtype == ATTN_F16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- residual add + RMSNorm, SwiGLU (16-bit path) ----

namespace {

// 16-bit tensors of N rows; the largest holds `elems` elements (< 2^31)
int check_rows(int N, long long elems, int dtype) {
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_DTYPE;
    if (N < 1 || elems < 1 || elems >= (1ll << 31)) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

int check_norm(int N, int C, int dtype) {
    if (C < 256 || C > 4096 || C % 256 != 0) return dtype == ATTN_BF16 || dtype == ATTN_F16
                                                          ? ATTN_ERR_SHAPE : ATTN_ERR_DTYPE;
    return check_rows(N, (long long)N * C, dtype);
}

int check_swiglu(int N, int F, int dtype) {
    if (F < 8 || F % 8 != 0) return dtype == ATTN_BF16 || dtype == ATTN_F16 ? ATTN_ERR_SHAPE
                                                                            : ATTN_ERR_DTYPE;
    return check_rows(N, 2ll * N * F, dtype);
}

size_t norm_ws_need(int N, int C) {
    return round256((size_t)attn::rmsnorm_bwd_parts(N) * C * sizeof(float));
}

}  // namespace

extern "C" {

int attn_rmsnorm_fwd(const void* x, const void* res, const void* g, float eps, void* h, void* y,
                     float* rstd, int N, int C, int dtype, void* stream) {
    int st = check_norm(N, C, dtype);
    if (st) return st;
    if (!(eps > 0.f) || eps != eps || eps > 1e30f) return ATTN_ERR_VALUE;
    st = check_ptrs({x, g, y, rstd});
    if (st) return st;
    if ((res != nullptr && misaligned(res)) || (h != nullptr && misaligned(h))) return ATTN_ERR_ALIGN;
    if (any_alias({y, rstd}, {x, g}) || (res != nullptr && any_alias({y, rstd}, {res})) ||
        (h != nullptr && any_alias({h}, {x, g, y, rstd})) ||
        (h != nullptr && res != nullptr && h == res))
        return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_rmsnorm_fwd(x, res, g, eps, h, y, rstd, N, C,
                                               dtype == ATTN_F16, static_cast<hipStream_t>(stream)));
}

size_t attn_rmsnorm_bwd_workspace_bytes(int N, int C, int dtype) {
    if (check_norm(N, C, dtype) != ATTN_OK) return 0;
    return norm_ws_need(N, C);
}

int attn_rmsnorm_bwd(const void* h, const void* g, const float* rstd, const void* dy,
                     const void* dres, void* dh, float* dg, void* workspace,
                     size_t workspace_bytes, int N, int C, int dtype, void* stream) {
    int st = check_norm(N, C, dtype);
    if (st) return st;
    st = check_ptrs({h, g, rstd, dy, dh, dg});
    if (st) return st;
    if (dres != nullptr && misaligned(dres)) return ATTN_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < norm_ws_need(N, C)) return ATTN_ERR_WORKSPACE;
    if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    if (any_alias({dh, dg, workspace}, {h, g, rstd, dy}) ||
        (dres != nullptr && any_alias({dh, dg, workspace}, {dres})))
        return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_rmsnorm_bwd(h, g, rstd, dy, dres, dh, dg,
                                               static_cast<float*>(workspace), N, C,
                                               dtype == ATTN_F16, static_cast<hipStream_t>(stream)));
}

int attn_swiglu_fwd(const void* u, void* out, int N, int F, int dtype, void* stream) {
    int st = check_swiglu(N, F, dtype);
    if (st) return st;
    st = check_ptrs({u, out});
    if (st) return st;
    if (any_alias({out}, {u})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_swiglu(u, nullptr, out, N, F, false, dtype == ATTN_F16,
                                          static_cast<hipStream_t>(stream)));
}

int attn_swiglu_bwd(const void* u, const void* dout, void* du, int N, int F, int dtype,
                    void* stream) {
    int st = check_swiglu(N, F, dtype);
    if (st) return st;
    st = check_ptrs({u, dout, du});
    if (st) return st;
    if (any_alias({du}, {u, dout})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_swiglu(u, dout, du, N, F, true, dtype == ATTN_F16,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
