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

// The bytes [p, p + n) a call reads or writes through one pointer argument.
struct Span {
    const void* p;
    size_t n;
};

bool overlap(const Span& a, const Span& b) {
    if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// True when an output's bytes overlap an input's or another output's (null
// pointers and empty spans are skipped).
bool any_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (const Span& a : outs) {
        for (const Span& b : ins)
            if (overlap(a, b)) return true;
        for (const Span& b : outs)
            if (&a != &b && overlap(a, b)) return true;
    }
    return false;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

// Byte sizes of the attention tensors of one call.
struct Sizes {
    size_t x;    // one [B, H, T, D] tensor of the dtype
    size_t row;  // one [B, H, T] fp32 tensor (lse)
    size_t tab;  // one [T, D/2] fp32 table
    Sizes(int B, int H, int T, int D, int dtype)
        : x((size_t)B * H * T * D * elem_bytes(dtype)),
          row((size_t)4 * B * H * T),
          tab((size_t)T * (D / 2) * 4) {}
};

size_t saved_need(int B, int H, int T, int D, int dtype) {
    return dtype != ATTN_F32 ? round256((size_t)4 * B * H * T * D) : 0;
}

// per-row entries of the pre-pass: -lse*log2(e) and -delta (16-bit), delta (fp32)
size_t rows_need(int B, int H, int T, int dtype) {
    return round256((size_t)(dtype != ATTN_F32 ? 8 : 4) * B * H * T);
}

// attn_bwd: the per-row entries, then (16-bit path) room for the rotated q, k
size_t workspace_need(int B, int H, int T, int D, int dtype) {
    return rows_need(B, H, T, dtype) + saved_need(B, H, T, D, dtype);
}

// the rotated q/k buffer an entry point reads or writes: used by the 16-bit path only
int check_saved(const void* saved, size_t saved_bytes, int B, int H, int T, int D, int dtype) {
    if (dtype == ATTN_F32) return ATTN_OK;
    if (saved == nullptr) return ATTN_ERR_NULL;
    if (misaligned(saved)) return ATTN_ERR_ALIGN;
    if (saved_bytes < saved_need(B, H, T, D, dtype)) return ATTN_ERR_SAVED;
    return ATTN_OK;
}

int check_workspace(const void* ws, size_t ws_bytes, size_t need) {
    if (ws == nullptr || ws_bytes < need) return ATTN_ERR_WORKSPACE;
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

attn::FwdArgs fwd_args(const void* q, const void* k, const void* v, const float* cs,
                       const float* sn, const void* rot, void* o, float* lse, int B, int H, int T,
                       int D, void* stream) {
    attn::FwdArgs a = {};
    a.q = q; a.k = k; a.v = v; a.cs = cs; a.sn = sn; a.rot = rot;
    a.o = o; a.lse = lse;
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

// the part of an attn_bwd workspace that holds the rotated q, k (16-bit path)
void* ws_rotated(void* ws, int B, int H, int T, int dtype) {
    return static_cast<char*>(ws) + rows_need(B, H, T, dtype);
}

// The forward of the [B, H, T, D] entry points. 16-bit path: without `save`, one
// launch of the RoPE-on-load kernel; with it, the rotation pass writes the
// rotated q, k there and the forward reads them (the backward needs them too,
// and one pass that feeds both is cheaper than the loader writing them out).
// fp32: the fp32 kernel (save ignored).
int run_fwd(const void* q, const void* k, const void* v, const float* cs, const float* sn,
            void* o, float* lse, void* save, int B, int H, int T, int D, int dtype,
            void* stream) {
    if (dtype == ATTN_F32)
        return hip_status(attn::launch_fwd_f32(
            fwd_args(q, k, v, cs, sn, nullptr, o, lse, B, H, T, D, stream)));
    if (save != nullptr) {
        const int st = hip_status(attn::launch_rotate_qk(q, k, attn::layout_bhtd(H, T, D), cs, sn,
                                                         save, B, H, T, D, dtype == ATTN_F16,
                                                         static_cast<hipStream_t>(stream)));
        if (st) return st;
    }
    return hip_status(attn::launch_fwd16(
        fwd_args(q, k, v, cs, sn, save, o, lse, B, H, T, D, stream), dtype == ATTN_F16));
}

// The backward's two stages, from a buffer of rotated q, k (16-bit path; the
// fp32 kernels rotate on load and ignore `rot`).
int run_bwd_stages(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, const float* cs, const float* sn, const void* rot,
                   void* dq, void* dk, void* dv, void* ws, int B, int H, int T, int D,
                   int dtype, void* stream) {
    const attn::BwdArgs a =
        bwd_args(q, k, v, o, dO, lse, cs, sn, rot, dq, dk, dv, ws, B, H, T, D, stream);
    if (dtype == ATTN_F32) {
        int st = hip_status(attn::launch_bwd_prep_f32(a));
        if (st) return st;
        st = hip_status(attn::launch_bwd_dq_f32(a));
        if (st) return st;
        return hip_status(attn::launch_bwd_dkdv_f32(a));
    }
    const int st = hip_status(attn::launch_bwd_prep16(a, dtype == ATTN_F16));
    if (st) return st;
    return hip_status(attn::launch_bwd_grads16(a, dtype == ATTN_F16));
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
    const size_t tab = (size_t)T * (D / 2) * 4;
    if (any_alias({{cos_tab, tab}, {sin_tab, tab}}, {})) return ATTN_ERR_ALIAS;
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
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{saved, saved_need(B, H, T, D, dtype)}},
                  {{q, z.x}, {k, z.x}, {cos_tab, z.tab}, {sin_tab, z.tab}}))
        return ATTN_ERR_ALIAS;
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
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{o, z.x}, {lse, z.row}}, {{v, z.x}, {saved, saved_need(B, H, T, D, dtype)}}))
        return ATTN_ERR_ALIAS;
    const attn::FwdArgs a =
        fwd_args(nullptr, nullptr, v, nullptr, nullptr, saved, o, lse, B, H, T, D, stream);
    return hip_status(attn::launch_fwd16(a, dtype == ATTN_F16));
}

int attn_fwd(const void* q, const void* k, const void* v, const float* cos_tab,
             const float* sin_tab, void* o, float* lse, int B, int H, int T, int D, int dtype,
             void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({q, k, v, cos_tab, sin_tab, o, lse});
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{o, z.x}, {lse, z.row}},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {cos_tab, z.tab}, {sin_tab, z.tab}}))
        return ATTN_ERR_ALIAS;
    return run_fwd(q, k, v, cos_tab, sin_tab, o, lse, nullptr, B, H, T, D, dtype, stream);
}

int attn_fwd_save(const void* q, const void* k, const void* v, const float* cos_tab,
                  const float* sin_tab, void* o, float* lse, void* saved, size_t saved_bytes,
                  int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({q, k, v, cos_tab, sin_tab, o, lse});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    const Span sv = {dtype == ATTN_F32 ? nullptr : saved, saved_need(B, H, T, D, dtype)};
    if (any_alias({{o, z.x}, {lse, z.row}, sv},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {cos_tab, z.tab}, {sin_tab, z.tab}}))
        return ATTN_ERR_ALIAS;
    return run_fwd(q, k, v, cos_tab, sin_tab, o, lse, saved, B, H, T, D, dtype, stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int T, int D, int dtype) {
    if (check_shape(B, H, T, D, dtype) != ATTN_OK) return 0;
    return workspace_need(B, H, T, D, dtype);
}

int attn_bwd_prep(const void* q, const void* k, const void* o, const void* dO, const float* lse,
                  const float* cos_tab, const float* sin_tab, void* workspace,
                  size_t workspace_bytes, int B, int H, int T, int D, int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({o, dO, lse});
    if (st) return st;
    // with q and k (16-bit path) the pass also writes their rotation to the workspace
    const bool rotate = dtype != ATTN_F32 && (q != nullptr || k != nullptr);
    if (rotate) {
        st = check_ptrs({q, k, cos_tab, sin_tab});
        if (st) return st;
    }
    const size_t need = rotate ? workspace_need(B, H, T, D, dtype) : rows_need(B, H, T, dtype);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{workspace, need}},
                  {{o, z.x}, {dO, z.x}, {lse, z.row}, {rotate ? q : nullptr, z.x},
                   {rotate ? k : nullptr, z.x}, {rotate ? cos_tab : nullptr, z.tab},
                   {rotate ? sin_tab : nullptr, z.tab}}))
        return ATTN_ERR_ALIAS;
    const attn::BwdArgs a = bwd_args(q, k, nullptr, o, dO, lse, cos_tab, sin_tab, nullptr, nullptr,
                                     nullptr, nullptr, workspace, B, H, T, D, stream);
    if (dtype == ATTN_F32) return hip_status(attn::launch_bwd_prep_f32(a));
    return hip_status(attn::launch_bwd_prep16(
        a, dtype == ATTN_F16, rotate ? ws_rotated(workspace, B, H, T, dtype) : nullptr));
}

int attn_bwd_grads(const void* q, const void* k, const void* v, const void* dO,
                   const float* lse, const float* cos_tab, const float* sin_tab,
                   const void* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                   const void* workspace, size_t workspace_bytes, int B, int H, int T, int D,
                   int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    // the 16-bit kernels take the rotated q, k from `saved` (or, without it, from
    // the workspace, where attn_bwd_prep wrote them) and do not read q, k
    st = dtype == ATTN_F32 ? check_ptrs({q, k, v, dO, lse, cos_tab, sin_tab, dq, dk, dv})
                           : check_ptrs({v, dO, lse, cos_tab, sin_tab, dq, dk, dv});
    if (st) return st;
    const bool in_ws = dtype != ATTN_F32 && saved == nullptr;
    if (!in_ws) {
        st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
        if (st) return st;
    }
    const size_t need = in_ws ? workspace_need(B, H, T, D, dtype) : rows_need(B, H, T, dtype);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    const Span sv = {dtype == ATTN_F32 ? nullptr : saved, saved_need(B, H, T, D, dtype)};
    if (any_alias({{dq, z.x}, {dk, z.x}, {dv, z.x}},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {dO, z.x}, {lse, z.row}, {cos_tab, z.tab},
                   {sin_tab, z.tab}, sv, {workspace, need}}))
        return ATTN_ERR_ALIAS;
    const void* rot = in_ws ? ws_rotated(const_cast<void*>(workspace), B, H, T, dtype) : saved;
    const attn::BwdArgs a = bwd_args(q, k, v, nullptr, dO, lse, cos_tab, sin_tab, rot, dq, dk,
                                     dv, workspace, B, H, T, D, stream);
    if (dtype != ATTN_F32) return hip_status(attn::launch_bwd_grads16(a, dtype == ATTN_F16));
    st = hip_status(attn::launch_bwd_dq_f32(a));
    if (st) return st;
    return hip_status(attn::launch_bwd_dkdv_f32(a));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, const float* cos_tab, const float* sin_tab, void* dq, void* dk,
             void* dv, void* workspace, size_t workspace_bytes, int B, int H, int T, int D,
             int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({q, k, v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv});
    if (st) return st;
    const size_t need = workspace_need(B, H, T, D, dtype);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{dq, z.x}, {dk, z.x}, {dv, z.x}, {workspace, need}},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {o, z.x}, {dO, z.x}, {lse, z.row},
                   {cos_tab, z.tab}, {sin_tab, z.tab}}))
        return ATTN_ERR_ALIAS;
    if (dtype == ATTN_F32)
        return run_bwd_stages(q, k, v, o, dO, lse, cos_tab, sin_tab, nullptr, dq, dk, dv,
                              workspace, B, H, T, D, dtype, stream);
    // the pre-pass also rotates this call's q and k into the workspace, then the
    // gradient kernel reads them there
    void* rot = ws_rotated(workspace, B, H, T, dtype);
    const attn::BwdArgs a =
        bwd_args(q, k, v, o, dO, lse, cos_tab, sin_tab, rot, dq, dk, dv, workspace, B, H, T, D,
                 stream);
    st = hip_status(attn::launch_bwd_prep16(a, dtype == ATTN_F16, rot));
    if (st) return st;
    return hip_status(attn::launch_bwd_grads16(a, dtype == ATTN_F16));
}

int attn_bwd_saved(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, const float* cos_tab, const float* sin_tab,
                   const void* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int H, int T, int D,
                   int dtype, void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = dtype == ATTN_F32 ? check_ptrs({q, k, v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv})
                           : check_ptrs({v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    const size_t need = rows_need(B, H, T, dtype);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    const Span sv = {dtype == ATTN_F32 ? nullptr : saved, saved_need(B, H, T, D, dtype)};
    if (any_alias({{dq, z.x}, {dk, z.x}, {dv, z.x}, {workspace, need}},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {o, z.x}, {dO, z.x}, {lse, z.row},
                   {cos_tab, z.tab}, {sin_tab, z.tab}, sv}))
        return ATTN_ERR_ALIAS;
    return run_bwd_stages(q, k, v, o, dO, lse, cos_tab, sin_tab, saved, dq, dk, dv, workspace, B,
                          H, T, D, dtype, stream);
}

int attn_fwd_packed(const void* qkv, const float* cos_tab, const float* sin_tab, void* o,
                    float* lse, void* saved, size_t saved_bytes, int B, int H, int T, int D,
                    int dtype, void* stream) {
    int st = check_packed(B, H, T, D, dtype);
    if (st) return st;
    st = check_ptrs({qkv, cos_tab, sin_tab, o, lse});
    if (st) return st;
    if (saved != nullptr) {
        st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
        if (st) return st;
    }
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{o, z.x}, {lse, z.row}, {saved, saved_need(B, H, T, D, dtype)}},
                  {{qkv, 3 * z.x}, {cos_tab, z.tab}, {sin_tab, z.tab}}))
        return ATTN_ERR_ALIAS;
    const attn::Layout lqkv = attn::layout_bthd(H, T, D, 3);
    if (saved != nullptr) {  // the rotation pass, then the forward from its output
        st = hip_status(attn::launch_rotate_qk(packed_slot(qkv, 0, H, D), packed_slot(qkv, 1, H, D),
                                               lqkv, cos_tab, sin_tab, saved, B, H, T, D,
                                               dtype == ATTN_F16, static_cast<hipStream_t>(stream)));
        if (st) return st;
    }
    attn::FwdArgs a = fwd_args(packed_slot(qkv, 0, H, D), packed_slot(qkv, 1, H, D),
                               packed_slot(qkv, 2, H, D), cos_tab, sin_tab, saved, o, lse, B, H, T,
                               D, stream);
    a.lqkv = lqkv;
    a.lo = attn::layout_bthd(H, T, D, 1);
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
    if (saved != nullptr) {
        st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
        if (st) return st;
    }
    // without a saved buffer the rotated q, k go into the workspace
    const size_t need = saved != nullptr ? rows_need(B, H, T, dtype)
                                         : workspace_need(B, H, T, D, dtype);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st) return st;
    const Sizes z(B, H, T, D, dtype);
    if (any_alias({{dqkv, 3 * z.x}, {workspace, need}},
                  {{qkv, 3 * z.x}, {o, z.x}, {dO, z.x}, {lse, z.row}, {cos_tab, z.tab},
                   {sin_tab, z.tab}, {saved, saved_need(B, H, T, D, dtype)}}))
        return ATTN_ERR_ALIAS;
    // without a saved buffer the pre-pass also rotates q and k, into the workspace
    void* fresh = saved == nullptr ? ws_rotated(workspace, B, H, T, dtype) : nullptr;
    const void* rot = saved != nullptr ? saved : fresh;
    char* g = static_cast<char*>(dqkv);
    attn::BwdArgs a = bwd_args(packed_slot(qkv, 0, H, D), packed_slot(qkv, 1, H, D),
                               packed_slot(qkv, 2, H, D), o, dO, lse, cos_tab, sin_tab, rot, g,
                               g + (size_t)H * D * 2, g + (size_t)2 * H * D * 2, workspace, B, H,
                               T, D, stream);
    a.lqkv = attn::layout_bthd(H, T, D, 3);
    a.lo = attn::layout_bthd(H, T, D, 1);
    st = hip_status(attn::launch_bwd_prep16(a, dtype == ATTN_F16, fresh));
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
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_VALUE: return "invalid scalar argument";
        case ATTN_ERR_SAVED: return "saved rotated q/k buffer too small";
        case ATTN_ERR_SCRATCH: return "too large for the library's static scratch";
        default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

// ---- the backward of a training step without a workspace argument ----
//
// attn_bwd_saved_noalloc is attn_bwd_saved for callers that cannot allocate (code
// under graph capture, tight serving loops): the pre-pass's per-row entries go to
// `scratch`, a file-scope device array the library owns, instead of a workspace
// the caller passes. Each GPU the library runs on holds its own copy until the
// process ends; every call on a GPU overwrites that GPU's copy, so calls that
// overlap on one GPU (other streams, other threads) race.

namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;

__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
void* g_scratch_addr[64] = {};

// The device address of the current device's copy of `scratch`. In host code the
// array's name stands for a host-side symbol, not device memory, so every use
// takes this address; it is looked up once per device, with that device current.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return ATTN_ERR_VALUE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (p == nullptr) return ATTN_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int attn_bwd_saved_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, const float* cos_tab,
                           const float* sin_tab, const void* saved, size_t saved_bytes,
                           void* dq, void* dk, void* dv, int B, int H, int T, int D, int dtype,
                           void* stream) {
    int st = check_shape(B, H, T, D, dtype);
    if (st) return st;
    st = dtype == ATTN_F32 ? check_ptrs({q, k, v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv})
                           : check_ptrs({v, o, dO, lse, cos_tab, sin_tab, dq, dk, dv});
    if (st) return st;
    st = check_saved(saved, saved_bytes, B, H, T, D, dtype);
    if (st) return st;
    if (rows_need(B, H, T, dtype) > kScratchBytes) return ATTN_ERR_SCRATCH;
    const Sizes z(B, H, T, D, dtype);
    const Span sv = {dtype == ATTN_F32 ? nullptr : saved, saved_need(B, H, T, D, dtype)};
    if (any_alias({{dq, z.x}, {dk, z.x}, {dv, z.x}},
                  {{q, z.x}, {k, z.x}, {v, z.x}, {o, z.x}, {dO, z.x}, {lse, z.row},
                   {cos_tab, z.tab}, {sin_tab, z.tab}, sv}))
        return ATTN_ERR_ALIAS;
    // the kernels run on the stream's device and use that device's copy of the scratch
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (stream != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
        if (e != hipSuccess) return hip_status(e);
        if (sd != cur) return ATTN_ERR_VALUE;
    }
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st) return st;
    return run_bwd_stages(q, k, v, o, dO, lse, cos_tab, sin_tab, saved, dq, dk, dv, ws, B, H, T,
                          D, dtype, stream);
}

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
    const size_t kv = (size_t)B * H * n * D * 2, tab = (size_t)Tmax * (D / 2) * 4;
    if (any_alias({{cache, cache_need(B, H, Tmax, D)}},
                  {{k, kv}, {v, kv}, {cos_tab, tab}, {sin_tab, tab}}))
        return ATTN_ERR_ALIAS;
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
    const size_t row = (size_t)B * H * D * 2, tab = (size_t)Tmax * (D / 2) * 4;
    if (any_alias({{o, row}, {lse, (size_t)4 * B * H}, {workspace, decode_ws_need(B, H, Tmax, D)}},
                  {{q, row}, {cache, cache_need(B, H, Tmax, D)}, {cos_tab, tab}, {sin_tab, tab}}))
        return ATTN_ERR_ALIAS;
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
    const size_t row = (size_t)B * H * D * 2, tab = (size_t)Tmax * (D / 2) * 4;
    if (any_alias({{o, row}, {lse, (size_t)4 * B * H}, {workspace, decode_ws_need(B, H, Tmax, D)},
                   {cache, cache_need(B, H, Tmax, D)}},
                  {{q, row}, {k_new, row}, {v_new, row}, {cos_tab, tab}, {sin_tab, tab}}))
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
    return round256((size_t)attn::rmsnorm_bwd_parts(N, C) * C * sizeof(float));
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
    const size_t nc = (size_t)N * C * 2;
    if (any_alias({{y, nc}, {rstd, (size_t)4 * N}, {h, nc}}, {{x, nc}, {res, nc}, {g, (size_t)C * 2}}))
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
    const size_t nc = (size_t)N * C * 2;
    if (any_alias({{dh, nc}, {dg, (size_t)4 * C}, {workspace, norm_ws_need(N, C)}},
                  {{h, nc}, {g, (size_t)C * 2}, {rstd, (size_t)4 * N}, {dy, nc}, {dres, nc}}))
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
    if (any_alias({{out, (size_t)N * F * 2}}, {{u, (size_t)2 * N * F * 2}})) return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_swiglu(u, nullptr, out, N, F, false, dtype == ATTN_F16,
                                          static_cast<hipStream_t>(stream)));
}

int attn_swiglu_bwd(const void* u, const void* dout, void* du, int N, int F, int dtype,
                    void* stream) {
    int st = check_swiglu(N, F, dtype);
    if (st) return st;
    st = check_ptrs({u, dout, du});
    if (st) return st;
    if (any_alias({{du, (size_t)2 * N * F * 2}}, {{u, (size_t)2 * N * F * 2}, {dout, (size_t)N * F * 2}}))
        return ATTN_ERR_ALIAS;
    return hip_status(attn::launch_swiglu(u, dout, du, N, F, true, dtype == ATTN_F16,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
