// Backward pre-pass: the per-row quantities the gradient kernels need,
// delta_t = sum_d dO[t,d] o[t,d] (the row sum of P * dP, since o_t = sum_u P v_u)
// and, for the 16-bit kernels, lse_t * log2(e). They depend only on rows of o, dO
// and lse, so one memory-bound pass computes them before the gradient kernels,
// which then have no dependency on each other.
//
// Layout written to the workspace:
//   bf16/fp16: ws[r] = -lse_r * log2(e), ws[R + r] = -delta_r  (R = B*H*T rows;
//              negated because they are the initial accumulators of the
//              S*log2(e) and dP products)
//   fp32:      ws[r] = delta_r
#include "device_common.h"
#include "launchers.h"

namespace attn {

// LPR lanes share one row; each loads 16 consecutive bytes of o and of dO, so a
// wave reads whole rows contiguously. Plain [B, H, T, D] tensors are walked as
// one flat array of rows; STRIDED ones (rows where the Layout puts them) give
// each head `bph` consecutive workgroups.
//
// ROT (16-bit path, the backward without a saved buffer): the same thread also
// rotates the same 16 bytes of its row of q and of k - the one chunk of four
// feature pairs the rotation helper takes - and writes the rotated, scaled q and
// the rotated k (fp16, [B, H, T, D] each, bitwise what the forward forms) to
// `rot`, so the rotation costs no pass of its own.
template <typename E, int D, bool HALF_LAYOUT, bool STRIDED, bool ROT>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const E* __restrict__ o,
                                                       const E* __restrict__ dO, Layout lo,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ ws, int H, int T,
                                                       int bph, long long rows,
                                                       const E* __restrict__ q,
                                                       const E* __restrict__ k, Layout lqk,
                                                       const float* __restrict__ cs,
                                                       const float* __restrict__ sn,
                                                       f16* __restrict__ rot, float qs) {
    constexpr int EPL = 16 / (int)sizeof(E);  // elements per 16-byte load
    constexpr int LPR = D / EPL;              // lanes per row (8 .. 32)
    static_assert(LPR >= 2 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
    static_assert(!ROT || EPL == 8, "the rotation takes 8 features of a 16-bit row");
    long long row, e0, qk0 = 0;
    int part, t;
    bool valid;
    if constexpr (STRIDED) {
        const int bh = blockIdx.x / bph;
        const int i = (blockIdx.x - bh * bph) * 256 + threadIdx.x;
        t = i / LPR;
        part = i % LPR;
        valid = t < T;
        row = (long long)bh * T + t;
        e0 = lo.head(bh, H) + (long long)t * lo.st + part * EPL;
        if constexpr (ROT) qk0 = lqk.head(bh, H) + (long long)t * lqk.st + part * EPL;
    } else {
        const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
        row = gid / LPR;
        part = (int)(gid % LPR);
        valid = row < rows;
        t = (int)(row % T);
        e0 = row * D + part * EPL;
        qk0 = e0;
    }
    float acc = 0.f, nl = 0.f;
    if (valid) {
        // lse is loaded with the rows, and the scheduling barrier keeps the
        // compiler from issuing it only once o has arrived: a thread waits for
        // one memory round trip, not two
        if constexpr (HALF_LAYOUT) nl = lse[row];
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + e0);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dO + e0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ROT) {
            const u32x4 wq = *reinterpret_cast<const u32x4*>(q + qk0);
            const u32x4 wk = *reinterpret_cast<const u32x4*>(k + qk0);
            const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + (size_t)t * (D / 2) + 4 * part);
            const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + (size_t)t * (D / 2) + 4 * part);
            const size_t dst = (size_t)row * D + part * 8;
            *reinterpret_cast<u32x4*>(rot + dst) = rope_chunk_f16<E>(wq, cv, sv, qs);
            *reinterpret_cast<u32x4*>(rot + (size_t)rows * D + dst) = rope_chunk_f16<E>(wk, cv, sv, 1.f);
        }
        if constexpr (sizeof(E) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x2 x = unpack2<E>(a[e]), y = unpack2<E>(b[e]);
                acc += x[0] * y[0] + x[1] * y[1];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += __uint_as_float(a[e]) * __uint_as_float(b[e]);
        }
    }
    // the LPR lanes of a row are consecutive and LPR divides the wave
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (valid && part == 0) {
        if constexpr (HALF_LAYOUT) {
            ws[row] = -nl * kLog2e;
            ws[rows + row] = -acc;
        } else {
            ws[row] = acc;
        }
    }
}

template <typename E, int D, bool HALF_LAYOUT, bool ROT>
static hipError_t launch_prep_t(const BwdArgs& a, f16* rot) {
    constexpr int LPR = D / (16 / (int)sizeof(E));
    const long long rows = (long long)a.B * a.H * a.T;
    const float qs = kLog2e / sqrtf((float)D);
    // rows not D apart (o, dO, or with ROT q, k): a strided layout (see Layout)
    if (a.lo.st != D || (ROT && a.lqkv.st != D)) {
        const int bph = (a.T * LPR + 255) / 256;
        const unsigned blocks = (unsigned)((long long)a.B * a.H * bph);
        hipLaunchKernelGGL((bwd_prep_kernel<E, D, HALF_LAYOUT, true, ROT>), dim3(blocks),
                           dim3(256), 0, a.stream, (const E*)a.o, (const E*)a.dO, a.lo, a.lse,
                           a.ws, a.H, a.T, bph, rows, (const E*)a.q, (const E*)a.k, a.lqkv, a.cs,
                           a.sn, rot, qs);
    } else {
        const unsigned blocks = (unsigned)((rows * LPR + 255) / 256);
        hipLaunchKernelGGL((bwd_prep_kernel<E, D, HALF_LAYOUT, false, ROT>), dim3(blocks),
                           dim3(256), 0, a.stream, (const E*)a.o, (const E*)a.dO, a.lo, a.lse,
                           a.ws, a.H, a.T, 0, rows, (const E*)a.q, (const E*)a.k, a.lqkv, a.cs,
                           a.sn, rot, qs);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_prep16(const BwdArgs& a, bool f16_storage, void* rot) {
    f16* r = static_cast<f16*>(rot);
    if (f16_storage) {
        if (rot) return a.D == 64 ? launch_prep_t<f16, 64, true, true>(a, r) : launch_prep_t<f16, 128, true, true>(a, r);
        return a.D == 64 ? launch_prep_t<f16, 64, true, false>(a, r) : launch_prep_t<f16, 128, true, false>(a, r);
    }
    if (rot) return a.D == 64 ? launch_prep_t<bf16, 64, true, true>(a, r) : launch_prep_t<bf16, 128, true, true>(a, r);
    return a.D == 64 ? launch_prep_t<bf16, 64, true, false>(a, r) : launch_prep_t<bf16, 128, true, false>(a, r);
}

hipError_t launch_bwd_prep_f32(const BwdArgs& a) {
    return a.D == 64 ? launch_prep_t<float, 64, false, false>(a, nullptr)
                     : launch_prep_t<float, 128, false, false>(a, nullptr);
}

}  // namespace attn
