// RoPE cosine/sine tables: cos_tab[t][i] = cos(t * theta_i), sin_tab[t][i] =
// sin(t * theta_i), theta_i = base^(-2i/D). Rotary position embedding on the
// query/key projections is what the pages use to encode relative positions
// ("Tiny Hackable CUDA", section 3). The angle and its cosine/sine are evaluated
// in double precision (an fp32 angle would be off by up to ~5e-4 rad at
// t = 8191) and rounded once to fp32.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launchers.h"

namespace attn {

__global__ void rope_tables_kernel(float* __restrict__ cs, float* __restrict__ sn, int T,
                                   int half, int D, double base) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)T * half) return;
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)i / (double)D);
    double s, c;
    sincos((double)t * theta, &s, &c);
    cs[idx] = (float)c;
    sn[idx] = (float)s;
}

hipError_t launch_rope_tables(float* cs, float* sn, int T, int D, double base, hipStream_t st) {
    const long n = (long)T * (D / 2);
    const int threads = 256;
    const long blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, cs, sn,
                       T, D / 2, D, base);
    return hipGetLastError();
}

// Rotate q and k once: out[0] = qs * R q, out[1] = R k, both [B, H, T, D] fp16
// (rounded once from the fp32 rotation). qs = log2(e)/sqrt(D) folds the score
// scale and the change to base-2 exponentials into the query, so a score
// product comes out of the MFMA directly as S * log2(e). The 16-bit kernels read
// these instead of applying RoPE per tile. One thread per 8 consecutive
// features of one row, for q and k together (one cos/sin read serves both).
// Plain [B, H, T, D] inputs are walked as one flat array; STRIDED inputs (rows
// where the Layout puts them) give each head `bph` consecutive workgroups.
template <int D, typename E, bool STRIDED>
__global__ __launch_bounds__(256) void rotate_qk_kernel(const E* __restrict__ q,
                                                        const E* __restrict__ k, Layout lqk,
                                                        const float* __restrict__ cs,
                                                        const float* __restrict__ sn,
                                                        f16* __restrict__ out, int H, int T,
                                                        int bph, long long n, float qs) {
    constexpr int NC = D / 8;
    long long src, dst;
    int t, c;
    if constexpr (STRIDED) {
        const int bh = blockIdx.x / bph;
        const int i = (blockIdx.x - bh * bph) * 256 + threadIdx.x;
        if (i >= T * NC) return;
        t = i / NC;
        c = i % NC;
        src = lqk.head(bh, H) + (long long)t * lqk.st + 8 * c;
        dst = ((long long)bh * T + t) * D + 8 * c;
    } else {
        const int idx = blockIdx.x * blockDim.x + threadIdx.x;
        if ((long long)idx * 8 >= n) return;
        c = idx % NC;
        t = (idx / NC) % T;
        src = dst = (long long)idx * 8;
    }
    const u32x4 wq = *reinterpret_cast<const u32x4*>(q + src);
    const u32x4 wk = *reinterpret_cast<const u32x4*>(k + src);
    const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + t * (D / 2) + 4 * c);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + t * (D / 2) + 4 * c);
    const u32x4 rq = rope_chunk_f16<E>(wq, cv, sv, qs);
    const u32x4 rk = rope_chunk_f16<E>(wk, cv, sv, 1.f);
    *reinterpret_cast<u32x4*>(out + dst) = rq;
    *reinterpret_cast<u32x4*>(out + n + dst) = rk;
}

template <int D, typename E>
static hipError_t launch_rotate_d(const void* q, const void* k, Layout lqk, const float* cs,
                                  const float* sn, void* out, int B, int H, int T,
                                  hipStream_t st) {
    const long long n = (long long)B * H * T * D;
    const float qs = kLog2e / sqrtf((float)D);
    if (lqk.st != D) {  // rows not D apart: a strided layout (see Layout)
        const int bph = (T * (D / 8) + 255) / 256;
        const unsigned blocks = (unsigned)((long long)B * H * bph);
        hipLaunchKernelGGL((rotate_qk_kernel<D, E, true>), dim3(blocks), dim3(256), 0, st,
                           (const E*)q, (const E*)k, lqk, cs, sn, (f16*)out, H, T, bph, n, qs);
    } else {
        const unsigned blocks = (unsigned)((n / 8 + 255) / 256);
        hipLaunchKernelGGL((rotate_qk_kernel<D, E, false>), dim3(blocks), dim3(256), 0, st,
                           (const E*)q, (const E*)k, lqk, cs, sn, (f16*)out, H, T, 0, n, qs);
    }
    return hipGetLastError();
}

hipError_t launch_rotate_qk(const void* q, const void* k, Layout lqk, const float* cs,
                            const float* sn, void* out, int B, int H, int T, int D,
                            bool f16_storage, hipStream_t st) {
    if (f16_storage)
        return D == 64 ? launch_rotate_d<64, f16>(q, k, lqk, cs, sn, out, B, H, T, st)
                       : launch_rotate_d<128, f16>(q, k, lqk, cs, sn, out, B, H, T, st);
    return D == 64 ? launch_rotate_d<64, bf16>(q, k, lqk, cs, sn, out, B, H, T, st)
                   : launch_rotate_d<128, bf16>(q, k, lqk, cs, sn, out, B, H, T, st);
}

}  // namespace attn
