// fp32 path of causal RoPE attention (forward, dq and dk/dv), gfx950.
//
// Same method as the bf16 kernels - RoPE applied on load, FlashAttention-style
// online softmax over LDS key tiles with causal tile skipping, and a
// recompute-based backward split into a dq kernel and a dk/dv kernel, both
// reading delta_t = sum_d dO o from the pre-pass - but evaluated with fp32 VALU
// arithmetic throughout, so that no value is ever rounded to a 16-bit type.
// This path serves fp32 callers and small shapes; it is not tuned for speed.
//
// Thread mapping: D/32 adjacent lanes share one row (query or key), each lane
// owning 32 consecutive features; dot products are completed with lane
// exchanges inside that group.
#include "device_common.h"
#include "launchers.h"

namespace attn {

template <int D>
struct F32Tile {
    static constexpr int NT = 256;
    static constexpr int LPR = D / 32;      // lanes per row
    static constexpr int ROWS = NT / LPR;   // rows per workgroup
    static constexpr int BN = 32;           // rows per LDS tile
};

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    if (LPR >= 2) x += __shfl_xor(x, 1);
    if (LPR >= 4) x += __shfl_xor(x, 2);
    return x;
}

// 32 consecutive features (d0 .. d0+31) of row t, rotated by R_t if ROT; zero rows past T.
template <int D, bool ROT>
__device__ __forceinline__ void load32(const float* __restrict__ x, int t, int d0, int T,
                                       const float* __restrict__ cs,
                                       const float* __restrict__ sn, float* out) {
    if (t >= T) {
#pragma unroll
        for (int i = 0; i < 32; ++i) out[i] = 0.f;
        return;
    }
    const float* row = x + (size_t)t * D + d0;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(row + i);
        out[i] = w[0]; out[i + 1] = w[1]; out[i + 2] = w[2]; out[i + 3] = w[3];
    }
    if (ROT) {
        const float* c = cs + (size_t)t * (D / 2) + d0 / 2;
        const float* s = sn + (size_t)t * (D / 2) + d0 / 2;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const float x0 = out[2 * p], x1 = out[2 * p + 1];
            out[2 * p] = x0 * c[p] - x1 * s[p];
            out[2 * p + 1] = x0 * s[p] + x1 * c[p];
        }
    }
}

// Stage rows [r0, r0 + BN) of a [T, D] head into LDS tile[BN][D] (rotated if ROT).
template <int D, int BN, int NT, bool ROT>
__device__ __forceinline__ void stage_f32(const float* __restrict__ x, int r0, int T,
                                          const float* __restrict__ cs,
                                          const float* __restrict__ sn, float* tile, int tid) {
    constexpr int UNITS = BN * D / 2;  // one feature pair per unit
    for (int u = tid; u < UNITS; u += NT) {
        const int r = u / (D / 2), p = u % (D / 2);
        const int t = r0 + r;
        float y0 = 0.f, y1 = 0.f;
        if (t < T) {
            const float x0 = x[(size_t)t * D + 2 * p], x1 = x[(size_t)t * D + 2 * p + 1];
            if (ROT) {
                const float c = cs[(size_t)t * (D / 2) + p], s = sn[(size_t)t * (D / 2) + p];
                y0 = x0 * c - x1 * s;
                y1 = x0 * s + x1 * c;
            } else {
                y0 = x0;
                y1 = x1;
            }
        }
        tile[r * D + 2 * p] = y0;
        tile[r * D + 2 * p + 1] = y1;
    }
}

template <int D>
__device__ __forceinline__ float dot32(const float* a, const float* tile_row) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(tile_row + i);
        acc = fmaf(a[i], w[0], acc);
        acc = fmaf(a[i + 1], w[1], acc);
        acc = fmaf(a[i + 2], w[2], acc);
        acc = fmaf(a[i + 3], w[3], acc);
    }
    return acc;
}

// Store 32 features; when UNROT, first apply R_t^T (rotation by -t*theta).
template <int D, bool UNROT>
__device__ __forceinline__ void store32(float* __restrict__ x, int t, int d0,
                                        const float* __restrict__ cs,
                                        const float* __restrict__ sn, const float* val) {
    float* row = x + (size_t)t * D + d0;
    float out[32];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        if (UNROT) {
            const float c = cs[(size_t)t * (D / 2) + d0 / 2 + p];
            const float s = sn[(size_t)t * (D / 2) + d0 / 2 + p];
            out[2 * p] = val[2 * p] * c + val[2 * p + 1] * s;
            out[2 * p + 1] = val[2 * p + 1] * c - val[2 * p] * s;
        } else {
            out[2 * p] = val[2 * p];
            out[2 * p + 1] = val[2 * p + 1];
        }
    }
#pragma unroll
    for (int i = 0; i < 32; i += 4)
        *reinterpret_cast<f32x4*>(row + i) = f32x4{out[i], out[i + 1], out[i + 2], out[i + 3]};
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ cs, const float* __restrict__ sn, float* __restrict__ o,
    float* __restrict__ lse, int BH, int T, int nqb, float sc) {
    using C = F32Tile<D>;
    __shared__ __attribute__((aligned(16))) float Ks[C::BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[C::BN * D];
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::ROWS;
    const int tid = threadIdx.x;
    const int t = q0 + tid / C::LPR, d0 = 32 * (tid % C::LPR);
    const size_t hoff = (size_t)bh * T * D;

    float qr[32], acc[32];
    load32<D, true>(q + hoff, t, d0, T, cs, sn, qr);
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int kend = min(T, q0 + C::ROWS);
    for (int k0 = 0; k0 < kend; k0 += C::BN) {
        __syncthreads();
        stage_f32<D, C::BN, C::NT, true>(k + hoff, k0, T, cs, sn, Ks, tid);
        stage_f32<D, C::BN, C::NT, false>(v + hoff, k0, T, cs, sn, Vs, tid);
        __syncthreads();
        float s[C::BN];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < C::BN; ++j) {
            const float x = row_sum<C::LPR>(dot32<D>(qr, Ks + j * D + d0)) * sc;
            s[j] = (k0 + j <= t) ? x : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float mnew = fmaxf(m, mx);
        if (mnew == -INFINITY) continue;  // row sees no key in this tile yet
        const float alpha = exp2_fast(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
        for (int j = 0; j < C::BN; ++j) {
            const float p = exp2_fast(s[j] - mnew);
            l += p;
            const float* vr = Vs + j * D + d0;
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] = fmaf(p, vr[i], acc[i]);
        }
    }
    if (t < T) {
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= inv;
        store32<D, false>(o + hoff, t, d0, cs, sn, acc);
        if (d0 == 0) lse[(size_t)bh * T + t] = (m + log2f(l)) * kLn2;
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ cs, const float* __restrict__ sn, float* __restrict__ dq,
    const float* __restrict__ delta, int BH, int T, int nqb, float sc, float scale) {
    using C = F32Tile<D>;
    __shared__ __attribute__((aligned(16))) float Ks[C::BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[C::BN * D];
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::ROWS;
    const int tid = threadIdx.x;
    const int t = q0 + tid / C::LPR, d0 = 32 * (tid % C::LPR);
    const size_t hoff = (size_t)bh * T * D;

    float qr[32], g[32], acc[32];
    load32<D, true>(q + hoff, t, d0, T, cs, sn, qr);
    load32<D, false>(dO + hoff, t, d0, T, cs, sn, g);
    const float dl = t < T ? delta[(size_t)bh * T + t] : 0.f;  // from the pre-pass
    const float lt = t < T ? lse[(size_t)bh * T + t] * kLog2e : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;

    const int kend = min(T, q0 + C::ROWS);
    for (int k0 = 0; k0 < kend; k0 += C::BN) {
        __syncthreads();
        stage_f32<D, C::BN, C::NT, true>(k + hoff, k0, T, cs, sn, Ks, tid);
        stage_f32<D, C::BN, C::NT, false>(v + hoff, k0, T, cs, sn, Vs, tid);
        __syncthreads();
#pragma unroll 4
        for (int j = 0; j < C::BN; ++j) {
            const float x = row_sum<C::LPR>(dot32<D>(qr, Ks + j * D + d0));
            const float dp = row_sum<C::LPR>(dot32<D>(g, Vs + j * D + d0));
            const float p = (k0 + j <= t) ? exp2_fast(fmaf(x, sc, -lt)) : 0.f;
            const float ds = p * (dp - dl);
            const float* kr = Ks + j * D + d0;
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] = fmaf(ds, kr[i], acc[i]);
        }
    }
    if (t < T) {
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= scale;
        store32<D, true>(dq + hoff, t, d0, cs, sn, acc);
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ cs,
    const float* __restrict__ sn, float* __restrict__ dk, float* __restrict__ dv, int BH,
    int T, int nkb, float sc, float scale) {
    using C = F32Tile<D>;
    __shared__ __attribute__((aligned(16))) float Qs[C::BN * D];
    __shared__ __attribute__((aligned(16))) float Gs[C::BN * D];
    __shared__ float Ls[C::BN], Dl[C::BN];
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int kb = bid / BH;
    const int k0 = kb * C::ROWS;
    const int tid = threadIdx.x;
    const int u = k0 + tid / C::LPR, d0 = 32 * (tid % C::LPR);
    const size_t hoff = (size_t)bh * T * D;
    const size_t roff = (size_t)bh * T;

    float kr[32], vv[32], gk[32], gv[32];
    load32<D, true>(k + hoff, u, d0, T, cs, sn, kr);
    load32<D, false>(v + hoff, u, d0, T, cs, sn, vv);
#pragma unroll
    for (int i = 0; i < 32; ++i) gk[i] = gv[i] = 0.f;

    for (int qb0 = (k0 / C::BN) * C::BN; qb0 < T; qb0 += C::BN) {
        __syncthreads();
        stage_f32<D, C::BN, C::NT, true>(q + hoff, qb0, T, cs, sn, Qs, tid);
        stage_f32<D, C::BN, C::NT, false>(dO + hoff, qb0, T, cs, sn, Gs, tid);
        if (tid < C::BN) {
            const int t = qb0 + tid;
            Ls[tid] = t < T ? lse[roff + t] * kLog2e : INFINITY;
            Dl[tid] = t < T ? delta[roff + t] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int j = 0; j < C::BN; ++j) {
            const float x = row_sum<C::LPR>(dot32<D>(kr, Qs + j * D + d0));
            const float dp = row_sum<C::LPR>(dot32<D>(vv, Gs + j * D + d0));
            const float p = (qb0 + j >= u) ? exp2_fast(fmaf(x, sc, -Ls[j])) : 0.f;
            const float ds = p * (dp - Dl[j]);
            const float* qr = Qs + j * D + d0;
            const float* gr = Gs + j * D + d0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                gv[i] = fmaf(p, gr[i], gv[i]);
                gk[i] = fmaf(ds, qr[i], gk[i]);
            }
        }
    }
    if (u < T) {
#pragma unroll
        for (int i = 0; i < 32; ++i) gk[i] *= scale;
        store32<D, true>(dk + hoff, u, d0, cs, sn, gk);
        store32<D, false>(dv + hoff, u, d0, cs, sn, gv);
    }
}

template <int D>
static hipError_t launch_fwd32(const FwdArgs& a) {
    using C = F32Tile<D>;
    const int BH = a.B * a.H;
    const int nqb = (a.T + C::ROWS - 1) / C::ROWS;
    hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3(nqb * BH), dim3(C::NT), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, a.cs, a.sn,
                       (float*)a.o, a.lse, BH, a.T, nqb, kLog2e / sqrtf((float)D));
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dq32(const BwdArgs& a) {
    using C = F32Tile<D>;
    const int BH = a.B * a.H;
    const int nqb = (a.T + C::ROWS - 1) / C::ROWS;
    const float scale = 1.f / sqrtf((float)D);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3(nqb * BH), dim3(C::NT), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dO, a.lse, a.cs, a.sn, (float*)a.dq,
                       a.ws, BH, a.T, nqb, scale * kLog2e, scale);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv32(const BwdArgs& a) {
    using C = F32Tile<D>;
    const int BH = a.B * a.H;
    const int nkb = (a.T + C::ROWS - 1) / C::ROWS;
    const float scale = 1.f / sqrtf((float)D);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3(nkb * BH), dim3(C::NT), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dO, a.lse, a.ws, a.cs, a.sn, (float*)a.dk,
                       (float*)a.dv, BH, a.T, nkb, scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
    return a.D == 64 ? launch_fwd32<64>(a) : launch_fwd32<128>(a);
}
hipError_t launch_bwd_dq_f32(const BwdArgs& a) {
    return a.D == 64 ? launch_dq32<64>(a) : launch_dq32<128>(a);
}
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a) {
    return a.D == 64 ? launch_dkdv32<64>(a) : launch_dkdv32<128>(a);
}

}  // namespace attn
