// The per-layer kernels next to attention, 16-bit storage (bf16 or fp16, type
// E) with fp32 arithmetic, gfx950: residual add + RMSNorm, and SwiGLU.
//
// The pages list RMSNorm and SwiGLU among the engine's hand-written CUDA kernels
// ("Show HN: NanoEuler", paragraph 2); each layer is causal attention plus a
// feed-forward network of two linear transforms with a Swish activation, both
// wrapped in residual connections ("Tiny Hackable CUDA", section 3). Readings:
//   h = x + r (the residual stream, stored as E), y = h * rstd * g,
//   rstd = 1 / sqrt(mean(h^2) + eps);  backward dh = rstd (g dy - h^ mean(h^ g dy))
//   + dres, dg = sum over rows of dy h^ (h^ = h rstd);
//   SwiGLU on the fused gate/up output u = [a | b]: out = silu(a) b,
//   da = dout b s (1 + a (1 - s)), db = dout silu(a), s = sigmoid(a).
//
// All of it is elementwise or a per-row reduction over C: bound by HBM. Rows
// are read with coalesced 8- or 16-byte loads, each row once (the RMSNorm row
// stays in registers between its two passes), and every output is written once.
#include "device_common.h"
#include "launchers.h"

namespace attn {

constexpr int kNormMaxChunks = 16;  // C <= 16 * 256 = 4096; kernels take NCH = C / 256

template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    const f32x2 lo = unpack2<E>(w[0]), hi = unpack2<E>(w[1]);
    return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <typename E>
__device__ __forceinline__ void store4(E* p, f32x4 v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2<E>(v[0], v[1]), pack2<E>(v[2], v[3])};
}

// Round each value to E and back (the stored residual stream is what the norm sees).
template <typename E>
__device__ __forceinline__ f32x4 round4(f32x4 v) {
    const f32x2 lo = unpack2<E>(pack2<E>(v[0], v[1])), hi = unpack2<E>(pack2<E>(v[2], v[3]));
    return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// One wave per row; lane l holds features 4l + 256j, j < NCH = C/256. RES: a
// residual r is added first (a template argument, not a null test: a runtime
// test splits every chunk's loads into branches, each ending in a wait for
// memory). Every load of a row is issued before the first is waited for.
template <typename E, int NCH, bool RES>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const E* __restrict__ x,
                                                          const E* __restrict__ r,
                                                          const E* __restrict__ g, float eps,
                                                          E* __restrict__ h, E* __restrict__ y,
                                                          float* __restrict__ rstd, int N, int C) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= N) return;
    const size_t base = (size_t)row * C + 4 * lane;
    f32x4 v[NCH], rv[NCH], gg[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        v[j] = load4(x + base + 256 * j);
        if constexpr (RES) rv[j] = load4(r + base + 256 * j);
        gg[j] = load4(g + 4 * lane + 256 * j);
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads before any arithmetic
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if constexpr (RES) v[j] = round4<E>(v[j] + rv[j]);
        ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
    }
    const float rs = 1.f / sqrtf(wave_sum(ss) / (float)C + eps);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (h != nullptr) store4(h + base + 256 * j, v[j]);
        store4(y + base + 256 * j, v[j] * rs * gg[j]);
    }
    if (lane == 0) rstd[row] = rs;
}

// Waves per workgroup of the RMSNorm backward: sixteen while a row's registers
// leave four waves per SIMD (rows of up to 768 features), else four. Fewer,
// larger workgroups leave fewer partial column sums for the dg reduction.
constexpr int norm_bwd_waves(int nch) { return nch <= 3 ? 16 : 4; }

// One wave per row, rows grid-strided; each workgroup leaves its column sums of
// dy * h^ in part[blockIdx.x][C] (fp32) for the dg reduction. RES: the residual
// stream's own gradient dres is added to dh (a template argument for the reason
// given at the forward kernel).
template <typename E, int NCH, bool RES>
__global__ __launch_bounds__(64 * norm_bwd_waves(NCH)) void rmsnorm_bwd_kernel(
    const E* __restrict__ h, const E* __restrict__ g, const float* __restrict__ rstd,
    const E* __restrict__ dy, const E* __restrict__ dres, E* __restrict__ dh,
    float* __restrict__ part, int N, int C) {
    constexpr int NW = norm_bwd_waves(NCH);
    constexpr int KPR = 16 / NW;  // chunks per LDS round (16 KB)
    __shared__ f32x4 red[NW][64][KPR];  // per wave: its lanes' column sums, KPR chunks at a time
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 gg[NCH], acc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        acc[j] = zero;
        gg[j] = load4(g + 4 * lane + 256 * j);
    }
    // RP rows per pass (two while they fit in registers), all of their loads
    // issued before any arithmetic
    constexpr int RP = NCH <= 8 ? 2 : 1;
    const int stride = gridDim.x * NW;
    for (int row0 = blockIdx.x * NW + wave; row0 < N; row0 += RP * stride) {
        f32x4 hv[RP][NCH], dv[RP][NCH], rv[RP][NCH];
        float rs[RP];
#pragma unroll
        for (int q = 0; q < RP; ++q) {
            // a row past N loads row N-1 instead (never used): the loads of all
            // RP rows then issue without a branch, and so without a wait, between
            const int row = min(row0 + q * stride, N - 1);
            const size_t base = (size_t)row * C + 4 * lane;
            rs[q] = rstd[row];
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                hv[q][j] = load4(h + base + 256 * j);
                dv[q][j] = load4(dy + base + 256 * j);
                rv[q][j] = RES ? load4(dres + base + 256 * j) : zero;
            }
        }
        if constexpr (NCH <= 4) {
            // all loads of the pass before any arithmetic (for wider rows holding
            // them all at once costs more registers than it saves waiting)
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (RES) {
                // a row's dres feeds only its conditional store; this empty use
                // keeps the compiler from sinking those loads behind the earlier
                // rows' work
#pragma unroll
                for (int q = 0; q < RP; ++q)
#pragma unroll
                    for (int j = 0; j < NCH; ++j) asm volatile("" ::"v"(rv[q][j]));
            }
        }
#pragma unroll
        for (int q = 0; q < RP; ++q) {
            const int row = row0 + q * stride;
            // a row past N (uniform) is computed with rstd 0, which keeps it out
            // of the column sums, and not stored; no branch before the
            // arithmetic, or the compiler sinks this row's loads behind it
            const bool live = row < N;
            const float rq = live ? rs[q] : 0.f;
            const size_t base = (size_t)row * C + 4 * lane;
            f32x4 hh[NCH], gd[NCH];
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                hh[j] = hv[q][j] * rq;
                gd[j] = gg[j] * dv[q][j];
                acc[j] += dv[q][j] * hh[j];
                const f32x4 p = hh[j] * gd[j];
                dot += p[0] + p[1] + p[2] + p[3];
            }
            const float mean = wave_sum(dot) / (float)C;
            if (live) {
#pragma unroll
                for (int j = 0; j < NCH; ++j)
                    store4(dh + base + 256 * j, (gd[j] - hh[j] * mean) * rq + rv[q][j]);
            }
        }
    }
    // the workgroup's column sums: its waves added through LDS in a fixed order,
    // KPR chunks at a time
#pragma unroll
    for (int j0 = 0; j0 < NCH; j0 += KPR) {
#pragma unroll
        for (int k = 0; k < KPR; ++k) red[wave][lane][k] = j0 + k < NCH ? acc[j0 + k] : zero;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int k = 0; k < KPR; ++k) {
                if (j0 + k < NCH) {
                    f32x4 s = red[0][lane][k];
#pragma unroll
                    for (int w = 1; w < NW; ++w) s += red[w][lane][k];
                    *reinterpret_cast<f32x4*>(part + (size_t)blockIdx.x * C + 4 * lane +
                                              256 * (j0 + k)) = s;
                }
            }
        }
        __syncthreads();
    }
}

// dg[c] = sum over the workgroups' partial column sums. A block of 1024 threads
// takes 64 columns; thread (k, c) adds partials k, k + 16, ... of its column with
// 16 loads in flight at a time (a load per iteration would pay the memory latency
// nparts times), then the 16 groups are added in a fixed order: deterministic.
__global__ __launch_bounds__(1024) void rmsnorm_dg_kernel(const float* __restrict__ part,
                                                          float* __restrict__ dg, int nparts,
                                                          int C) {
    __shared__ float red[16][64];
    const int cx = threadIdx.x & 63, k0 = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + cx;  // C is a multiple of 256: always < C
    float s = 0.f;
    for (int i0 = k0; i0 < nparts; i0 += 16 * 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = i0 + 16 * j;
            v[j] = i < nparts ? part[(size_t)i * C + c] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) s += v[j];
    }
    red[k0][cx] = s;
    __syncthreads();
    if (k0 == 0) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) t += red[j][cx];
        dg[c] = t;
    }
}

__device__ __forceinline__ float sigmoid_f(float a) { return 1.f / (1.f + __expf(-a)); }

// One thread per 8 consecutive outputs of a row.
template <typename E, bool BACKWARD>
__global__ __launch_bounds__(256) void swiglu_kernel(const E* __restrict__ u,
                                                     const E* __restrict__ dout,
                                                     E* __restrict__ out, long long n8, int F) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const int f8 = F >> 3;
    const long long row = i / f8;
    const int col = (int)(i - row * f8) * 8;
    const E* ur = u + row * 2 * F;
    const u32x4 wa = *reinterpret_cast<const u32x4*>(ur + col);
    const u32x4 wb = *reinterpret_cast<const u32x4*>(ur + F + col);
    if constexpr (!BACKWARD) {
        u32x4 w;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f32x2 a = unpack2<E>(wa[p]), b = unpack2<E>(wb[p]);
            w[p] = pack2<E>(a[0] * sigmoid_f(a[0]) * b[0], a[1] * sigmoid_f(a[1]) * b[1]);
        }
        *reinterpret_cast<u32x4*>(out + row * F + col) = w;
    } else {
        const u32x4 wd = *reinterpret_cast<const u32x4*>(dout + row * F + col);
        u32x4 da, db;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f32x2 a = unpack2<E>(wa[p]), b = unpack2<E>(wb[p]), d = unpack2<E>(wd[p]);
            float ga[2], gb[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float s = sigmoid_f(a[e]);
                ga[e] = d[e] * b[e] * s * (1.f + a[e] * (1.f - s));
                gb[e] = d[e] * a[e] * s;
            }
            da[p] = pack2<E>(ga[0], ga[1]);
            db[p] = pack2<E>(gb[0], gb[1]);
        }
        E* gr = out + row * 2 * F;
        *reinterpret_cast<u32x4*>(gr + col) = da;
        *reinterpret_cast<u32x4*>(gr + F + col) = db;
    }
}

// Explicit instantiations: the host pass does not always emit the launch stub of
// a kernel template with a 16-bit element-type argument on its own.
#define ATTN_NORM_INST_R(E_, K_, R_)                                                            \
    template __global__ void rmsnorm_fwd_kernel<E_, K_, R_>(const E_*, const E_*, const E_*,    \
                                                            float, E_*, E_*, float*, int, int);  \
    template __global__ void rmsnorm_bwd_kernel<E_, K_, R_>(const E_*, const E_*, const float*, \
                                                            const E_*, const E_*, E_*, float*,   \
                                                            int, int);
#define ATTN_NORM_INST(E_, K_) ATTN_NORM_INST_R(E_, K_, false) ATTN_NORM_INST_R(E_, K_, true)
#define ATTN_NORM_INST_ALL(E_)                                                                  \
    ATTN_NORM_INST(E_, 1) ATTN_NORM_INST(E_, 2) ATTN_NORM_INST(E_, 3) ATTN_NORM_INST(E_, 4)     \
    ATTN_NORM_INST(E_, 5) ATTN_NORM_INST(E_, 6) ATTN_NORM_INST(E_, 7) ATTN_NORM_INST(E_, 8)     \
    ATTN_NORM_INST(E_, 9) ATTN_NORM_INST(E_, 10) ATTN_NORM_INST(E_, 11) ATTN_NORM_INST(E_, 12)  \
    ATTN_NORM_INST(E_, 13) ATTN_NORM_INST(E_, 14) ATTN_NORM_INST(E_, 15) ATTN_NORM_INST(E_, 16)
ATTN_NORM_INST_ALL(bf16) ATTN_NORM_INST_ALL(f16)
#undef ATTN_NORM_INST_ALL
#undef ATTN_NORM_INST
#undef ATTN_NORM_INST_R
template __global__ void swiglu_kernel<bf16, false>(const bf16*, const bf16*, bf16*, long long, int);
template __global__ void swiglu_kernel<bf16, true>(const bf16*, const bf16*, bf16*, long long, int);
template __global__ void swiglu_kernel<f16, false>(const f16*, const f16*, f16*, long long, int);
template __global__ void swiglu_kernel<f16, true>(const f16*, const f16*, f16*, long long, int);

// Calls f(std::integral_constant<int, nch>{}) for nch in 1 .. kNormMaxChunks.
template <int K = 1, typename F>
static hipError_t with_chunks(int nch, F&& f) {
    if constexpr (K > kNormMaxChunks) {
        return hipErrorInvalidValue;
    } else {
        if (nch == K) return f(std::integral_constant<int, K>{});
        return with_chunks<K + 1>(nch, f);
    }
}

// 4096 waves at most (all resident), one row per wave and pass
int rmsnorm_bwd_parts(int N, int C) {
    const int nw = norm_bwd_waves(C >> 8);
    const int wgs = (N + nw - 1) / nw, cap = 4096 / nw;
    return wgs < cap ? wgs : cap;
}

template <typename E>
static hipError_t rmsnorm_fwd_t(const void* x, const void* r, const void* g, float eps, void* h,
                                void* y, float* rstd, int N, int C, hipStream_t st) {
    return with_chunks(C >> 8, [&](auto K) {
        constexpr int NCH = decltype(K)::value;
        const dim3 grid((unsigned)((N + 3) / 4));
        if (r != nullptr)
            hipLaunchKernelGGL((rmsnorm_fwd_kernel<E, NCH, true>), grid, dim3(256), 0, st,
                               (const E*)x, (const E*)r, (const E*)g, eps, (E*)h, (E*)y, rstd, N,
                               C);
        else
            hipLaunchKernelGGL((rmsnorm_fwd_kernel<E, NCH, false>), grid, dim3(256), 0, st,
                               (const E*)x, (const E*)r, (const E*)g, eps, (E*)h, (E*)y, rstd, N,
                               C);
        return hipGetLastError();
    });
}

hipError_t launch_rmsnorm_fwd(const void* x, const void* r, const void* g, float eps, void* h,
                              void* y, float* rstd, int N, int C, bool f16_storage,
                              hipStream_t st) {
    return f16_storage ? rmsnorm_fwd_t<f16>(x, r, g, eps, h, y, rstd, N, C, st)
                       : rmsnorm_fwd_t<bf16>(x, r, g, eps, h, y, rstd, N, C, st);
}

template <typename E>
static hipError_t rmsnorm_bwd_t(const void* h, const void* g, const float* rstd, const void* dy,
                                const void* dres, void* dh, float* dg, float* part, int N,
                                int C, hipStream_t st) {
    const int parts = rmsnorm_bwd_parts(N, C);
    hipError_t e = with_chunks(C >> 8, [&](auto K) {
        constexpr int NCH = decltype(K)::value;
        const dim3 grid((unsigned)parts), block(64 * norm_bwd_waves(NCH));
        if (dres != nullptr)
            hipLaunchKernelGGL((rmsnorm_bwd_kernel<E, NCH, true>), grid, block, 0, st,
                               (const E*)h, (const E*)g, rstd, (const E*)dy, (const E*)dres,
                               (E*)dh, part, N, C);
        else
            hipLaunchKernelGGL((rmsnorm_bwd_kernel<E, NCH, false>), grid, block, 0, st,
                               (const E*)h, (const E*)g, rstd, (const E*)dy, (const E*)dres,
                               (E*)dh, part, N, C);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rmsnorm_dg_kernel, dim3((unsigned)(C / 64)), dim3(1024), 0, st, part, dg,
                       parts, C);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const void* h, const void* g, const float* rstd, const void* dy,
                              const void* dres, void* dh, float* dg, float* part, int N, int C,
                              bool f16_storage, hipStream_t st) {
    return f16_storage ? rmsnorm_bwd_t<f16>(h, g, rstd, dy, dres, dh, dg, part, N, C, st)
                       : rmsnorm_bwd_t<bf16>(h, g, rstd, dy, dres, dh, dg, part, N, C, st);
}

template <typename E>
static hipError_t swiglu_t(const void* u, const void* dout, void* out, int N, int F,
                           bool backward, hipStream_t st) {
    const long long n8 = (long long)N * (F / 8);
    const unsigned blocks = (unsigned)((n8 + 255) / 256);
    if (backward)
        hipLaunchKernelGGL((swiglu_kernel<E, true>), dim3(blocks), dim3(256), 0, st, (const E*)u,
                           (const E*)dout, (E*)out, n8, F);
    else
        hipLaunchKernelGGL((swiglu_kernel<E, false>), dim3(blocks), dim3(256), 0, st,
                           (const E*)u, (const E*)nullptr, (E*)out, n8, F);
    return hipGetLastError();
}

hipError_t launch_swiglu(const void* u, const void* dout, void* out, int N, int F, bool backward,
                         bool f16_storage, hipStream_t st) {
    return f16_storage ? swiglu_t<f16>(u, dout, out, N, F, backward, st)
                       : swiglu_t<bf16>(u, dout, out, N, F, backward, st);
}

}  // namespace attn
