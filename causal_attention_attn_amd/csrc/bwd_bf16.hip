// Backward pass of causal RoPE attention, bf16 storage / fp32 accumulation, gfx950.
//
// The pages' engine computes every gradient by hand, RoPE's included, and checks
// them against centred differences ("Show HN: NanoEuler", paragraph 2). Here the
// backward recomputes the probabilities from q, k and the saved log-sum-exp
// instead of storing the T x T matrix, in two deterministic kernels (no atomics):
//
//   dq kernel   (one workgroup = 128 queries of a head; loops over key tiles
//                up to the diagonal): delta_t = sum_d dO[t,d] o[t,d] in its
//                prologue (written to the workspace), then
//                P = exp(S - lse), dP = dO V^T, dS = P (dP - delta),
//                dQ^r += s dS K^r, and finally dq = R_t^T dQ^r.
//   dkdv kernel (one workgroup = 128 keys of a head; loops over query tiles
//                from the diagonal down): with the same P and dS,
//                dV += P^T dO, dK^r += s dS^T Q^r, and finally dk = R_u^T dK^r.
//
// Every product is a 32x32x16 MFMA contraction with fp32 accumulation: the
// score recompute uses fp16 operands (rotated q and k, as in the forward), the
// others bf16 (dO, V, P, dS and bf16 copies of rotated q and k). In the dq kernel a
// lane column is a query (S^T, dP^T, dQ^T), in the dkdv kernel a lane column is
// a key (S, dP, dV^T, dK^T); the row operand is fed in key_perm order so that
// rounded P and dS are directly the B operand of the next contraction.
#include "device_common.h"
#include "launchers.h"

namespace attn {

template <int D>
struct BwdTile {
    static constexpr int NT = 256;
    static constexpr int DK = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int RS = D + 8;   // LDS row stride, row-major tiles
    // dq kernel
    static constexpr int QM = 128;     // queries per workgroup
    static constexpr int KN = 64;      // keys per LDS tile
    static constexpr int KTS = KN + 8; // LDS row stride, transposed key tile
    // dkdv kernel
    static constexpr int KM = 128;     // keys per workgroup
    static constexpr int QN = 64;      // queries per LDS tile
    static constexpr int QTS = QN + 8; // LDS row stride, transposed query tiles
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ cs, const float* __restrict__ sn, bf16* __restrict__ dq,
    float* __restrict__ delta, int BH, int T, int nqb, float sc, float scale) {
    using C = BwdTile<D>;
    __shared__ __attribute__((aligned(16))) f16 Ks[C::KN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Vs[C::KN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Kt[D * C::KTS];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::QM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;

    f16x8 qf[C::DK];
    bf16x8 df[C::DK];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const int d0 = 16 * c + 8 * hf;
        qf[c] = load_rope8<D, f16>(q + hoff, tq, d0, cs, sn, T);
        const u32x4 g = load_row8<D>(dO + hoff, tq, d0, T);
        const u32x4 y = load_row8<D>(o + hoff, tq, d0, T);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dot += bf16_lo(g[e]) * bf16_lo(y[e]) + bf16_hi(g[e]) * bf16_hi(y[e]);
        df[c] = as_bf16x8(g);
    }
    const float dl = dot + __shfl_xor(dot, 32);
    const float lt = tq < T ? lse[(size_t)bh * T + tq] * kLog2e : 0.f;
    if (tq < T && hf == 0) delta[(size_t)bh * T + tq] = dl;

    f32x16 acc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};

    const int kend = min(T, q0 + C::QM);
    const int ntiles = (kend + C::KN - 1) / C::KN;
    const int kp = key_perm(c32);

    for (int n = 0; n < ntiles; ++n) {
        const int k0 = n * C::KN;
        __syncthreads();
        stage_rows<D, C::KN, C::NT, true, f16, bf16>(k + hoff, k0, T, cs, sn, Ks, Kt, tid);
        stage_rows<D, C::KN, C::NT, false, bf16, void>(v + hoff, k0, T, cs, sn, Vs, nullptr, tid);
        __syncthreads();
        if (k0 > wq0) continue;

#pragma unroll
        for (int sb = 0; sb < C::KN / 32; ++sb) {
            const int kb = k0 + 32 * sb;
            if (kb > wq0) break;
            f32x16 s = f32x16{}, dp = f32x16{};
            const f16* krow = Ks + (32 * sb + kp) * C::RS + 8 * hf;
            const bf16* vrow = Vs + (32 * sb + kp) * C::RS + 8 * hf;
#pragma unroll
            for (int c = 0; c < C::DK; ++c) {
                s = mfma32(*reinterpret_cast<const f16x8*>(krow + 16 * c), qf[c], s);
                dp = mfma32(*reinterpret_cast<const bf16x8*>(vrow + 16 * c), df[c], dp);
            }
            const bool diag = (kb == wq0);
            bf16x8 dsb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float r[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int i = 8 * j + 2 * e + x;
                        float p = exp2_fast(fmaf(s[i], sc, -lt));
                        if (diag && item_row(i, hf) > c32) p = 0.f;
                        r[x] = p * (dp[i] - dl);
                    }
                    w[e] = pack_bf16x2(r[0], r[1]);
                }
                dsb[j] = as_bf16x8(w);
            }
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const bf16* trow = Kt + (32 * b + c32) * C::KTS + 32 * sb + 8 * hf;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[b] = mfma32(*reinterpret_cast<const bf16x8*>(trow + 16 * j), dsb[j], acc[b]);
            }
        }
    }

    if (tq < T) {
        bf16* out = dq + hoff + (size_t)tq * D;
        const float* crow = cs + (size_t)tq * (D / 2);
        const float* srow = sn + (size_t)tq * (D / 2);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * b + 8 * g + 4 * hf;
                u32x2 w;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const float x0 = acc[b][4 * g + 2 * pr] * scale;
                    const float x1 = acc[b][4 * g + 2 * pr + 1] * scale;
                    const float c = crow[d / 2 + pr], sv = srow[d / 2 + pr];
                    w[pr] = pack_bf16x2(x0 * c + x1 * sv, x1 * c - x0 * sv);
                }
                *reinterpret_cast<u32x2*>(out + d) = w;
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ cs,
    const float* __restrict__ sn, bf16* __restrict__ dk, bf16* __restrict__ dv, int BH, int T,
    int nkb, float sc, float scale) {
    using C = BwdTile<D>;
    __shared__ __attribute__((aligned(16))) f16 Qs[C::QN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Gs[C::QN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Qt[D * C::QTS];
    __shared__ __attribute__((aligned(16))) bf16 Gt[D * C::QTS];
    __shared__ __attribute__((aligned(16))) float Ls[C::QN];
    __shared__ __attribute__((aligned(16))) float Dl[C::QN];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int kb = bid / BH;  // key block 0 has the most query tiles: issued first
    const int k0 = kb * C::KM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const size_t roff = (size_t)bh * T;
    const int wk0 = k0 + wave * 32;
    const int tk = wk0 + c32;

    f16x8 kf[C::DK];
    bf16x8 vf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const int d0 = 16 * c + 8 * hf;
        kf[c] = load_rope8<D, f16>(k + hoff, tk, d0, cs, sn, T);
        vf[c] = as_bf16x8(load_row8<D>(v + hoff, tk, d0, T));
    }

    f32x16 dva[C::DB], dka[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dva[b] = dka[b] = f32x16{};

    const int qt0 = k0 / C::QN;
    const int nqt = (T + C::QN - 1) / C::QN;
    const int kp = key_perm(c32);

    for (int qt = qt0; qt < nqt; ++qt) {
        const int qbase = qt * C::QN;
        __syncthreads();
        stage_rows<D, C::QN, C::NT, true, f16, bf16>(q + hoff, qbase, T, cs, sn, Qs, Qt, tid);
        stage_rows<D, C::QN, C::NT, false, bf16, bf16>(dO + hoff, qbase, T, cs, sn, Gs, Gt, tid);
        if (tid < C::QN) {
            const int t = qbase + tid;
            Ls[tid] = t < T ? lse[roff + t] * kLog2e : INFINITY;
            Dl[tid] = t < T ? delta[roff + t] : 0.f;
        }
        __syncthreads();
        if (qbase + C::QN - 1 < wk0) continue;  // every query of the tile precedes this wave's keys

#pragma unroll
        for (int sb = 0; sb < C::QN / 32; ++sb) {
            const int qb = qbase + 32 * sb;
            if (qb + 31 < wk0) continue;
            f32x16 s = f32x16{}, dp = f32x16{};
            const f16* qrow = Qs + (32 * sb + kp) * C::RS + 8 * hf;
            const bf16* grow = Gs + (32 * sb + kp) * C::RS + 8 * hf;
#pragma unroll
            for (int c = 0; c < C::DK; ++c) {
                s = mfma32(*reinterpret_cast<const f16x8*>(qrow + 16 * c), kf[c], s);
                dp = mfma32(*reinterpret_cast<const bf16x8*>(grow + 16 * c), vf[c], dp);
            }
            const bool diag = (qb == wk0);
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(Ls + 32 * sb + 16 * j + 8 * hf);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(Ls + 32 * sb + 16 * j + 8 * hf + 4);
                const f32x4 e0 = *reinterpret_cast<const f32x4*>(Dl + 32 * sb + 16 * j + 8 * hf);
                const f32x4 e1 = *reinterpret_cast<const f32x4*>(Dl + 32 * sb + 16 * j + 8 * hf + 4);
                u32x4 wp, wd;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pr[2], dr[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int r = 2 * e + x;  // 0..7
                        const int i = 8 * j + r;
                        const float lr = r < 4 ? l0[r] : l1[r - 4];
                        const float er = r < 4 ? e0[r] : e1[r - 4];
                        float p = exp2_fast(fmaf(s[i], sc, -lr));
                        if (diag && item_row(i, hf) < c32) p = 0.f;
                        pr[x] = p;
                        dr[x] = p * (dp[i] - er);
                    }
                    wp[e] = pack_bf16x2(pr[0], pr[1]);
                    wd[e] = pack_bf16x2(dr[0], dr[1]);
                }
                pb[j] = as_bf16x8(wp);
                dsb[j] = as_bf16x8(wd);
            }
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const bf16* gtr = Gt + (32 * b + c32) * C::QTS + 32 * sb + 8 * hf;
                const bf16* qtr = Qt + (32 * b + c32) * C::QTS + 32 * sb + 8 * hf;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    dva[b] = mfma32(*reinterpret_cast<const bf16x8*>(gtr + 16 * j), pb[j], dva[b]);
                    dka[b] = mfma32(*reinterpret_cast<const bf16x8*>(qtr + 16 * j), dsb[j], dka[b]);
                }
            }
        }
    }

    if (tk < T) {
        bf16* ko = dk + hoff + (size_t)tk * D;
        bf16* vo = dv + hoff + (size_t)tk * D;
        const float* crow = cs + (size_t)tk * (D / 2);
        const float* srow = sn + (size_t)tk * (D / 2);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * b + 8 * g + 4 * hf;
                u32x2 wk, wv;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const float x0 = dka[b][4 * g + 2 * pr] * scale;
                    const float x1 = dka[b][4 * g + 2 * pr + 1] * scale;
                    const float c = crow[d / 2 + pr], sv = srow[d / 2 + pr];
                    wk[pr] = pack_bf16x2(x0 * c + x1 * sv, x1 * c - x0 * sv);
                    wv[pr] = pack_bf16x2(dva[b][4 * g + 2 * pr], dva[b][4 * g + 2 * pr + 1]);
                }
                *reinterpret_cast<u32x2*>(ko + d) = wk;
                *reinterpret_cast<u32x2*>(vo + d) = wv;
            }
        }
    }
}

template <int D>
static hipError_t launch_dq(const BwdArgs& a) {
    using C = BwdTile<D>;
    const int BH = a.B * a.H;
    const int nqb = (a.T + C::QM - 1) / C::QM;
    const float scale = 1.f / sqrtf((float)D);
    hipLaunchKernelGGL(bwd_dq_bf16_kernel<D>, dim3(nqb * BH), dim3(C::NT), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.o,
                       (const bf16*)a.dO, a.lse, a.cs, a.sn, (bf16*)a.dq, a.delta, BH, a.T, nqb,
                       scale * kLog2e, scale);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv(const BwdArgs& a) {
    using C = BwdTile<D>;
    const int BH = a.B * a.H;
    const int nkb = (a.T + C::KM - 1) / C::KM;
    const float scale = 1.f / sqrtf((float)D);
    hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<D>, dim3(nkb * BH), dim3(C::NT), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dO,
                       a.lse, a.delta, a.cs, a.sn, (bf16*)a.dk, (bf16*)a.dv, BH, a.T, nkb,
                       scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) {
    return a.D == 64 ? launch_dq<64>(a) : launch_dq<128>(a);
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a) {
    return a.D == 64 ? launch_dkdv<64>(a) : launch_dkdv<128>(a);
}

}  // namespace attn
