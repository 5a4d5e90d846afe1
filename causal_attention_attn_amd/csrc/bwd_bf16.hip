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
// a key (S, dP, dV^T, dK^T). Transposed LDS tiles store their columns in
// col_perm order, so rounded P and dS are directly the B operand of the next
// contraction and every A operand is one 16-byte LDS read.
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
    // D = 64: two LDS buffers, the next tile's global loads issued before the
    // current tile's math. D = 128: one buffer and no register prefetch (the
    // staging registers would push the kernels past 256 VGPRs and two buffers
    // would leave room for one workgroup per CU).
    static constexpr int NBUF = D == 64 ? 2 : 1;
};

// One 64-key tile of the dq kernel for one wave (32 queries). DIAG: the tile may
// reach this wave's diagonal (32-key blocks above it skipped, the diagonal one masked).
template <int D, bool DIAG>
__device__ __forceinline__ void dq_tile(f32x16* acc, const f16x8* qf, const bf16x8* df,
                                        const f16* ks, const bf16* vs, const bf16* kt, int k0,
                                        int wq0, int c32, int hf, float sc, float nlt,
                                        float dl) {
    using C = BwdTile<D>;
#pragma unroll
    for (int sb = 0; sb < C::KN / 32; ++sb) {
        const int kb = k0 + 32 * sb;
        if (DIAG && kb > wq0) break;
        const f16* krow = ks + (32 * sb + c32) * C::RS + 8 * hf;
        const bf16* vrow = vs + (32 * sb + c32) * C::RS + 8 * hf;
        f32x16 s = mfma32(*reinterpret_cast<const f16x8*>(krow), qf[0], f32x16{});
        f32x16 dp = mfma32(*reinterpret_cast<const bf16x8*>(vrow), df[0], f32x16{});
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            s = mfma32(*reinterpret_cast<const f16x8*>(krow + 16 * c), qf[c], s);
            dp = mfma32(*reinterpret_cast<const bf16x8*>(vrow + 16 * c), df[c], dp);
        }
        if (DIAG && kb == wq0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) > c32) s[i] = -INFINITY;
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * j + 2 * e;
                const float p0 = exp2_fast(fmaf(s[i], sc, nlt));
                const float p1 = exp2_fast(fmaf(s[i + 1], sc, nlt));
                w[e] = pack_bf16x2(p0 * (dp[i] - dl), p1 * (dp[i + 1] - dl));
            }
            dsb[j] = as_bf16x8(w);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
            const bf16* trow = kt + (32 * b + c32) * C::KTS + 32 * sb + 8 * hf;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[b] = mfma32(*reinterpret_cast<const bf16x8*>(trow + 16 * j), dsb[j], acc[b]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dq_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ cs, const float* __restrict__ sn, bf16* __restrict__ dq,
    float* __restrict__ delta, int BH, int T, int nqb, float sc, float scale) {
    using C = BwdTile<D>;
    constexpr int NB = C::NBUF;
    __shared__ __attribute__((aligned(16))) f16 Ks[NB][C::KN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Vs[NB][C::KN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Kt[NB][D * C::KTS];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::QM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const HeadBufs<D> qh(q + hoff, cs, sn, T), kh(k + hoff, cs, sn, T), vh(v + hoff, cs, sn, T);
    const rsrc_t gr = make_rsrc(dO + hoff, (uint32_t)T * D * 2);
    const rsrc_t orr = make_rsrc(o + hoff, (uint32_t)T * D * 2);
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;

    const int kend = min(T, q0 + C::QM);
    const int ntiles = (kend + C::KN - 1) / C::KN;
    const int nfull = min(ntiles, q0 / C::KN);
    RowStage<D, C::KN, C::NT, true> kst;
    RowStage<D, C::KN, C::NT, false> vst;
    kst.load(kh, 0, tid);
    vst.load(vh, 0, tid);

    // this lane's query: rotated q (fp16), dO (bf16), and delta = sum_d dO o
    f16x8 qf[C::DK];
    bf16x8 df[C::DK];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const int d0 = 16 * c + 8 * hf;
        qf[c] = rope_operand<D, f16>(qh, tq, d0);
        const u32x4 g = buf_load16(gr, (uint32_t)(tq * D + d0) * 2);
        const u32x4 y = buf_load16(orr, (uint32_t)(tq * D + d0) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dot += bf16_lo(g[e]) * bf16_lo(y[e]) + bf16_hi(g[e]) * bf16_hi(y[e]);
        df[c] = as_bf16x8(g);
    }
    const float dl = sum_across_halves(dot);
    const float nlt = tq < T ? -lse[(size_t)bh * T + tq] * kLog2e : 0.f;
    if (tq < T && hf == 0) delta[(size_t)bh * T + tq] = dl;

    f32x16 acc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};

    kst.template store<f16, bf16>(Ks[0], Kt[0], tid);
    vst.template store<bf16, void>(Vs[0], nullptr, tid);
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
        const int k0 = n * C::KN;
        const int cur = n % NB;
        const bool more = n + 1 < ntiles;
        if (NB == 2 && more) {
            kst.load(kh, k0 + C::KN, tid);
            vst.load(vh, k0 + C::KN, tid);
        }
        if (n < nfull)
            dq_tile<D, false>(acc, qf, df, Ks[cur], Vs[cur], Kt[cur], k0, wq0, c32, hf, sc, nlt, dl);
        else if (k0 <= wq0)
            dq_tile<D, true>(acc, qf, df, Ks[cur], Vs[cur], Kt[cur], k0, wq0, c32, hf, sc, nlt, dl);
        if (more) {
            if (NB == 1) {  // no prefetch: wait for every wave, then load and store
                __syncthreads();
                kst.load(kh, k0 + C::KN, tid);
                vst.load(vh, k0 + C::KN, tid);
            }
            kst.template store<f16, bf16>(Ks[(n + 1) % NB], Kt[(n + 1) % NB], tid);
            vst.template store<bf16, void>(Vs[(n + 1) % NB], nullptr, tid);
        }
        __syncthreads();
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
                const f32x2 c2 = *reinterpret_cast<const f32x2*>(crow + d / 2);
                const f32x2 s2 = *reinterpret_cast<const f32x2*>(srow + d / 2);
                u32x2 w;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const float x0 = acc[b][4 * g + 2 * pr] * scale;
                    const float x1 = acc[b][4 * g + 2 * pr + 1] * scale;
                    w[pr] = pack_bf16x2(x0 * c2[pr] + x1 * s2[pr], x1 * c2[pr] - x0 * s2[pr]);
                }
                *reinterpret_cast<u32x2*>(out + d) = w;
            }
        }
    }
}

// One 64-query tile of the dk/dv kernel for one wave (32 keys). DIAG: the tile
// may reach this wave's diagonal (32-query blocks wholly before the wave's
// first key skipped, the diagonal one masked).
template <int D, bool DIAG>
__device__ __forceinline__ void dkdv_tile(f32x16* dva, f32x16* dka, const f16x8* kf,
                                          const bf16x8* vf, const f16* qs, const bf16* gs,
                                          const bf16* qt, const bf16* gt, const float* ls,
                                          const float* dls, int qbase, int wk0, int c32, int hf,
                                          float sc) {
    using C = BwdTile<D>;
#pragma unroll
    for (int sb = 0; sb < C::QN / 32; ++sb) {
        const int qb = qbase + 32 * sb;
        if (DIAG && qb + 31 < wk0) continue;
        const f16* qrow = qs + (32 * sb + c32) * C::RS + 8 * hf;
        const bf16* grow = gs + (32 * sb + c32) * C::RS + 8 * hf;
        f32x16 s = mfma32(*reinterpret_cast<const f16x8*>(qrow), kf[0], f32x16{});
        f32x16 dp = mfma32(*reinterpret_cast<const bf16x8*>(grow), vf[0], f32x16{});
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            s = mfma32(*reinterpret_cast<const f16x8*>(qrow + 16 * c), kf[c], s);
            dp = mfma32(*reinterpret_cast<const bf16x8*>(grow + 16 * c), vf[c], dp);
        }
        if (DIAG && qb == wk0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) < c32) s[i] = -INFINITY;
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 wp, wd;
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
                // items 8j + 4*g2 .. +3 belong to queries 16j + 8*g2 + 4*hf .. +3
                const int qo = 32 * sb + 16 * j + 8 * g2 + 4 * hf;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qo);
                const f32x4 e4 = *reinterpret_cast<const f32x4*>(dls + qo);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int i = 8 * j + 4 * g2 + 2 * x;
                    const float p0 = exp2_fast(fmaf(s[i], sc, l4[2 * x]));
                    const float p1 = exp2_fast(fmaf(s[i + 1], sc, l4[2 * x + 1]));
                    wp[2 * g2 + x] = pack_bf16x2(p0, p1);
                    wd[2 * g2 + x] = pack_bf16x2(p0 * (dp[i] - e4[2 * x]),
                                                 p1 * (dp[i + 1] - e4[2 * x + 1]));
                }
            }
            pb[j] = as_bf16x8(wp);
            dsb[j] = as_bf16x8(wd);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
            const bf16* gtr = gt + (32 * b + c32) * C::QTS + 32 * sb + 8 * hf;
            const bf16* qtr = qt + (32 * b + c32) * C::QTS + 32 * sb + 8 * hf;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dva[b] = mfma32(*reinterpret_cast<const bf16x8*>(gtr + 16 * j), pb[j], dva[b]);
                dka[b] = mfma32(*reinterpret_cast<const bf16x8*>(qtr + 16 * j), dsb[j], dka[b]);
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ cs,
    const float* __restrict__ sn, bf16* __restrict__ dk, bf16* __restrict__ dv, int BH, int T,
    int nkb, float sc, float scale) {
    using C = BwdTile<D>;
    constexpr int NB = C::NBUF;
    __shared__ __attribute__((aligned(16))) f16 Qs[NB][C::QN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Gs[NB][C::QN * C::RS];
    __shared__ __attribute__((aligned(16))) bf16 Qt[NB][D * C::QTS];
    __shared__ __attribute__((aligned(16))) bf16 Gt[NB][D * C::QTS];
    __shared__ __attribute__((aligned(16))) float Ls[NB][C::QN];
    __shared__ __attribute__((aligned(16))) float Dl[NB][C::QN];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int kb = bid / BH;  // key block 0 has the most query tiles: issued first
    const int k0 = kb * C::KM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const size_t roff = (size_t)bh * T;
    const HeadBufs<D> qh(q + hoff, cs, sn, T), kh(k + hoff, cs, sn, T), vh(v + hoff, cs, sn, T),
        gh(dO + hoff, cs, sn, T);
    const int wk0 = k0 + wave * 32;
    const int tk = wk0 + c32;

    const int qt0 = k0 / C::QN;
    const int nqt = (T + C::QN - 1) / C::QN;
    const int qfull = min(nqt, (k0 + C::KM) / C::QN);  // from here on no query precedes a key
    RowStage<D, C::QN, C::NT, true> qst;
    RowStage<D, C::QN, C::NT, false> gst;
    float l_pre = 0.f, d_pre = 0.f;
    auto load_tile = [&](int qt) {
        const int qbase = qt * C::QN;
        qst.load(qh, qbase, tid);
        gst.load(gh, qbase, tid);
        if (tid < C::QN) {
            const int t = qbase + tid;
            l_pre = t < T ? -lse[roff + t] * kLog2e : -INFINITY;
            d_pre = t < T ? delta[roff + t] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
        qst.template store<f16, bf16>(Qs[buf], Qt[buf], tid);
        gst.template store<bf16, bf16>(Gs[buf], Gt[buf], tid);
        if (tid < C::QN) {
            Ls[buf][tid] = l_pre;
            Dl[buf][tid] = d_pre;
        }
    };
    load_tile(qt0);

    f16x8 kf[C::DK];
    bf16x8 vf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const int d0 = 16 * c + 8 * hf;
        kf[c] = rope_operand<D, f16>(kh, tk, d0);
        vf[c] = as_bf16x8(buf_load16(vh.x, (uint32_t)(tk * D + d0) * 2));
    }
    f32x16 dva[C::DB], dka[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dva[b] = dka[b] = f32x16{};

    store_tile(0);
    __syncthreads();

    for (int qt = qt0; qt < nqt; ++qt) {
        const int qbase = qt * C::QN;
        const int it = qt - qt0;
        const int cur = it % NB;
        const bool more = qt + 1 < nqt;
        if (NB == 2 && more) load_tile(qt + 1);
        if (qt >= qfull)
            dkdv_tile<D, false>(dva, dka, kf, vf, Qs[cur], Gs[cur], Qt[cur], Gt[cur], Ls[cur],
                                Dl[cur], qbase, wk0, c32, hf, sc);
        else if (qbase + C::QN - 1 >= wk0)
            dkdv_tile<D, true>(dva, dka, kf, vf, Qs[cur], Gs[cur], Qt[cur], Gt[cur], Ls[cur],
                               Dl[cur], qbase, wk0, c32, hf, sc);
        if (more) {
            if (NB == 1) {  // no prefetch: wait for every wave, then load and store
                __syncthreads();
                load_tile(qt + 1);
            }
            store_tile((it + 1) % NB);
        }
        __syncthreads();
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
                const f32x2 c2 = *reinterpret_cast<const f32x2*>(crow + d / 2);
                const f32x2 s2 = *reinterpret_cast<const f32x2*>(srow + d / 2);
                u32x2 wk, wv;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const float x0 = dka[b][4 * g + 2 * pr] * scale;
                    const float x1 = dka[b][4 * g + 2 * pr + 1] * scale;
                    wk[pr] = pack_bf16x2(x0 * c2[pr] + x1 * s2[pr], x1 * c2[pr] - x0 * s2[pr]);
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
