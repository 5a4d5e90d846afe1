// Backward pass of causal RoPE attention, bf16 storage / fp32 accumulation, gfx950.
//
// The pages' engine computes every gradient by hand, RoPE's included, and checks
// them against centred differences ("Show HN: NanoEuler", paragraph 2). Here the
// backward recomputes the probabilities from the rotated q, k and the saved
// log-sum-exp instead of storing the T x T matrix, in two deterministic kernels
// (no atomics):
//
//   dq kernel   (one workgroup = 128 queries of a head; loops over key tiles
//                up to the diagonal): delta_t = sum_d dO[t,d] o[t,d] in its
//                prologue, written with lse_t*log2(e) to the workspace, then
//                P = exp(S - lse), dP = dO V^T, dS = P (dP - delta),
//                dQ^r += s dS K^r, and finally dq = R_t^T dQ^r.
//   dkdv kernel (one workgroup = 128 keys of a head; loops over query tiles
//                from the diagonal down): with the same P and dS,
//                dV += P^T dO, dK^r += s dS^T Q^r, and finally dk = R_u^T dK^r.
//
// Every product is a 32x32x16 MFMA contraction with fp32 accumulation. The
// rotated q and k and dS are fp16 (the score recompute needs the 11-bit
// significand, see the forward; dS then shares the fp16 MFMA with them, which
// bounds |dS| by 65504); dO, V and P are bf16. In the dq kernel a lane column
// is a query (S^T, dP^T, dQ^T), in the dkdv kernel a key (S, dP, dV^T, dK^T).
// Tiles stream from global memory straight into an NS-stage LDS ring
// (buffer_load ... lds); row-major tiles give the row operands with 16-byte
// reads and the transposed operands through ds_read_b64_tr_b16, so rounded P
// and dS registers are directly the B operand of the next contraction.
#include "device_common.h"
#include "launchers.h"

namespace attn {

template <int D>
struct BwdTile {
    static constexpr int NT = 256;
    static constexpr int NW = 4;
    static constexpr int DK = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int QM = 128;     // dq kernel: queries per workgroup
    static constexpr int KN = 64;      // dq kernel: keys per LDS tile
    static constexpr int KM = 128;     // dkdv kernel: keys per workgroup
    static constexpr int QN = 64;      // dkdv kernel: queries per LDS tile
    static constexpr int TILE = 64 * D * 2;            // bytes of one 64-row tile
    static constexpr int NS = D == 64 ? 3 : 2;         // LDS ring stages
    static constexpr int LPT = 2 * TILE / 1024 / NW;   // tile load instructions per wave
};

// One 64-key tile of the dq kernel for one wave (32 queries). DIAG: the tile may
// reach this wave's diagonal (32-key blocks above it skipped, the diagonal one masked).
template <int D, bool DIAG>
__device__ __forceinline__ void dq_tile(f32x16* acc, const f16x8* qf, const bf16x8* df,
                                        const char* ks, const char* vs, int k0, int wq0,
                                        int lane, float sc, float lt, float dl) {
    using C = BwdTile<D>;
    const int c32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int sb = 0; sb < C::KN / 32; ++sb) {
        const int kb = k0 + 32 * sb;
        if (DIAG && kb > wq0) break;
        const int row = 32 * sb + c32;
        f32x16 s = mfma32(lds_row8<D, f16x8>(ks, row, 8 * hf), qf[0], f32x16{});
        f32x16 dp = mfma32(lds_row8<D, bf16x8>(vs, row, 8 * hf), df[0], f32x16{});
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            s = mfma32(lds_row8<D, f16x8>(ks, row, 16 * c + 8 * hf), qf[c], s);
            dp = mfma32(lds_row8<D, bf16x8>(vs, row, 16 * c + 8 * hf), df[c], dp);
        }
        if (DIAG && kb == wq0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) > c32) s[i] = -INFINITY;
        }
        f16x8 dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * j + 2 * e;
                const float p0 = exp2_fast(fmaf(s[i], sc, -lt));
                const float p1 = exp2_fast(fmaf(s[i + 1], sc, -lt));
                w[e] = pack2<f16>(p0 * (dp[i] - dl), p1 * (dp[i + 1] - dl));
            }
            dsb[j] = as_vec8<f16x8>(w);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[b] = mfma32(lds_tr8<D, f16x8>(ks, 32 * sb + 16 * j, 32 * b, lane), dsb[j], acc[b]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dq_bf16_kernel(
    const f16* __restrict__ qr, const f16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ cs, const float* __restrict__ sn, bf16* __restrict__ dq,
    float* __restrict__ ws, int BH, int T, int nqb, float sc, float scale) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    __shared__ __attribute__((aligned(1024))) char smem[NS][2 * C::TILE];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::QM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const uint32_t hbytes = (uint32_t)T * D * 2;
    const rsrc_t qh = make_rsrc(qr + hoff, hbytes), kh = make_rsrc(kr + hoff, hbytes),
                 vh = make_rsrc(v + hoff, hbytes), gh = make_rsrc(dO + hoff, hbytes),
                 oh = make_rsrc(o + hoff, hbytes);
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;

    // this lane's query: rotated q (fp16), dO (bf16), and delta = sum_d dO o
    f16x8 qf[C::DK];
    bf16x8 df[C::DK];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const uint32_t off = (uint32_t)(tq * D + 16 * c + 8 * hf) * 2;
        qf[c] = __builtin_bit_cast(f16x8, buf_load16(qh, off));
        const u32x4 g = buf_load16(gh, off);
        const u32x4 y = buf_load16(oh, off);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dot += bf16_lo(g[e]) * bf16_lo(y[e]) + bf16_hi(g[e]) * bf16_hi(y[e]);
        df[c] = as_bf16x8(g);
    }
    const float dl = sum_across_halves(dot);
    const float lt = tq < T ? lse[(size_t)bh * T + tq] * kLog2e : 0.f;
    if (tq < T && hf == 0) *reinterpret_cast<f32x2*>(ws + 2 * ((size_t)bh * T + tq)) = f32x2{lt, dl};

    const int kend = min(T, q0 + C::QM);
    const int ntiles = (kend + C::KN - 1) / C::KN;
    const int nfull = min(ntiles, q0 / C::KN);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
        issue_tile<D, C::KN, C::NW>(kh, s * C::KN, smem[s], wave, lane);
        issue_tile<D, C::KN, C::NW>(vh, s * C::KN, smem[s] + C::TILE, wave, lane);
    }

    f32x16 acc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};

    for (int n = 0; n < ntiles; ++n) {
        wait_vmcnt<C::LPT * (NS - 2)>();
        __syncthreads();
        const int nx = n + NS - 1;
        issue_tile<D, C::KN, C::NW>(kh, nx * C::KN, smem[nx % NS], wave, lane);
        issue_tile<D, C::KN, C::NW>(vh, nx * C::KN, smem[nx % NS] + C::TILE, wave, lane);
        const char* ks = smem[n % NS];
        const char* vs = ks + C::TILE;
        const int k0 = n * C::KN;
        if (n < nfull)
            dq_tile<D, false>(acc, qf, df, ks, vs, k0, wq0, lane, sc, lt, dl);
        else if (k0 <= wq0)
            dq_tile<D, true>(acc, qf, df, ks, vs, k0, wq0, lane, sc, lt, dl);
    }
    wait_vmcnt<0>();

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
// first key skipped, the diagonal one masked). ld holds (lse*log2 e, delta)
// for the tile's 64 queries.
template <int D, bool DIAG>
__device__ __forceinline__ void dkdv_tile(f32x16* dva, f32x16* dka, const f16x8* kf,
                                          const bf16x8* vf, const char* qs, const char* gs,
                                          const float* ld, int qbase, int wk0, int lane,
                                          float sc) {
    using C = BwdTile<D>;
    const int c32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int sb = 0; sb < C::QN / 32; ++sb) {
        const int qb = qbase + 32 * sb;
        if (DIAG && qb + 31 < wk0) continue;
        const int row = 32 * sb + c32;
        f32x16 s = mfma32(lds_row8<D, f16x8>(qs, row, 8 * hf), kf[0], f32x16{});
        f32x16 dp = mfma32(lds_row8<D, bf16x8>(gs, row, 8 * hf), vf[0], f32x16{});
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            s = mfma32(lds_row8<D, f16x8>(qs, row, 16 * c + 8 * hf), kf[c], s);
            dp = mfma32(lds_row8<D, bf16x8>(gs, row, 16 * c + 8 * hf), vf[c], dp);
        }
        if (DIAG && qb == wk0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) < c32) s[i] = -INFINITY;
        }
        bf16x8 pb[2];
        f16x8 dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 wp, wd;
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
                // items 8j + 4*g2 .. +3 belong to queries 16j + 8*g2 + 4*hf .. +3
                const float* lq = ld + 2 * (32 * sb + 16 * j + 8 * g2 + 4 * hf);
                const f32x4 a01 = *reinterpret_cast<const f32x4*>(lq);      // l0 d0 l1 d1
                const f32x4 a23 = *reinterpret_cast<const f32x4*>(lq + 4);  // l2 d2 l3 d3
                const int i = 8 * j + 4 * g2;
                const float p0 = exp2_fast(fmaf(s[i], sc, -a01[0]));
                const float p1 = exp2_fast(fmaf(s[i + 1], sc, -a01[2]));
                const float p2 = exp2_fast(fmaf(s[i + 2], sc, -a23[0]));
                const float p3 = exp2_fast(fmaf(s[i + 3], sc, -a23[2]));
                wp[2 * g2] = pack_bf16x2(p0, p1);
                wp[2 * g2 + 1] = pack_bf16x2(p2, p3);
                wd[2 * g2] = pack2<f16>(p0 * (dp[i] - a01[1]), p1 * (dp[i + 1] - a01[3]));
                wd[2 * g2 + 1] = pack2<f16>(p2 * (dp[i + 2] - a23[1]), p3 * (dp[i + 3] - a23[3]));
            }
            pb[j] = as_bf16x8(wp);
            dsb[j] = as_vec8<f16x8>(wd);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dva[b] = mfma32(lds_tr8<D, bf16x8>(gs, 32 * sb + 16 * j, 32 * b, lane), pb[j], dva[b]);
                dka[b] = mfma32(lds_tr8<D, f16x8>(qs, 32 * sb + 16 * j, 32 * b, lane), dsb[j], dka[b]);
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_bf16_kernel(
    const f16* __restrict__ qr, const f16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ ws, const float* __restrict__ cs,
    const float* __restrict__ sn, bf16* __restrict__ dk, bf16* __restrict__ dv, int BH, int T,
    int nkb, float sc, float scale) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    constexpr int STAGE = 2 * C::TILE + 512;  // Q tile, dO tile, 64 x (lse*log2 e, delta)
    __shared__ __attribute__((aligned(1024))) char smem[NS][STAGE];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int kb = bid / BH;  // key block 0 has the most query tiles: issued first
    const int k0 = kb * C::KM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const uint32_t hbytes = (uint32_t)T * D * 2;
    const rsrc_t qh = make_rsrc(qr + hoff, hbytes), kh = make_rsrc(kr + hoff, hbytes),
                 vh = make_rsrc(v + hoff, hbytes), gh = make_rsrc(dO + hoff, hbytes),
                 lh = make_rsrc(ws + 2 * (size_t)bh * T, (uint32_t)T * 8);
    const int wk0 = k0 + wave * 32;
    const int tk = wk0 + c32;

    const int qt0 = k0 / C::QN;
    const int nqt = (T + C::QN - 1) / C::QN;
    const int qfull = min(nqt, (k0 + C::KM) / C::QN);  // from here on no query precedes a key
    // one tile = Q, dO (row-major) and the (lse*log2 e, delta) pairs of its 64
    // queries; each wave fetches 16 of those pairs with one dword load
    auto issue = [&](int qt, char* st) {
        issue_tile<D, C::QN, C::NW>(qh, qt * C::QN, st, wave, lane);
        issue_tile<D, C::QN, C::NW>(gh, qt * C::QN, st + C::TILE, wave, lane);
        if (lane < 32)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                lh, LDS_PTR(st + 2 * C::TILE + 128 * wave), 4,
                (uint32_t)((qt * C::QN + 16 * wave) * 8 + 4 * lane), 0, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(qt0 + s, smem[s]);

    f16x8 kf[C::DK];
    bf16x8 vf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const uint32_t off = (uint32_t)(tk * D + 16 * c + 8 * hf) * 2;
        kf[c] = __builtin_bit_cast(f16x8, buf_load16(kh, off));
        vf[c] = as_bf16x8(buf_load16(vh, off));
    }
    f32x16 dva[C::DB], dka[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dva[b] = dka[b] = f32x16{};

    for (int qt = qt0; qt < nqt; ++qt) {
        const int it = qt - qt0;
        wait_vmcnt<(C::LPT + 1) * (NS - 2)>();
        __syncthreads();
        issue(qt + NS - 1, smem[(it + NS - 1) % NS]);
        const char* qs = smem[it % NS];
        const char* gs = qs + C::TILE;
        const float* ld = reinterpret_cast<const float*>(qs + 2 * C::TILE);
        const int qbase = qt * C::QN;
        if (qt >= qfull)
            dkdv_tile<D, false>(dva, dka, kf, vf, qs, gs, ld, qbase, wk0, lane, sc);
        else if (qbase + C::QN - 1 >= wk0)
            dkdv_tile<D, true>(dva, dka, kf, vf, qs, gs, ld, qbase, wk0, lane, sc);
    }
    wait_vmcnt<0>();

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
    const size_t n = (size_t)a.B * a.H * a.T * a.D;
    const f16* rot = static_cast<const f16*>(a.rot);
    hipLaunchKernelGGL(bwd_dq_bf16_kernel<D>, dim3(nqb * BH), dim3(C::NT), 0, a.stream, rot,
                       rot + n, (const bf16*)a.v, (const bf16*)a.o, (const bf16*)a.dO, a.lse,
                       a.cs, a.sn, (bf16*)a.dq, a.ws, BH, a.T, nqb, scale * kLog2e, scale);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv(const BwdArgs& a) {
    using C = BwdTile<D>;
    const int BH = a.B * a.H;
    const int nkb = (a.T + C::KM - 1) / C::KM;
    const float scale = 1.f / sqrtf((float)D);
    const size_t n = (size_t)a.B * a.H * a.T * a.D;
    const f16* rot = static_cast<const f16*>(a.rot);
    hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<D>, dim3(nkb * BH), dim3(C::NT), 0, a.stream, rot,
                       rot + n, (const bf16*)a.v, (const bf16*)a.dO, a.ws, a.cs, a.sn,
                       (bf16*)a.dk, (bf16*)a.dv, BH, a.T, nkb, scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) {
    return a.D == 64 ? launch_dq<64>(a) : launch_dq<128>(a);
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a) {
    return a.D == 64 ? launch_dkdv<64>(a) : launch_dkdv<128>(a);
}

}  // namespace attn
