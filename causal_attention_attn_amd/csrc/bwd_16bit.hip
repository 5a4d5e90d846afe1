// Backward pass of causal RoPE attention, 16-bit storage (bf16 or fp16, type E)
// with fp32 accumulation, gfx950.
//
// The pages' engine computes every gradient by hand, RoPE's included, and checks
// them against centred differences ("Show HN: NanoEuler", paragraph 2). Here the
// backward recomputes the probabilities from the rotated q, k and the saved
// log-sum-exp instead of storing the T x T matrix. After the per-row pre-pass
// (bwd_prep.hip: -lse*log2(e) and -delta in the workspace) one deterministic
// launch (no atomics) runs two kinds of work item:
//
//   dq item   (128 queries of a head; loops over key tiles up to the diagonal):
//             P = exp(S - lse), dP = dO V^T, dS = P (dP - delta),
//             dQ^r += s dS K^r, and finally dq = R_t^T dQ^r.
//   dkdv item (128 keys of a head; loops over query tiles from the diagonal
//             down): with the same P and dS, dV += P^T dO, dK^r += s dS^T Q^r,
//             and finally dk = R_u^T dK^r.
//
// Running both kinds in one grid lets the light items of one kind fill the
// gaps the other leaves, with a single tail.
//
// The saved query carries the factor log2(e)/sqrt(D), so a score product is
// S log2(e) and P = 2^(S log2(e) - lse log2(e)). The per-query offsets
// -lse log2(e) and -delta are the initial accumulators of the S and dP
// products, which leaves one exp2 and one multiply per element for dS; the
// factor on the query is undone in dK^r (ln 2 instead of s).
//
// Every product is a 32x32x16 MFMA contraction with fp32 accumulation. The
// rotated q and k and dS are fp16 (the score recompute needs the 11-bit
// significand, see the forward; dS then shares the fp16 MFMA with them, which
// bounds |dS| by 65504); dO, V and P are of the storage type E. In a dq item a lane column is a
// query (S^T, dP^T, dQ^T), in a dkdv item a key (S, dP, dV^T, dK^T). Tiles
// stream from global memory straight into an NS-stage LDS ring
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

// The RoPE table entries this lane's epilogue needs to rotate its row t back:
// features d = 32b + 8g + 4h .. +3 (h = lane >> 5), i.e. the cos/sin pairs
// d/2, d/2 + 1. Loaded once the item's tile loop is done, so that the loop
// runs without these 32 registers (held through the loop they pushed the
// kernel to its register limit and into spills). Rows past the end read row 0
// (their results are not stored).
template <int D>
struct RowTables {
    f32x2 c[D / 32][4], s[D / 32][4];
    __device__ __forceinline__ void load(const float* cs, const float* sn, int t, int T, int hf) {
        const size_t row = (size_t)(t < T ? t : 0) * (D / 2);
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * b + 8 * g + 4 * hf;
                c[b][g] = *reinterpret_cast<const f32x2*>(cs + row + d / 2);
                s[b][g] = *reinterpret_cast<const f32x2*>(sn + row + d / 2);
            }
    }
    // The same entries from the table rows stage_tables copied into LDS: row r
    // (0 .. 63) of the 64-row blocks cb (cos) and sb (sin) that hold this lane's row.
    __device__ __forceinline__ void load_lds(const char* cb, const char* sb, int r, int hf) {
        static_assert(D == 64, "LDS table rows are 128 bytes");
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int off = r * 128 + 16 * ((4 * b + g) ^ (r & 7)) + 8 * hf;
                c[b][g] = *reinterpret_cast<const f32x2*>(cb + off);
                s[b][g] = *reinterpret_cast<const f32x2*>(sb + off);
            }
    }
};

// At D = 64 (three ring stages) an item's RoPE table rows - cos and sin of its
// 128 rows, 16 KB each - are copied straight into LDS during its last tile
// step, into the two stages that step leaves free (no tile follows it), so the
// epilogue finds them there instead of waiting for a memory round trip after
// the loop. Wave w copies one 8 KB block: w = 0, 1 the cos rows 0-63 and 64-127
// (into ca, cb), w = 2, 3 the sin rows (into sa, sb). In LDS the 16-byte chunk
// c of row r sits at position c ^ (r & 7), so that 32 lanes reading one chunk
// of 32 consecutive rows spread over the banks. Rows past T read as zeros (their
// results are not stored).
template <int D>
__device__ __forceinline__ void stage_tables(const float* cs, const float* sn, int r0, int T,
                                             char* ca, char* cb, char* sa, char* sb, int wave,
                                             int lane) {
    static_assert(D == 64, "one table row is 128 bytes");
    const int rows = T > r0 ? T - r0 : 0;
    const rsrc_t src = make_rsrc((wave < 2 ? cs : sn) + (size_t)r0 * (D / 2),
                                 (uint32_t)rows * (D / 2) * 4);
    char* dst = wave == 0 ? ca : wave == 1 ? cb : wave == 2 ? sa : sb;
    // instruction i fills LDS bytes [1024 i, +1024) of the block: rows 8i + rr.
    // The whole offset goes in the per-lane register: an instruction's immediate
    // offset would be added to the LDS address as well.
    const int rr = lane >> 3, pos = lane & 7;
    const uint32_t v0 = (uint32_t)((wave & 1) * 64 * 128 + rr * 128 + 16 * (pos ^ rr));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, LDS_PTR(dst + i * 1024), 16,
                                                 v0 + (uint32_t)i * 1024, 0, 0, 0);
}

// Epilogue stores through LDS. A wave's 32 output rows (2D bytes each) are put
// into a 32 x 2D-byte LDS buffer in the accumulator layout (lane (c, h) owns
// features 32b + 8g + 4h .. +3 of row c: 8 bytes), with the 16-byte chunks of
// row r rotated by XOR with r & 7 so that the rows of a put spread over the
// banks; then each 16-byte store of the wave covers 64 x 16 / 2D whole rows
// (contiguous in a plain head) instead of 16 bytes of 32 rows.
template <int D>
struct RowStage {
    static constexpr int NCH = D / 8;     // 16-byte chunks per row
    static constexpr int RPI = 64 / NCH;  // rows per store instruction
    char* buf;
    __device__ __forceinline__ void put(int c32, int hf, int b, int g, u32x2 w) const {
        const int ch = 4 * b + g;
        *reinterpret_cast<u32x2*>(buf + c32 * (2 * D) + 16 * (ch ^ (c32 & 7)) + 8 * hf) = w;
    }
    // rows row0 .. row0+31 (those below T) of a head whose rows are `pitch`
    // elements apart
    template <typename E>
    __device__ __forceinline__ void store(E* head, int row0, int T, int pitch, int lane) const {
        const int c = lane % NCH;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = it * RPI + lane / NCH;
            const u32x4 w =
                *reinterpret_cast<const u32x4*>(buf + r * (2 * D) + 16 * (c ^ (r & 7)));
            if (row0 + r < T)
                *reinterpret_cast<u32x4*>(row_ptr(head, row0 + r, pitch) + 8 * c) = w;
        }
    }
};

// An item's output rows: this wave's 32 rows of R^T (scale * acc) (dq, dk) or of
// acc itself (dv), rounded to E, staged through LDS and stored as whole rows.
template <int D, typename E>
__device__ __forceinline__ void rope_out(const f32x16* acc, float scale, const RowTables<D>& tb,
                                         const RowStage<D>& sg, E* head, int row0, int T,
                                         int pitch, int c32, int hf, int lane) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x2 c2 = tb.c[b][g], s2 = tb.s[b][g];
            u32x2 w;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const float x0 = acc[b][4 * g + 2 * pr] * scale;
                const float x1 = acc[b][4 * g + 2 * pr + 1] * scale;
                w[pr] = pack2<E>(x0 * c2[pr] + x1 * s2[pr], x1 * c2[pr] - x0 * s2[pr]);
            }
            sg.put(c32, hf, b, g, w);
        }
    }
    sg.store(head, row0, T, pitch, lane);
}
template <int D, typename E>
__device__ __forceinline__ void plain_out(const f32x16* acc, const RowStage<D>& sg, E* head,
                                          int row0, int T, int pitch, int c32, int hf, int lane) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
                w[pr] = pack2<E>(acc[b][4 * g + 2 * pr], acc[b][4 * g + 2 * pr + 1]);
            sg.put(c32, hf, b, g, w);
        }
    }
    sg.store(head, row0, T, pitch, lane);
}

// This wave's staging buffer once the ring is idle: one of the ring's stage
// buffers (64 x 2D bytes each: room for two outputs of 32 rows).
template <int D>
__device__ __forceinline__ char* stage_buffer(const Ring& rg, int wave) {
    constexpr int NS = BwdTile<D>::NS;
    if (wave == 0) return rg.k[0];
    if (wave == 1) return rg.k[1];
    if constexpr (NS > 2) return wave == 2 ? rg.k[2] : rg.v[0];
    else return wave == 2 ? rg.v[0] : rg.v[1];
}

// One 64-key tile of the dq kernel for one wave (32 queries). DIAG: the tile may
// reach this wave's diagonal (32-key blocks above it skipped, the diagonal one masked).
template <int D, typename E, bool DIAG>
__device__ __forceinline__ void dq_tile(f32x16* acc, const f16x8* qf, const vec8<E>* df,
                                        const char* ks, const char* vs, const OperandOffs<D>& of,
                                        int k0, int wq0, int lane, const f32x16& nl,
                                        const f32x16& nd) {
    using C = BwdTile<D>;
    constexpr int ROWB = 2 * D;
    const int c32 = lane & 31, hf = lane >> 5;
    if (DIAG && k0 > wq0) return;
#pragma unroll
    for (int sb = 0; sb < C::KN / 32; ++sb) {
        const int kb = k0 + 32 * sb;
        if (DIAG && kb > wq0) break;
        const char* kr = ks + 32 * sb * ROWB;
        const char* vr = vs + 32 * sb * ROWB;
        // x = S log2(e) - lse log2(e) and dp = dP - delta: the offsets are the
        // accumulators' initial values
        f32x16 x = mfma32(*reinterpret_cast<const f16x8*>(kr + of.k[0]), qf[0], nl);
        f32x16 dp = mfma32(*reinterpret_cast<const vec8<E>*>(vr + of.k[0]), df[0], nd);
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            x = mfma32(*reinterpret_cast<const f16x8*>(kr + of.k[c]), qf[c], x);
            dp = mfma32(*reinterpret_cast<const vec8<E>*>(vr + of.k[c]), df[c], dp);
        }
        if (DIAG && kb == wq0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) > c32) x[i] = -INFINITY;
        }
        f16x8 dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * j + 2 * e;
                w[e] = pack2<f16>(exp2_fast(x[i]) * dp[i], exp2_fast(x[i + 1]) * dp[i + 1]);
            }
            dsb[j] = as_vec8<f16x8>(w);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const char* t = ks + (32 * sb + 16 * j) * ROWB;
                acc[b] = mfma32(tr_pair<f16x8>(t + of.v[b][0], t + of.v[b][1]), dsb[j], acc[b]);
            }
        }
    }
}

// Where an item's RoPE table rows come from (see stage_tables): the tables and
// the item's first row.
struct TabSrc {
    const float* cs;
    const float* sn;
    int r0;
};

// Step n of the dq kernel's key-tile loop on ring stage STG (= n % NS). LAST:
// the item's last step (D = 64 only), which copies the item's RoPE table rows
// into the two stages it leaves free.
template <int D, typename E, int STG, bool DIAG, bool STRIDED, bool LAST = false>
__device__ __forceinline__ void dq_step(f32x16* acc, const f16x8* qf, const vec8<E>* df,
                                        const Ring& rg,
                                        const TileLoads<D, 64, 4>& ld, const OperandOffs<D>& of,
                                        const f16* kr, const E* v, int vst, int T, int n,
                                        int ntiles,
                                        int wq0, int lane, int wave, const f32x16& nl,
                                        const f32x16& nd, const TabSrc& tab = {}) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    constexpr int NXT = (STG + NS - 1) % NS;
    // tiles past the item's last one are never loaded, so the last step has no
    // younger tile in flight and waits for everything
    if (!LAST && n + 1 < ntiles) wait_vmcnt<C::LPT * (NS - 2)>();
    else wait_vmcnt<0>();
    ring_barrier();
    if constexpr (LAST) {
        static_assert(NS == 3, "the last step's free stages");
        constexpr int A = (STG + 1) % NS, B = (STG + 2) % NS;
        stage_tables<D>(tab.cs, tab.sn, tab.r0, T, rg.k[A], rg.v[A], rg.k[B], rg.v[B], wave,
                        lane);
    } else {
        const int nx = n + NS - 1;
        if (nx < ntiles) {
            ld.issue(kr, T, nx * C::KN, rg.k[NXT], wave);
            if constexpr (STRIDED) ld.issue_strided(v, T, nx * C::KN, rg.v[NXT], wave, vst);
            else ld.issue(v, T, nx * C::KN, rg.v[NXT], wave);
        }
    }
    dq_tile<D, E, DIAG>(acc, qf, df, rg.k[STG], rg.v[STG], of, n * C::KN, wq0, lane, nl, nd);
}

// Pointers and sizes shared by the two kinds of work item of the gradient kernel.
template <typename E>
struct BwdPtrs {
    const f16* qr;     // rotated q * log2(e)/sqrt(D), fp16
    const f16* kr;     // rotated k, fp16
    const E* v;
    const E* dO;
    const float* ws;   // -lse*log2(e) of every row, then -delta of every row
    const float* cs;
    const float* sn;
    E *dq, *dk, *dv;
    Layout lv;         // v, dq, dk and dv
    Layout lo;         // dO
    int H, BH, T;
};

// dq item: the 128 queries of q-block qb of head bh (loops over key tiles up
// to the diagonal; rg.k / rg.v hold K / V tiles).
template <int D, typename E, bool STRIDED>
__device__ __forceinline__ void dq_item(const BwdPtrs<E>& pp, const Ring& rg, int bh, int qb) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    const int T = pp.T, BH = pp.BH;
    const f16* __restrict__ qr = pp.qr;
    const E* __restrict__ dO = pp.dO;
    const float* __restrict__ ws = pp.ws;
    const float* __restrict__ cs = pp.cs;
    const float* __restrict__ sn = pp.sn;
    E* __restrict__ dq = pp.dq;
    const float scale = 1.f / sqrtf((float)D);
    const int q0 = qb * C::QM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const uint32_t hbytes = (uint32_t)T * D * 2;
    const f16* kh = pp.kr + hoff;
    // v, dO and dq: [B, H, T, D] unless STRIDED (then where their layouts put them)
    const int vst = STRIDED ? pp.lv.st : D, gst = STRIDED ? pp.lo.st : D;
    const long long vhead = STRIDED ? pp.lv.head(bh, pp.H) : (long long)hoff;
    const E* vh = pp.v + vhead;
    const rsrc_t qbuf = make_rsrc(qr + hoff, hbytes);
    const rsrc_t gbuf =
        STRIDED ? make_rsrc(dO + pp.lo.head(bh, pp.H), pp.lo.head_bytes(T, D))
                : make_rsrc(dO + hoff, hbytes);
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;
    const TileLoads<D, 64, 4> ld(wave, lane);
    const OperandOffs<D> of(lane);

    const int kend = min(T, q0 + C::QM);
    const int ntiles = (kend + C::KN - 1) / C::KN;
    const int nfull = min(ntiles, q0 / C::KN);
    // tile 0, then this lane's query: rotated q (fp16), dO (E) and its two row
    // offsets, then tiles 1 .. NS-2; the first step waits for tile 0 and the query only
    ld.issue(kh, T, 0, rg.k[0], wave);
    if constexpr (STRIDED) ld.issue_strided(vh, T, 0, rg.v[0], wave, vst);
    else ld.issue(vh, T, 0, rg.v[0], wave);
    f16x8 qf[C::DK];
    vec8<E> df[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const uint32_t col = (uint32_t)(16 * c + 8 * hf) * 2;
        qf[c] = __builtin_bit_cast(f16x8, buf_load16(qbuf, (uint32_t)tq * D * 2 + col));
        df[c] = as_vec8<vec8<E>>(buf_load16(gbuf, (uint32_t)tq * gst * 2 + col));
    }
    const float nlt = tq < T ? ws[(size_t)bh * T + tq] : 0.f;
    const float ndl = tq < T ? ws[(size_t)BH * T + (size_t)bh * T + tq] : 0.f;
#pragma unroll
    for (int s = 1; s < NS - 1; ++s) {
        if (s < ntiles) {
            ld.issue(kh, T, s * C::KN, rg.k[s], wave);
            if constexpr (STRIDED) ld.issue_strided(vh, T, s * C::KN, rg.v[s], wave, vst);
            else ld.issue(vh, T, s * C::KN, rg.v[s], wave);
        }
    }
    const f32x16 nl = splat16(nlt), nd = splat16(ndl);

    f32x16 acc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};

    int n = 0;
    for (; n + NS <= nfull; n += NS) {
        dq_step<D, E, 0, false, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd);
        dq_step<D, E, 1, false, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n + 1, ntiles, wq0, lane, wave, nl, nd);
        if constexpr (NS > 2)
            dq_step<D, E, 2, false, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n + 2, ntiles, wq0, lane, wave, nl, nd);
    }
    // the remaining steps reach the diagonal; with three stages the last one is
    // peeled off (it copies the RoPE table rows for the epilogue into LDS)
    constexpr bool TAB = NS == 3;
    if constexpr (TAB) {
        // at most NS-1 full tiles and one of the two diagonal tiles precede the
        // last step, on stages 0, 1, 2 in turn: straight-line steps with
        // compile-time stages (a loop that picks the stage at run time makes the
        // compiler copy the accumulators between its branches)
        static_assert(C::QM / C::KN == 2, "two diagonal key tiles per q-block");
        if (n + 1 < ntiles) {
            dq_step<D, E, 0, true, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd);
            ++n;
        }
        if (n + 1 < ntiles) {
            dq_step<D, E, 1, true, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd);
            ++n;
        }
        if (n + 1 < ntiles) {
            dq_step<D, E, 2, true, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd);
            ++n;
        }
    } else {
        // two stages, no peeled step: at most one full tile and the two diagonal
        // tiles remain, on stages 0, 1, 0
        static_for<3>([&](auto S) {
            if (n < ntiles) {
                dq_step<D, E, S % NS, true, STRIDED>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd);
                ++n;
            }
        });
    }
    if constexpr (TAB) {
        // the last step and the epilogue, with the last step's ring stage L a
        // compile-time constant (the stage buffers are distinct LDS objects)
        const TabSrc tab = {cs, sn, q0};
        const int stg = n % NS;
        static_for<NS>([&](auto S) {
            constexpr int L = decltype(S)::value;
            if (stg != L) return;
            dq_step<D, E, L, true, STRIDED, true>(acc, qf, df, rg, ld, of, kh, vh, vst, T, n, ntiles, wq0, lane, wave, nl, nd, tab);
            wait_vmcnt<0>();
            __syncthreads();  // the table rows have landed and every wave is done with the ring
            // the table rows sit in the two stages after L; stage L itself (16 KB)
            // stages the output rows, 4 KB per wave
            constexpr int A = (L + 1) % NS, B = (L + 2) % NS;
            const bool h = wave >= 2;
            RowTables<D> tb;
            tb.load_lds(h ? rg.v[A] : rg.k[A], h ? rg.v[B] : rg.k[B], 32 * (wave & 1) + c32, hf);
            const RowStage<D> sg = {(h ? rg.v[L] : rg.k[L]) + (wave & 1) * 32 * 2 * D};
            rope_out<D, E>(acc, scale, tb, sg, dq + vhead, wq0, T, vst, c32, hf, lane);
        });
    } else {
        RowTables<D> tb;
        tb.load(cs, sn, tq, T, hf);
        wait_vmcnt<0>();
        __syncthreads();  // the ring is idle: its stage buffers hold the output rows
        const RowStage<D> sg = {stage_buffer<D>(rg, wave)};
        rope_out<D, E>(acc, scale, tb, sg, dq + vhead, wq0, T, vst, c32, hf, lane);
    }
}

// One 64-query tile of the dk/dv kernel for one wave (32 keys). DIAG: the tile
// may reach this wave's diagonal (32-query blocks wholly before the wave's
// first key skipped, the diagonal one masked). ld holds -lse*log2(e) of the
// tile's 64 queries, then their -delta; in S and dP a lane is a key and the
// items are queries, so these per-query offsets, read as the accumulators'
// initial values, give x = S log2(e) - lse log2(e) and dp = dP - delta.
template <int D, typename E, bool DIAG>
__device__ __forceinline__ void dkdv_tile(f32x16* dva, f32x16* dka, const f16x8* kf,
                                          const vec8<E>* vf, const char* qs, const char* gs,
                                          const float* ld, const OperandOffs<D>& of, int qbase,
                                          int wk0, int lane) {
    using C = BwdTile<D>;
    constexpr int ROWB = 2 * D;
    const int c32 = lane & 31, hf = lane >> 5;
    if (DIAG && qbase + C::QN - 1 < wk0) return;
#pragma unroll
    for (int sb = 0; sb < C::QN / 32; ++sb) {
        const int qb = qbase + 32 * sb;
        if (DIAG && qb + 31 < wk0) continue;
        const char* qr = qs + 32 * sb * ROWB;
        const char* gr = gs + 32 * sb * ROWB;
        // items 4g .. 4g+3 of a lane half hf are queries 8g + 4hf .. +3 of the block
        f32x16 nl, nd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(ld + 32 * sb + 8 * g + 4 * hf);
            const f32x4 b = *reinterpret_cast<const f32x4*>(ld + 64 + 32 * sb + 8 * g + 4 * hf);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nl[4 * g + e] = a[e];
                nd[4 * g + e] = b[e];
            }
        }
        f32x16 x = mfma32(*reinterpret_cast<const f16x8*>(qr + of.k[0]), kf[0], nl);
        f32x16 dp = mfma32(*reinterpret_cast<const vec8<E>*>(gr + of.k[0]), vf[0], nd);
#pragma unroll
        for (int c = 1; c < C::DK; ++c) {
            x = mfma32(*reinterpret_cast<const f16x8*>(qr + of.k[c]), kf[c], x);
            dp = mfma32(*reinterpret_cast<const vec8<E>*>(gr + of.k[c]), vf[c], dp);
        }
        if (DIAG && qb == wk0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) < c32) x[i] = -INFINITY;
        }
        vec8<E> pb[2];
        f16x8 dsb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 wp, wd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * j + 2 * e;
                const float p0 = exp2_fast(x[i]), p1 = exp2_fast(x[i + 1]);
                wp[e] = pack2<E>(p0, p1);
                wd[e] = pack2<f16>(p0 * dp[i], p1 * dp[i + 1]);
            }
            pb[j] = as_vec8<vec8<E>>(wp);
            dsb[j] = as_vec8<f16x8>(wd);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const char* gt = gs + (32 * sb + 16 * j) * ROWB;
                const char* qt = qs + (32 * sb + 16 * j) * ROWB;
                dva[b] = mfma32(tr_pair<vec8<E>>(gt + of.v[b][0], gt + of.v[b][1]), pb[j], dva[b]);
                dka[b] = mfma32(tr_pair<f16x8>(qt + of.v[b][0], qt + of.v[b][1]), dsb[j], dka[b]);
            }
        }
    }
}

template <int D, typename E, bool STRIDED>
struct DkdvCtx {
    const f16* qh;
    const E* gh;
    const float* oh;  // this wave's per-row offsets: -lse*log2(e) (waves 0, 1) or -delta (2, 3)
    int gst;          // elements between consecutive rows of dO
    int T, wk0, lane, wave;

    // query tile qt -> LDS stage: rotated Q and dO tiles, then 32 of the 128
    // per-query offsets of its 64 queries from each wave (rows past T read 0)
    __device__ __forceinline__ void issue(const TileLoads<D, 64, 4>& ld, int qt, char* qs,
                                          char* gs, char* ls) const {
        constexpr int QN = BwdTile<D>::QN;
        ld.issue(qh, T, qt * QN, qs, wave);
        if constexpr (STRIDED) ld.issue_strided(gh, T, qt * QN, gs, wave, gst);
        else ld.issue(gh, T, qt * QN, gs, wave);
        if (lane < 32)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                make_rsrc(oh, (uint32_t)T * 4), LDS_PTR(ls + 128 * wave), 4,
                (uint32_t)((qt * QN + 32 * (wave & 1)) * 4 + 4 * lane), 0, 0, 0);
    }
};

// Step of the dk/dv kernel's query-tile loop on ring stage STG. LAST: the
// item's last step (D = 64 only), which copies the item's RoPE table rows into
// the two stages it leaves free.
template <int D, typename E, int STG, bool DIAG, bool STRIDED, bool LAST = false>
__device__ __forceinline__ void dkdv_step(f32x16* dva, f32x16* dka, const f16x8* kf,
                                          const vec8<E>* vf, const Ring& rg,
                                          const TileLoads<D, 64, 4>& ld, const OperandOffs<D>& of,
                                          const DkdvCtx<D, E, STRIDED>& x, int qt, int nqt,
                                          const TabSrc& tab = {}) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    constexpr int NXT = (STG + NS - 1) % NS;
    // tiles past the last query tile are never loaded (see dq_step)
    if (!LAST && qt + 1 < nqt) wait_vmcnt<(C::LPT + 1) * (NS - 2)>();
    else wait_vmcnt<0>();
    ring_barrier();
    if constexpr (LAST) {
        static_assert(NS == 3, "the last step's free stages");
        constexpr int A = (STG + 1) % NS, B = (STG + 2) % NS;
        stage_tables<D>(tab.cs, tab.sn, tab.r0, x.T, rg.k[A], rg.v[A], rg.k[B], rg.v[B], x.wave,
                        x.lane);
    } else if (qt + NS - 1 < nqt) {
        x.issue(ld, qt + NS - 1, rg.k[NXT], rg.v[NXT], rg.x[NXT]);
    }
    dkdv_tile<D, E, DIAG>(dva, dka, kf, vf, rg.k[STG], rg.v[STG],
                       reinterpret_cast<const float*>(rg.x[STG]), of, qt * C::QN, x.wk0, x.lane);
}

// dk/dv item: the 128 keys of key block kb of head bh (loops over query tiles
// from the diagonal down; rg.k / rg.v / rg.x hold Q / dO tiles and offsets).
template <int D, typename E, bool STRIDED>
__device__ __forceinline__ void dkdv_item(const BwdPtrs<E>& pp, const Ring& rg, int bh, int kb) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    const int T = pp.T, BH = pp.BH;
    const f16* __restrict__ qr = pp.qr;
    const f16* __restrict__ kr = pp.kr;
    const E* __restrict__ v = pp.v;
    const E* __restrict__ dO = pp.dO;
    const float* __restrict__ ws = pp.ws;
    const float* __restrict__ cs = pp.cs;
    const float* __restrict__ sn = pp.sn;
    E* __restrict__ dk = pp.dk;
    E* __restrict__ dv = pp.dv;
    const float scale = kLn2;  // dK^r = s dS^T Q^r = ln 2 * dS^T (log2(e) s Q^r)
    const int k0 = kb * C::KM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const uint32_t hbytes = (uint32_t)T * D * 2;
    const int wk0 = k0 + wave * 32;
    const int tk = wk0 + c32;
    // v, dO, dk and dv: [B, H, T, D] unless STRIDED (then where their layouts put them)
    const int vst = STRIDED ? pp.lv.st : D;
    const long long vhead = STRIDED ? pp.lv.head(bh, pp.H) : (long long)hoff;
    const DkdvCtx<D, E, STRIDED> x = {qr + hoff, dO + (STRIDED ? pp.lo.head(bh, pp.H) : (long long)hoff),
                             ws + (size_t)(wave >> 1) * BH * T + (size_t)bh * T,
                             STRIDED ? pp.lo.st : D, T, wk0, lane, wave};
    const TileLoads<D, 64, 4> ld(wave, lane);
    const OperandOffs<D> of(lane);

    const int qt0 = k0 / C::QN;
    const int nqt = (T + C::QN - 1) / C::QN;
    const int qfull = min(nqt, (k0 + C::KM) / C::QN);  // from here on no query precedes a key
    // tile qt0, this lane's key and value, then tiles qt0+1 .. qt0+NS-2; the
    // first step waits for tile qt0 and the key and value only
    x.issue(ld, qt0, rg.k[0], rg.v[0], rg.x[0]);
    const rsrc_t kbuf = make_rsrc(kr + hoff, hbytes);
    const rsrc_t vbuf = make_rsrc(v + vhead, STRIDED ? pp.lv.head_bytes(T, D) : hbytes);
    f16x8 kf[C::DK];
    vec8<E> vf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) {
        const uint32_t col = (uint32_t)(16 * c + 8 * hf) * 2;
        kf[c] = __builtin_bit_cast(f16x8, buf_load16(kbuf, (uint32_t)tk * D * 2 + col));
        vf[c] = as_vec8<vec8<E>>(buf_load16(vbuf, (uint32_t)tk * vst * 2 + col));
    }
#pragma unroll
    for (int s = 1; s < NS - 1; ++s)
        if (qt0 + s < nqt) x.issue(ld, qt0 + s, rg.k[s], rg.v[s], rg.x[s]);
    f32x16 dva[C::DB], dka[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dva[b] = dka[b] = f32x16{};

    // ring stage of query tile qt is (qt - qt0) % NS; the diagonal tiles come
    // first. With three stages the last step is peeled off (it copies the RoPE
    // table rows for the epilogue into LDS), so the loops stop before it.
    constexpr bool TAB = NS == 3;
    const int qlast = TAB ? nqt - 1 : nqt;
    int qt = qt0;
    {
        // straight-line steps with compile-time stages wherever the stage is
        // known (see dq_item): the diagonal tiles (at most two, stages 0 and 1),
        // then full tiles up to the next stage 0
        static_assert(C::KM / C::QN == 2, "two diagonal query tiles per key block");
        const int qd = min(qfull, qlast);
        if (qt < qd) {
            dkdv_step<D, E, 0, true, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
            ++qt;
        }
        if (qt < qd) {
            dkdv_step<D, E, 1, true, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
            ++qt;
        }
        if (qt < qlast && qt - qt0 == 1) {
            dkdv_step<D, E, 1, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
            ++qt;
        }
        if constexpr (NS > 2) {
            if (qt < qlast && qt - qt0 == 2) {
                dkdv_step<D, E, 2, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
                ++qt;
            }
        }
    }
    for (; qt + NS <= qlast; qt += NS) {
        dkdv_step<D, E, 0, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
        dkdv_step<D, E, 1, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt + 1, nqt);
        if constexpr (NS > 2) dkdv_step<D, E, 2, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt + 2, nqt);
    }
    // at most NS-1 full tiles remain, from stage 0
    if (qt < qlast) {
        dkdv_step<D, E, 0, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
        ++qt;
    }
    if constexpr (NS > 2) {
        if (qt < qlast) {
            dkdv_step<D, E, 1, false, STRIDED>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt);
            ++qt;
        }
    }
    if constexpr (TAB) {
        // the last step (it may also be a diagonal one: the diagonal variant
        // gives the same result on a full tile) and the epilogue, with the last
        // step's ring stage L a compile-time constant
        const TabSrc tab = {cs, sn, k0};
        const int stg = (qt - qt0) % NS;
        static_for<NS>([&](auto S) {
            constexpr int L = decltype(S)::value;
            if (stg != L) return;
            dkdv_step<D, E, L, true, STRIDED, true>(dva, dka, kf, vf, rg, ld, of, x, qt, nqt, tab);
            wait_vmcnt<0>();
            __syncthreads();  // the table rows have landed and every wave is done with the ring
            // the table rows sit in the two stages after L; stage L itself (16 KB)
            // stages the output rows, 4 KB per wave: dk, then dv in the same place
            // (one wave's own LDS accesses stay in program order)
            constexpr int A = (L + 1) % NS, B = (L + 2) % NS;
            const bool h = wave >= 2;
            RowTables<D> tb;
            tb.load_lds(h ? rg.v[A] : rg.k[A], h ? rg.v[B] : rg.k[B], 32 * (wave & 1) + c32, hf);
            const RowStage<D> sg = {(h ? rg.v[L] : rg.k[L]) + (wave & 1) * 32 * 2 * D};
            rope_out<D, E>(dka, scale, tb, sg, dk + vhead, wk0, T, vst, c32, hf, lane);
            plain_out<D, E>(dva, sg, dv + vhead, wk0, T, vst, c32, hf, lane);
        });
    } else {
        RowTables<D> tb;
        tb.load(cs, sn, tk, T, hf);
        wait_vmcnt<0>();
        __syncthreads();  // the ring is idle: its stage buffers hold the output rows
        const RowStage<D> sk = {stage_buffer<D>(rg, wave)};
        const RowStage<D> sv = {sk.buf + 32 * 2 * D};
        rope_out<D, E>(dka, scale, tb, sk, dk + vhead, wk0, T, vst, c32, hf, lane);
        plain_out<D, E>(dva, sv, dv + vhead, wk0, T, vst, c32, hf, lane);
    }
}

// The gradient kernel: one launch runs both kinds of item, so the light items
// of one kind fill the gaps left by the other and there is a single tail.
// Item classes alternate dk/dv key block r and dq q-block nqb-1-r
// (r = 0, 1, ...), which is heaviest first up to the 4:3 ratio of their
// products per tile; each class holds one item per head. Workgroup i runs item
// i: the grid is several times the resident slots, and once the first ones are
// placed the dispatcher hands the next workgroup id to whichever slot frees
// first, so ids in falling order of work are longest-first list scheduling
// (the forward's round reversal would start light items before heavy ones).
template <int D, typename E, bool STRIDED>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd16_kernel(BwdPtrs<E> pp, int nqb,
                                                                         int nkb, int kinds) {
    using C = BwdTile<D>;
    constexpr int NS = C::NS;
    constexpr int T3 = NS > 2 ? C::TILE : 1024;
    // one __shared__ object per ring stage (see Ring); both kinds use the same ones
    __shared__ __attribute__((aligned(1024))) char a0[C::TILE], a1[C::TILE], a2[T3];
    __shared__ __attribute__((aligned(1024))) char b0[C::TILE], b1[C::TILE], b2[T3];
    __shared__ __attribute__((aligned(512))) char x0[512], x1[512], x2[512];
    const Ring rg = {{a0, a1, a2}, {b0, b1, b2}, {x0, x1, x2}};

    // kinds: 1 = dq items only, 2 = dk/dv items only, 3 = both
    const int per = kinds == 3 ? 2 : 1;
    const int item = blockIdx.x;
    const int c = item / pp.BH, bh = item % pp.BH;
    const int r = c / per;
    const bool is_dkdv = kinds == 2 || (kinds == 3 && (c % 2) == 0);
    if (is_dkdv) {
        if (r < nkb) dkdv_item<D, E, STRIDED>(pp, rg, bh, r);
    } else {
        if (r < nqb) dq_item<D, E, STRIDED>(pp, rg, bh, nqb - 1 - r);
    }
}

template <int D, typename E>
static hipError_t launch_grads(const BwdArgs& a, int kinds) {
    using C = BwdTile<D>;
    const size_t n = (size_t)a.B * a.H * a.T * a.D;
    const f16* rot = static_cast<const f16*>(a.rot);
    const BwdPtrs<E> pp = {rot,        rot + n,    (const E*)a.v, (const E*)a.dO, a.ws,
                           a.cs,       a.sn,       (E*)a.dq,      (E*)a.dk,       (E*)a.dv,
                           a.lqkv,     a.lo,       a.H,           a.B * a.H,      a.T};
    const int nqb = (a.T + C::QM - 1) / C::QM;
    const int nkb = (a.T + C::KM - 1) / C::KM;
    const int per = kinds == 3 ? 2 : 1;
    const int items = per * (nqb > nkb ? nqb : nkb) * a.B * a.H;
    // row pitch D for both means plain [B, H, T, D] (see Layout)
    if (a.lqkv.st != a.D || a.lo.st != a.D)
        hipLaunchKernelGGL((bwd16_kernel<D, E, true>), dim3(items), dim3(C::NT), 0, a.stream, pp,
                           nqb, nkb, kinds);
    else
        hipLaunchKernelGGL((bwd16_kernel<D, E, false>), dim3(items), dim3(C::NT), 0, a.stream, pp,
                           nqb, nkb, kinds);
    return hipGetLastError();
}

hipError_t launch_bwd_grads16(const BwdArgs& a, bool f16_storage) {
    if (f16_storage) return a.D == 64 ? launch_grads<64, f16>(a, 3) : launch_grads<128, f16>(a, 3);
    return a.D == 64 ? launch_grads<64, bf16>(a, 3) : launch_grads<128, bf16>(a, 3);
}

}  // namespace attn
