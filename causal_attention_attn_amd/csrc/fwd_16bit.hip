// Forward pass of causal RoPE attention, 16-bit storage (bf16 or fp16, type E)
// with fp32 accumulation, gfx950.
//
// FlashAttention-style exact attention ("Show HN: NanoEuler", paragraph 2): the
// score matrix is produced tile by tile in registers, a running row maximum and
// row sum implement the softmax online, and only o and the per-row log-sum-exp
// reach HBM. RoPE ("Tiny Hackable CUDA", section 3: on the query and key
// projections) is applied on load, or has been applied by the rotation pass:
//   * RoPE on load (ROPE): each lane rotates its own query once, in registers,
//     and every 64-key tile goes global -> registers (raw keys and their cos/sin
//     rows) -> rotation in fp32 -> fp16 -> LDS, one step ahead of its use;
//   * rotated input: the rotation pass has written the rotated q, k (fp16), and
//     key tiles stream straight from global memory into LDS.
// Both form the same fp16 values (rope_chunk_f16), so both give the same o and
// lse bitwise. Causality (keys u <= query t) is enforced by skipping every
// 32x32 block wholly above the diagonal and masking only the diagonal blocks.
//
// Work decomposition (one workgroup = 4 waves = 128 queries of one head):
//   * each wave owns 32 queries; its rotated queries live in registers as the
//     B operand of S^T = K Q^T (v_mfma_f32_32x32x16_f16, k = head dim). The
//     rotated q and k are not bf16 values; fp16's 11-bit significand keeps the
//     score error small where the softmax is sharp (bf16 operands give ~3e-2
//     error on O for logits of standard deviation ~9). P and V are of the
//     storage type E (P is rounded to E before the PV product).
//   * 64-key tiles of V (E) - and of rotated K without ROPE - stream straight
//     from global memory into a three-stage LDS ring (buffer_load ... lds),
//     issued two tiles ahead of use; one barrier per tile both publishes a tile
//     and frees the oldest stage;
//   * S^T puts one query per lane column, so each lane owns one query's running
//     max/sum; the running maximum enters as the MFMA's initial accumulator, so
//     the per-element softmax work is exp2, rounding to E and a packed pair sum
//     (the exact tile maximum is only taken when the probabilities would leave
//     their bound, see fwd_softmax_pv);
//   * the rounded probabilities of S^T are directly the B operand of
//     O^T += V^T P^T; the V^T operand comes from the row-major V tile through
//     the LDS transpose read (ds_read_b64_tr_b16);
//   * tiles wholly below the block's first query take a branch-free path; only
//     the last one or two tiles check for skipped and masked 32-key blocks;
//   * workgroups are issued heaviest q-block first; consecutive block ids walk
//     the heads so that the q-blocks of one head share an XCD's L2 whenever
//     the head count is a multiple of the XCD count.
#include "device_common.h"
#include "launchers.h"

namespace attn {

template <int D>
struct FwdTile {
    static constexpr int BM = 128;      // queries per workgroup
    static constexpr int BN = 64;       // keys per LDS tile
    static constexpr int NT = 256;      // threads per workgroup
    static constexpr int NW = 4;        // waves per workgroup
    static constexpr int DK = D / 16;   // MFMA k-chunks over the head dimension
    static constexpr int DB = D / 32;   // 32-row blocks of the head dimension
    static constexpr int NSB = BN / 32;
    static constexpr int TILE = BN * D * 2;            // bytes of one K or V tile
    static constexpr int NS = 3;                       // LDS ring stages
    static constexpr int LPT = 2 * TILE / 1024 / NW;   // load instructions per wave per tile
};

// Running state of one lane's query: O^T accumulator (this lane's half of the
// head dimension), reference maximum m (log2 units), -m in every entry of an
// accumulator (the initial value of the score MFMAs) and the partial row sum l.
template <int D>
struct FwdState {
    f32x16 o[D / 32];
    f32x16 negm;
    float m, l;
};

// Probabilities p = 2^x of the tile's live 32-key blocks, rounded to E and
// packed as the B operand of O^T += V^T P^T; returns this lane's sum of the
// rounded values.
template <int D, typename E, bool DIAG>
__device__ __forceinline__ float fwd_probs(const f32x16* x, vec8<E> (*pb)[2], int k0, int wq0) {
    using C = FwdTile<D>;
    float part[C::NSB][2];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w;
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[e] = pack2<E>(exp2_fast(x[sb][8 * j + 2 * e]),
                                exp2_fast(x[sb][8 * j + 2 * e + 1]));
                a = add_pair<E>(w[e], a);
            }
            pb[sb][j] = as_vec8<vec8<E>>(w);
            part[sb][j] = a;
        }
    }
    float t = part[0][0] + part[0][1];
#pragma unroll
    for (int sb = 1; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
        t += part[sb][0] + part[sb][1];
    }
    return t;
}

// K operands of one 64-key tile for this lane: the A operands of the two
// 32-key score products, one per 16-wide chunk of the head dimension.
template <int D>
struct KOps {
    f16x8 a[FwdTile<D>::NSB][FwdTile<D>::DK];
};

template <int D>
__device__ __forceinline__ void read_k(KOps<D>& kr, const char* ks, const OperandOffs<D>& of) {
    using C = FwdTile<D>;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int c = 0; c < C::DK; ++c)
            kr.a[sb][c] = *reinterpret_cast<const f16x8*>(ks + 32 * sb * 2 * D + of.k[c]);
}

// Scores of one 64-key tile, x = S^T log2(e) - m (the query carries
// log2(e)/sqrt(D) and -m is the initial accumulator). DIAG: 32-key blocks
// above the wave's diagonal are skipped and the diagonal one is masked.
template <int D, bool DIAG>
__device__ __forceinline__ void fwd_scores(f32x16* x, const FwdState<D>& st, const f16x8* qf,
                                           const KOps<D>& kr, int k0, int wq0, int lane) {
    using C = FwdTile<D>;
    const int c32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
        f32x16 acc = mfma32(kr.a[sb][0], qf[0], st.negm);
#pragma unroll
        for (int c = 1; c < C::DK; ++c) acc = mfma32(kr.a[sb][c], qf[c], acc);
        x[sb] = acc;
        if (DIAG && k0 + 32 * sb == wq0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) > c32) x[sb][i] = -INFINITY;
        }
    }
}

// Online softmax and O^T += V^T P^T for one 64-key tile whose scores are x.
//
// The online softmax needs no per-tile maximum while the probabilities stay
// bounded: if every lane's sum of this tile's p = 2^x is at most 2^8, no single
// x exceeds 8, so O and l may keep the reference m (the bound on unnormalised
// probabilities is the same as a lazy rescale with threshold 8). Otherwise
// (and on the wave's first tile, which sets m) the exact maximum is taken, O
// and l are rescaled and the tile's probabilities are recomputed. The V^T
// operands are read from LDS first, so their latency overlaps the softmax.
template <int D, typename E, bool DIAG>
__device__ __forceinline__ void fwd_softmax_pv(FwdState<D>& st, f32x16* x, const char* vs,
                                               const OperandOffs<D>& of, int k0, int wq0,
                                               bool first) {
    using C = FwdTile<D>;
    constexpr float kLimit = 256.f;
    constexpr int ROWB = 2 * D;
    vec8<E> va[C::NSB][C::DB][2];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const char* vb = vs + (32 * sb + 16 * j) * ROWB;
                va[sb][b][j] = tr_pair<vec8<E>>(vb + of.v[b][0], vb + of.v[b][1]);
            }
    }
    vec8<E> pb[C::NSB][2];
    float ts = 0.f;
    bool slow = first;
    if (!first) {
        ts = fwd_probs<D, E, DIAG>(x, pb, k0, wq0);
        slow = wave_any(ts > kLimit);
    }
    if (slow) {
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
            if (DIAG && k0 + 32 * sb > wq0) break;
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(x[sb][i], x[sb][i + 1]));
        }
        mx = max_across_halves(mx);
        // first tile: every query sees key 0, so mx is finite and becomes m;
        // later tiles only move m up
        const float d = first ? mx : fmaxf(mx, 0.f);
        if (!first) {
            const float alpha = exp2_fast(-d);
            st.l *= alpha;
#pragma unroll
            for (int b = 0; b < C::DB; ++b) st.o[b] *= alpha;
        }
        st.m += d;
        st.negm = splat16(-st.m);
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
            if (DIAG && k0 + 32 * sb > wq0) break;
            x[sb] -= d;
        }
        ts = fwd_probs<D, E, DIAG>(x, pb, k0, wq0);
    }
    st.l += ts;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j) st.o[b] = mfma32(va[sb][b][j], pb[sb][j], st.o[b]);
    }
}

// Raw key rows of one 64-row tile and the RoPE table entries they need, held in
// registers from their load until they are rotated into the LDS ring (RoPE on
// load: the forward reads the caller's un-rotated k). Thread tid owns CPT = D/32
// 16-byte chunks: chunk cc = tid % NC of tile rows tid / NC + i * RSTEP. Loads go
// through buffer resources that end at row T, so rows past the sequence read as
// zeros (cos = sin = 0 rotates them to zero).
template <int D, typename E>
struct KRot {
    static constexpr int NC = D / 8;          // 16-byte chunks per row
    static constexpr int CPT = D / 32;        // chunks per thread
    static constexpr int RSTEP = 256 / NC;    // rows between a thread's chunks
    u32x4 raw[CPT];
    f32x4 c[CPT], s[CPT];

    // rows r0 .. r0+63 of a head whose rows are `pitch` elements apart
    __device__ __forceinline__ void load(const E* head, int pitch, const float* cs,
                                         const float* sn, int T, int r0, int tid) {
        const int rows = T > r0 ? T - r0 : 0;
        const rsrc_t kb = make_rsrc(head + (size_t)r0 * pitch,
                                    rows > 0 ? (uint32_t)((rows - 1) * pitch + D) * 2 : 0u);
        const rsrc_t cb = make_rsrc(cs + (size_t)r0 * (D / 2), (uint32_t)rows * (D / 2) * 4);
        const rsrc_t sb = make_rsrc(sn + (size_t)r0 * (D / 2), (uint32_t)rows * (D / 2) * 4);
        const int cc = tid % NC, r = tid / NC;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int rr = r + i * RSTEP;
            raw[i] = buf_load16(kb, (uint32_t)(rr * pitch + 8 * cc) * 2);
            c[i] = __builtin_bit_cast(f32x4, buf_load16(cb, (uint32_t)(rr * (D / 2) + 4 * cc) * 4));
            s[i] = __builtin_bit_cast(f32x4, buf_load16(sb, (uint32_t)(rr * (D / 2) + 4 * cc) * 4));
        }
    }

    // Rotate, round to fp16 and put the chunks at their swizzled LDS positions in
    // `tile`.
    __device__ __forceinline__ void store(char* tile, int tid) const {
        const int cc = tid % NC, r = tid / NC;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int rr = r + i * RSTEP;
            *reinterpret_cast<u32x4*>(tile + rr * (2 * D) + 16 * swz<D>(rr, cc)) =
                rope_chunk_f16<E>(raw[i], c[i], s[i], 1.f);
        }
    }
};

// Shared state of one workgroup's pass over its key tiles.
template <int D, typename E>
struct FwdCtx {
    const f16* kr;      // pre-rotated keys (ROPE = false)
    const E* k;         // un-rotated keys (ROPE = true)
    const E* v;
    const float *cs, *sn;
    int kst;            // elements between consecutive rows of k (ROPE)
    int vst;            // elements between consecutive rows of v
    int T, wq0, lane, wave, tid;
    int ntiles;  // key tiles of the block (no tile past the last one is loaded)
};

// Step n of the tile loop; tile n sits in ring stage STG = n % NS and its K
// operands are already in kr. Scores of tile n first; then (ROPE) rotate the raw
// rows of tile n+1, loaded one step earlier, into their stage; wait for tile
// n+1's V, publish both with the barrier (which also frees the stage of tile
// n-1, whose last reads were made before it) and start loading tile n+2 (V
// straight into LDS, K into registers; without ROPE both straight into LDS);
// finish tile n (its V operands are read before the softmax, which hides their
// latency) and read tile n+1's K operands while the PV products run.
template <int D, typename E, int STG, bool DIAG, bool STRIDED, bool ROPE>
__device__ __forceinline__ void fwd_step(FwdState<D>& st, const f16x8* qf, KOps<D>& kr,
                                         KRot<D, E>& kq, const Ring& rg,
                                         const TileLoads<D, 64, 4>& ld,
                                         const OperandOffs<D>& of, const FwdCtx<D, E>& x, int n) {
    using C = FwdTile<D>;
    constexpr int NS = C::NS;
    static_assert(NS == 3, "the loaders assume a three-stage ring");
    constexpr int NXT = (STG + 1) % NS;
    constexpr int FREE = (STG + NS - 1) % NS;
    const int k0 = n * C::BN;
    const bool live = !(DIAG && k0 > x.wq0);  // false: tile wholly above this wave's diagonal
    // RoPE on load at D = 128 holds 48 registers of raw key rows and tables per
    // thread; there the K operands are read when the step starts instead of one
    // step ahead (their 64 registers would push the kernel into heavy spills)
    constexpr bool KPF = !(ROPE && D == 128);
    if constexpr (!KPF) read_k(kr, rg.k[STG], of);
    f32x16 s[C::NSB];
    if (live) fwd_scores<D, DIAG>(s, st, qf, kr, k0, x.wq0, x.lane);
    if constexpr (ROPE) {
        if (!DIAG || n + 1 < x.ntiles) kq.store(rg.k[NXT], x.tid);
    }
    wait_vmcnt<0>();
    ring_barrier();
    const int nx = n + NS - 1;
    // full steps load unchecked: their tile nx lies past the block's last one
    // only for a ragged T, and is then read within the head or as zeros
    if (!DIAG || nx < x.ntiles) {
        if constexpr (ROPE) kq.load(x.k, x.kst, x.cs, x.sn, x.T, nx * C::BN, x.tid);
        else ld.issue(x.kr, x.T, nx * C::BN, rg.k[FREE], x.wave);
        if constexpr (STRIDED) ld.issue_strided(x.v, x.T, nx * C::BN, rg.v[FREE], x.wave, x.vst);
        else ld.issue(x.v, x.T, nx * C::BN, rg.v[FREE], x.wave);
    }
    if (live) fwd_softmax_pv<D, E, DIAG>(st, s, rg.v[STG], of, k0, x.wq0, n == 0);
    if constexpr (KPF) read_k(kr, rg.k[NXT], of);
}

// The forward kernel. ROPE: q and k are the caller's un-rotated tensors (layout
// lqk) and are rotated on load - each lane's query once, in registers, and every
// key tile on its way into LDS. Without ROPE, qr and kr hold the rotated values
// already (the rotation pass).
template <int D, typename E, bool STRIDED, bool ROPE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void fwd16_kernel(
    const f16* __restrict__ qr, const f16* __restrict__ kr, const E* __restrict__ q,
    const E* __restrict__ k, const float* __restrict__ cs, const float* __restrict__ sn,
    const E* __restrict__ v, E* __restrict__ o, float* __restrict__ lse, Layout lqk, Layout lv,
    Layout lo, int H, int BH, int T, int nqb, int ncu) {
    using C = FwdTile<D>;
    constexpr int NS = C::NS;
    // one __shared__ object per ring stage (see Ring); stages >= NS are stubs
#define ATTN_STAGE(i) \
    __shared__ __attribute__((aligned(256))) char k##i[i < NS ? C::TILE : 16]; \
    __shared__ __attribute__((aligned(256))) char v##i[i < NS ? C::TILE : 16];
    ATTN_STAGE(0) ATTN_STAGE(1) ATTN_STAGE(2) ATTN_STAGE(3)
    ATTN_STAGE(4) ATTN_STAGE(5) ATTN_STAGE(6) ATTN_STAGE(7)
#undef ATTN_STAGE
    const Ring rg = {{k0, k1, k2, k3, k4, k5, k6, k7}, {v0, v1, v2, v3, v4, v5, v6, v7}, {}};

    const int bid = snake_item(blockIdx.x, ncu, nqb * BH);
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;
    const int kend = min(T, q0 + C::BM);
    const int ntiles = (kend + C::BN - 1) / C::BN;
    const int nfull = min(ntiles, q0 / C::BN);  // tiles wholly below every query of the block
    // q, k and v: [B, H, T, D] unless STRIDED (then where their layouts put them)
    const long long qkhead = STRIDED ? lqk.head(bh, H) : (long long)hoff;
    const int qkst = STRIDED ? lqk.st : D;
    const FwdCtx<D, E> x = {kr + hoff, k + qkhead, v + (STRIDED ? lv.head(bh, H) : (long long)hoff),
                            cs, sn, qkst, STRIDED ? lv.st : D, T, wq0, lane, wave, tid, ntiles};
    const TileLoads<D, 64, 4> ld(wave, lane);
    const OperandOffs<D> of(lane);
    KRot<D, E> kq;

    // prologue: tile 0, this lane's query, then tile 1 (rows past T read as
    // zeros); the first step waits for tile 0 and the query only
    if constexpr (ROPE) kq.load(x.k, qkst, cs, sn, T, 0, tid);
    else ld.issue(x.kr, T, 0, rg.k[0], wave);
    if constexpr (STRIDED) ld.issue_strided(x.v, T, 0, rg.v[0], wave, x.vst);
    else ld.issue(x.v, T, 0, rg.v[0], wave);

    f16x8 qf[C::DK];
    if constexpr (ROPE) {
        // this lane's query, features 16c + 8hf .. +7 for c < DK, rotated by R_tq
        // and scaled by log2(e)/sqrt(D) in fp32, rounded once to fp16
        const float qs = kLog2e / sqrtf((float)D);
        const rsrc_t qh = make_rsrc(q + qkhead, (uint32_t)((T - 1) * qkst + D) * 2);
        const rsrc_t ch = make_rsrc(cs, (uint32_t)T * (D / 2) * 4);
        const rsrc_t sh = make_rsrc(sn, (uint32_t)T * (D / 2) * 4);
        u32x4 wq[C::DK];
        f32x4 cq[C::DK], sq[C::DK];
#pragma unroll
        for (int c = 0; c < C::DK; ++c) {
            const int col = 16 * c + 8 * hf;
            wq[c] = buf_load16(qh, (uint32_t)(tq * qkst + col) * 2);
            cq[c] = __builtin_bit_cast(f32x4, buf_load16(ch, (uint32_t)(tq * (D / 2) + col / 2) * 4));
            sq[c] = __builtin_bit_cast(f32x4, buf_load16(sh, (uint32_t)(tq * (D / 2) + col / 2) * 4));
        }
#pragma unroll
        for (int c = 0; c < C::DK; ++c)
            qf[c] = __builtin_bit_cast(f16x8, rope_chunk_f16<E>(wq[c], cq[c], sq[c], qs));
        // tile 0's keys into stage 0
        kq.store(rg.k[0], tid);
    } else {
        const rsrc_t qh = make_rsrc(qr + hoff, (uint32_t)T * D * 2);
#pragma unroll
        for (int c = 0; c < C::DK; ++c)
            qf[c] = __builtin_bit_cast(f16x8, buf_load16(qh, (uint32_t)(tq * D + 16 * c + 8 * hf) * 2));
    }

    if (1 < ntiles) {
        if constexpr (ROPE) kq.load(x.k, qkst, cs, sn, T, C::BN, tid);
        else ld.issue(x.kr, T, C::BN, rg.k[1], wave);
        if constexpr (STRIDED) ld.issue_strided(x.v, T, C::BN, rg.v[1], wave, x.vst);
        else ld.issue(x.v, T, C::BN, rg.v[1], wave);
    }

    FwdState<D> st;
#pragma unroll
    for (int b = 0; b < C::DB; ++b) st.o[b] = f32x16{};
    st.negm = f32x16{};
    st.m = 0.f;
    st.l = 0.f;

    // tile 0 published; its K operands in registers (tile 1's V, and with ROPE
    // its raw keys, may still be in flight)
    if (1 < ntiles) {
        if constexpr (ROPE) wait_vmcnt<C::LPT / 2 + 3 * KRot<D, E>::CPT>();
        else wait_vmcnt<C::LPT>();
    } else {
        wait_vmcnt<0>();
    }
    ring_barrier();
    KOps<D> kops;
    if constexpr (!(ROPE && D == 128)) read_k(kops, rg.k[0], of);

    int n = 0;
    // full tiles: branch-free bodies, ring stages as compile-time constants
    for (; n + NS <= nfull; n += NS)
        static_for<NS>([&](auto S) {
            fwd_step<D, E, S, false, STRIDED, ROPE>(st, qf, kops, kq, rg, ld, of, x, n + S);
        });
    // the rest (at most NS-1 full tiles, then the diagonal tiles)
    for (; n < ntiles; ++n) {
        const int stg = n % NS;
        static_for<NS>([&](auto S) {
            if (stg == S) fwd_step<D, E, S, true, STRIDED, ROPE>(st, qf, kops, kq, rg, ld, of, x, n);
        });
    }
    wait_vmcnt<0>();  // no LDS writes may land after this workgroup's LDS is released

    const float l_tot = sum_across_halves(st.l);
    if (tq < T) {
        const float inv = 1.f / l_tot;
        E* orow = STRIDED ? row_ptr(o + lo.head(bh, H), tq, lo.st) : o + hoff + (size_t)tq * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack2<E>(st.o[b][4 * g] * inv, st.o[b][4 * g + 1] * inv);
                w[1] = pack2<E>(st.o[b][4 * g + 2] * inv, st.o[b][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * g + 4 * hf) = w;
            }
        }
        if (hf == 0) lse[(size_t)bh * T + tq] = (st.m + log2f(l_tot)) * kLn2;
    }
}

// Explicit instantiations: the host pass does not always emit the launch stub of
// a kernel template with a 16-bit element-type argument on its own.
#define ATTN_FWD_INST(D_, E_, S_, R_)                                                            \
    template __global__ void fwd16_kernel<D_, E_, S_, R_>(                                       \
        const f16*, const f16*, const E_*, const E_*, const float*, const float*, const E_*, E_*, \
        float*, Layout, Layout, Layout, int, int, int, int, int);
#define ATTN_FWD_INST2(D_, E_, S_) ATTN_FWD_INST(D_, E_, S_, false) ATTN_FWD_INST(D_, E_, S_, true)
ATTN_FWD_INST2(64, bf16, false) ATTN_FWD_INST2(128, bf16, false)
ATTN_FWD_INST2(64, f16, false) ATTN_FWD_INST2(128, f16, false)
ATTN_FWD_INST2(64, bf16, true) ATTN_FWD_INST2(128, bf16, true)
ATTN_FWD_INST2(64, f16, true) ATTN_FWD_INST2(128, f16, true)
#undef ATTN_FWD_INST2
#undef ATTN_FWD_INST

template <int D, typename E, bool STRIDED, bool ROPE>
static void launch_fwd_t(const FwdArgs& a, int nqb, int BH) {
    using C = FwdTile<D>;
    const size_t n = (size_t)a.B * a.H * a.T * a.D;
    const f16* rot = static_cast<const f16*>(a.rot);
    hipLaunchKernelGGL((fwd16_kernel<D, E, STRIDED, ROPE>), dim3(nqb * BH), dim3(C::NT), 0,
                       a.stream, rot, rot ? rot + n : nullptr, (const E*)a.q, (const E*)a.k,
                       a.cs, a.sn, (const E*)a.v, (E*)a.o, a.lse, a.lqkv, a.lqkv, a.lo, a.H, BH,
                       a.T, nqb, device_cu_count());
}

// rot non-null: the rotated q, k are there (the rotation pass ran); otherwise
// the RoPE-on-load instance rotates the caller's q, k
template <int D, typename E, bool STRIDED>
static void launch_fwd_s(const FwdArgs& a, int nqb, int BH) {
    if (a.rot != nullptr) launch_fwd_t<D, E, STRIDED, false>(a, nqb, BH);
    else launch_fwd_t<D, E, STRIDED, true>(a, nqb, BH);
}

template <int D, typename E>
static hipError_t launch_fwd(const FwdArgs& a) {
    using C = FwdTile<D>;
    const int BH = a.B * a.H;
    const int nqb = (a.T + C::BM - 1) / C::BM;
    // row pitch D for both means plain [B, H, T, D] (see Layout)
    if (a.lqkv.st != a.D || a.lo.st != a.D) launch_fwd_s<D, E, true>(a, nqb, BH);
    else launch_fwd_s<D, E, false>(a, nqb, BH);
    return hipGetLastError();
}

hipError_t launch_fwd16(const FwdArgs& a, bool f16_storage) {
    if (f16_storage) return a.D == 64 ? launch_fwd<64, f16>(a) : launch_fwd<128, f16>(a);
    return a.D == 64 ? launch_fwd<64, bf16>(a) : launch_fwd<128, bf16>(a);
}

}  // namespace attn
