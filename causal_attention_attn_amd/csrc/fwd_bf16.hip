// Forward pass of causal RoPE attention, bf16 storage / fp32 accumulation, gfx950.
//
// FlashAttention-style exact attention ("Show HN: NanoEuler", paragraph 2): the
// score matrix is produced tile by tile in registers, a running row maximum and
// row sum implement the softmax online, and only o and the per-row log-sum-exp
// reach HBM. RoPE ("Tiny Hackable CUDA", section 3) is applied while q and k are
// loaded. Causality (keys u <= query t) is enforced by skipping every 32x32 block
// that lies wholly above the diagonal and masking only the diagonal blocks.
//
// Work decomposition (one workgroup = 4 waves = 128 queries of one head):
//   * each wave owns 32 queries; its rotated queries live in registers as the
//     B operand of S^T = K Q^T (v_mfma_f32_32x32x16_f16, k = head dim);
//   * 64-key tiles of rotated K (row-major) and of V (transposed, [d][key]) are
//     staged in LDS and shared by the four waves;
//   * rotated q and k are no longer bf16 values, so they are rounded once to
//     fp16 (11-bit significand) for the score product: the softmax turns score
//     errors into relative weight errors, and with bf16 operands they reach
//     ~3e-2 on O for logits of standard deviation ~9. P and V stay bf16
//     (v_mfma_f32_32x32x16_bf16). fp16 bounds |rotated q|, |rotated k| by 65504;
//   * S^T puts one query per lane column, so each lane owns one query's running
//     max/sum and only one cross-lane exchange (lane ^ 32) is needed per tile;
//   * V is stored transposed with its key columns in col_perm order, so the
//     rounded probabilities of S^T are directly the B operand of
//     O^T += V^T P^T and each A operand is one 16-byte LDS read;
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
    static constexpr int BM = 128;     // queries per workgroup
    static constexpr int BN = 64;      // keys per LDS tile
    static constexpr int NT = 256;     // threads per workgroup
    static constexpr int DK = D / 16;  // MFMA k-chunks over the head dimension
    static constexpr int DB = D / 32;  // 32-row blocks of the head dimension
    static constexpr int KS = D + 8;   // LDS row stride of the K tile (elements)
    static constexpr int VS = BN + 8;  // LDS row stride of the transposed V tile
    static constexpr int NSB = BN / 32;
};

// Running state of one lane's query: O^T accumulator (this lane's half of the
// head dimension), reference maximum m (log2 units) and partial row sum l.
template <int D>
struct FwdState {
    f32x16 o[D / 32];
    float m, l;
};

// One 64-key tile for one wave. DIAG: the tile may reach this wave's diagonal,
// so 32-key sub-blocks above it are skipped and the diagonal one is masked.
template <int D, bool DIAG>
__device__ __forceinline__ void fwd_tile(FwdState<D>& st, const f16x8* qf, const f16* ks,
                                         const bf16* vt, int k0, int wq0, int c32, int hf,
                                         float sc) {
    using C = FwdTile<D>;
    constexpr float kRescale = 8.f;
    f32x16 s[C::NSB];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
        const f16* krow = ks + (32 * sb + c32) * C::KS + 8 * hf;
        f32x16 acc = mfma32(*reinterpret_cast<const f16x8*>(krow), qf[0], f32x16{});
#pragma unroll
        for (int c = 1; c < C::DK; ++c)
            acc = mfma32(*reinterpret_cast<const f16x8*>(krow + 16 * c), qf[c], acc);
        s[sb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
        if (DIAG && k0 + 32 * sb == wq0) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (item_row(i, hf) > c32) s[sb][i] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[sb][i], s[sb][i + 1]));
    }
    mx = max_across_halves(mx) * sc;
    // the reference maximum only moves when the tile maximum exceeds it by more
    // than kRescale (log2 units), so the O/l rescale is rare; unnormalised
    // probabilities stay below 2^kRescale
    if (mx > st.m + kRescale) {
        const float alpha = exp2_fast(st.m - mx);
        st.m = mx;
        st.l *= alpha;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) st.o[b] *= alpha;
    }
    const float mneg = -st.m;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
        if (DIAG && k0 + 32 * sb > wq0) break;
        bf16x8 pb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = exp2_fast(fmaf(s[sb][8 * j + 2 * e], sc, mneg));
                const float p1 = exp2_fast(fmaf(s[sb][8 * j + 2 * e + 1], sc, mneg));
                st.l += p0 + p1;
                w[e] = pack_bf16x2(p0, p1);
            }
            pb[j] = as_bf16x8(w);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
            const bf16* vrow = vt + (32 * b + c32) * C::VS + 32 * sb + 8 * hf;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                st.o[b] = mfma32(*reinterpret_cast<const bf16x8*>(vrow + 16 * j), pb[j], st.o[b]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ cs, const float* __restrict__ sn, bf16* __restrict__ o,
    float* __restrict__ lse, int BH, int T, int nqb, float sc) {
    using C = FwdTile<D>;
    // two buffers of (rotated K row-major, V transposed); one barrier per tile
    __shared__ __attribute__((aligned(16))) f16 Ks[2][C::BN * C::KS];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * C::VS];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const HeadBufs<D> qb_(q + hoff, cs, sn, T), kb_(k + hoff, cs, sn, T), vb_(v + hoff, cs, sn, T);
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;

    const int kend = min(T, q0 + C::BM);
    const int ntiles = (kend + C::BN - 1) / C::BN;
    const int nfull = min(ntiles, q0 / C::BN);  // tiles wholly below every query of the block
    RowStage<D, C::BN, C::NT, true> kst;
    RowStage<D, C::BN, C::NT, false> vst;
    kst.load(kb_, 0, tid);
    vst.load(vb_, 0, tid);

    f16x8 qf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = rope_operand<D, f16>(qb_, tq, 16 * c + 8 * hf);

    FwdState<D> st;
#pragma unroll
    for (int b = 0; b < C::DB; ++b) st.o[b] = f32x16{};
    st.m = -INFINITY;
    st.l = 0.f;

    kst.template store<f16, void>(Ks[0], nullptr, tid);
    vst.template store<void, bf16>(nullptr, Vt[0], tid);
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
        const int k0 = n * C::BN;
        const int cur = n & 1;
        const bool more = n + 1 < ntiles;
        if (more) {
            kst.load(kb_, k0 + C::BN, tid);
            vst.load(vb_, k0 + C::BN, tid);
        }
        if (n < nfull)
            fwd_tile<D, false>(st, qf, Ks[cur], Vt[cur], k0, wq0, c32, hf, sc);
        else if (k0 <= wq0)
            fwd_tile<D, true>(st, qf, Ks[cur], Vt[cur], k0, wq0, c32, hf, sc);
        if (more) {
            kst.template store<f16, void>(Ks[cur ^ 1], nullptr, tid);
            vst.template store<void, bf16>(nullptr, Vt[cur ^ 1], tid);
        }
        __syncthreads();
    }

    const float l_tot = sum_across_halves(st.l);
    if (tq < T) {
        const float inv = 1.f / l_tot;
        bf16* orow = o + hoff + (size_t)tq * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(st.o[b][4 * g] * inv, st.o[b][4 * g + 1] * inv);
                w[1] = pack_bf16x2(st.o[b][4 * g + 2] * inv, st.o[b][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * g + 4 * hf) = w;
            }
        }
        if (hf == 0) lse[(size_t)bh * T + tq] = (st.m + log2f(l_tot)) * kLn2;
    }
}

template <int D>
static hipError_t launch_fwd(const FwdArgs& a) {
    using C = FwdTile<D>;
    const int BH = a.B * a.H;
    const int nqb = (a.T + C::BM - 1) / C::BM;
    const float sc = kLog2e / sqrtf((float)D);
    hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(nqb * BH), dim3(C::NT), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.cs, a.sn,
                       (bf16*)a.o, a.lse, BH, a.T, nqb, sc);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    return a.D == 64 ? launch_fwd<64>(a) : launch_fwd<128>(a);
}

}  // namespace attn
