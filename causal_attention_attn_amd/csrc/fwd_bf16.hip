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
//   * the K rows are fed in the key_perm order, which makes the rounded
//     probabilities directly the B operand of O^T += V^T P^T;
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

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ cs, const float* __restrict__ sn, bf16* __restrict__ o,
    float* __restrict__ lse, int BH, int T, int nqb, float sc) {
    using C = FwdTile<D>;
    __shared__ __attribute__((aligned(16))) f16 Ks[C::BN * C::KS];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * C::VS];

    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = nqb - 1 - bid / BH;
    const int q0 = qb * C::BM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, hf = lane >> 5;
    const size_t hoff = (size_t)bh * T * D;
    const bf16* qh = q + hoff;
    const bf16* kh = k + hoff;
    const bf16* vh = v + hoff;
    const int wq0 = q0 + wave * 32;
    const int tq = wq0 + c32;

    f16x8 qf[C::DK];
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = load_rope8<D, f16>(qh, tq, 16 * c + 8 * hf, cs, sn, T);

    f32x16 oacc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const int kend = min(T, q0 + C::BM);
    const int ntiles = (kend + C::BN - 1) / C::BN;
    const int kp = key_perm(c32);

    for (int n = 0; n < ntiles; ++n) {
        const int k0 = n * C::BN;
        __syncthreads();
        stage_rows<D, C::BN, C::NT, true, f16, void>(kh, k0, T, cs, sn, Ks, nullptr, tid);
        stage_rows<D, C::BN, C::NT, false, void, bf16>(vh, k0, T, cs, sn, nullptr, Vt, tid);
        __syncthreads();

        if (k0 > wq0) continue;  // whole tile above this wave's diagonal

        f32x16 s[C::NSB];
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
            const int kb = k0 + 32 * sb;
            if (kb > wq0) break;
            f32x16 acc = f32x16{};
            const f16* krow = Ks + (32 * sb + kp) * C::KS + 8 * hf;
#pragma unroll
            for (int c = 0; c < C::DK; ++c)
                acc = mfma32(*reinterpret_cast<const f16x8*>(krow + 16 * c), qf[c], acc);
            if (kb == wq0) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (item_row(i, hf) > c32) acc[i] = -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
            s[sb] = acc;
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run, mx * sc);
        const float alpha = exp2_fast(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) oacc[b] *= alpha;

        float lsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
            const int kb = k0 + 32 * sb;
            if (kb > wq0) break;
            bf16x8 pb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = exp2_fast(fmaf(s[sb][8 * j + 2 * e], sc, -mnew));
                    const float p1 = exp2_fast(fmaf(s[sb][8 * j + 2 * e + 1], sc, -mnew));
                    lsum += p0 + p1;
                    w[e] = pack_bf16x2(p0, p1);
                }
                pb[j] = as_bf16x8(w);
            }
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const bf16* vrow = Vt + (32 * b + c32) * C::VS + 32 * sb + 8 * hf;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    oacc[b] = mfma32(*reinterpret_cast<const bf16x8*>(vrow + 16 * j), pb[j], oacc[b]);
            }
        }
        l_run += lsum;
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (tq < T) {
        const float inv = 1.f / l_tot;
        bf16* orow = o + hoff + (size_t)tq * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * g + 4 * hf) = w;
            }
        }
        if (hf == 0) lse[(size_t)bh * T + tq] = (m_run + log2f(l_tot)) * kLn2;
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
