// Decode: one generation step of causal RoPE attention over a key/value cache,
// 16-bit storage (bf16 or fp16, type E), gfx950.
//
// The pages' model generates one token at a time and a position may attend only
// to itself and earlier positions, with RoPE on the query and key projections
// encoding relative position ("Tiny Hackable CUDA", section 3, causal attention
// paragraph). At generation step `pos` the new query is rotated by its own
// position and scored against the cached keys of positions 0 .. pos, each
// rotated once, by its own position, when it entered the cache.
//
// Cache (one caller buffer): K' = R_u k_u for every head and position, fp16
// [B, H, Tmax, D] (rotated in fp32 and rounded once, like the forward's rotated
// keys), followed by V, E [B, H, Tmax, D].
//
// A step reads (pos + 1) K' and V rows per head and does O(D) arithmetic per
// row: it is bound by memory, not by MFMA (one query row is no contraction
// worth a matrix core). The keys of a head are split into 64-key slices, one
// slice per wave: a wave loads its slice's K' and V rows with coalesced 16-byte
// loads (a row's 16-byte chunks on consecutive lanes), forms the scores with
// fp16 dot products against the rotated, log2(e)/sqrt(D)-scaled query, and keeps
// (max m, sum l, unnormalised o) of its slice. The slices of a head are then
// merged: M = max m_i, o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i and
// lse = (M + log2 L) ln 2. Two launch shapes:
//   with many heads (kHeadKernelMinHeads or more), one workgroup per head
//                   (decode_head_kernel): its waves take the head's slices
//                   and merge them through LDS, all in one launch;
//   with few heads, waves of all heads spread over the chip (partial kernel,
//                   partials to the workspace) and a combine kernel merges
//                   each head's slices.
#include "device_common.h"
#include "launchers.h"

namespace attn {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kSlice = 64;  // keys per wave (one partial result each)
// heads from which one workgroup per head (decode_head_kernel) is used
constexpr int kHeadKernelMinHeads = 64;
// waves per workgroup of decode_head_kernel at most (its registers: 16 waves of
// D = 64 or 8 of D = 128 fit a CU without spills)
template <int D>
constexpr int kHeadWaves() { return D == 64 ? 16 : 8; }

template <int D>
constexpr int partial_stride() { return D + 4; }  // o[D], m, l, 2 pad: 16-byte rows

// R_u k for one 16-byte chunk (4 feature pairs) of a key row, rounded once to fp16.
template <typename E>
__device__ __forceinline__ u32x4 rotate_key_chunk(u32x4 wk, f32x4 cv, f32x4 sv) {
    return rope_chunk_f16<E>(wk, cv, sv, 1.f);
}

// Append n tokens to the cache: K' rows R_u k_u (u = pos0 + i) rounded once to
// fp16, V rows copied. k and v are [B, H, n, D]. One thread per 8 features.
template <int D, typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(const E* __restrict__ k,
                                                        const E* __restrict__ v,
                                                        const float* __restrict__ cs,
                                                        const float* __restrict__ sn,
                                                        f16* __restrict__ kc, E* __restrict__ vc,
                                                        int n, int pos0, int Tmax,
                                                        long long chunks) {
    constexpr int NC = D / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= chunks) return;
    const int c = (int)(idx % NC);
    const long long row = idx / NC;  // over B*H*n source rows
    const int i = (int)(row % n);
    const long long bh = row / n;
    const int u = pos0 + i;
    const long long src = row * D + 8 * c;
    const long long dst = (bh * Tmax + u) * D + 8 * c;
    const u32x4 wk = *reinterpret_cast<const u32x4*>(k + src);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(v + src);
    const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + (long long)u * (D / 2) + 4 * c);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + (long long)u * (D / 2) + 4 * c);
    *reinterpret_cast<u32x4*>(kc + dst) = rotate_key_chunk<E>(wk, cv, sv);
    *reinterpret_cast<u32x4*>(vc + dst) = wv;
}

// One wave per (head, 64-key slice). Lane l holds 16-byte chunk l % NC of rows
// l / NC, l / NC + RPI, ... of the slice, for K' and for V. APPEND: the token at
// position pos is new (knew, vnew [B, H, D], pre-RoPE k): the cache is read up
// to pos - 1 only, and the wave whose slice holds pos rotates the new key,
// uses it and the new value directly, and writes both into cache row pos (no
// other wave reads that row).
template <int D, typename E, bool APPEND>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const E* __restrict__ q, f16* __restrict__ kc, E* __restrict__ vc,
    const float* __restrict__ cs, const float* __restrict__ sn, float* __restrict__ part,
    const E* __restrict__ knew, const E* __restrict__ vnew, int Tmax, int pos, int nsplit,
    int nwaves, float qs) {
    constexpr int NC = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / NC;       // rows per load instruction
    constexpr int NI = kSlice / RPI;   // load instructions per operand
    const int lane = threadIdx.x & 63;
    // = bh * nsplit + slice, uniform over the wave (its loads use scalar descriptors)
    const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (gw >= nwaves) return;                             // no barriers below
    const int bh = gw / nsplit, u0 = (gw % nsplit) * kSlice;
    const int cc = lane % NC, rl = lane / NC;

    // cache rows 0 .. pos of this head (0 .. pos - 1 when appending); rows past
    // them read as zeros
    const uint32_t bytes = (uint32_t)(APPEND ? pos : pos + 1) * D * 2;
    const rsrc_t kb = make_rsrc(kc + (size_t)bh * Tmax * D, bytes);
    const rsrc_t vb = make_rsrc(vc + (size_t)bh * Tmax * D, bytes);
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint32_t off = (uint32_t)((u0 + i * RPI + rl) * D + 8 * cc) * 2;
        kr[i] = buf_load16(kb, off);
        vr[i] = buf_load16(vb, off);
    }

    // this lane's chunk of the query: R_pos q scaled by log2(e)/sqrt(D), fp16
    const u32x4 wq = *reinterpret_cast<const u32x4*>(q + (size_t)bh * D + 8 * cc);
    const f32x4 c4 = *reinterpret_cast<const f32x4*>(cs + (size_t)pos * (D / 2) + 4 * cc);
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(sn + (size_t)pos * (D / 2) + 4 * cc);
    const u32x4 rq = rope_chunk_f16<E>(wq, c4, s4, qs);
    f16x2 qh[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t w = rq[p];  // a plain value: bit_cast of a vector element reads element 0
        qh[p] = __builtin_bit_cast(f16x2, w);
    }
    if constexpr (APPEND) {
        if (pos - u0 < kSlice) {  // uniform: this wave's slice holds the new row
            const int r = pos - u0;
            if (rl == r % RPI) {
                const size_t cell = ((size_t)bh * Tmax + pos) * D + 8 * cc;
                const u32x4 kn = rotate_key_chunk<E>(
                    *reinterpret_cast<const u32x4*>(knew + (size_t)bh * D + 8 * cc), c4, s4);
                const u32x4 vn = *reinterpret_cast<const u32x4*>(vnew + (size_t)bh * D + 8 * cc);
                *reinterpret_cast<u32x4*>(kc + cell) = kn;
                *reinterpret_cast<u32x4*>(vc + cell) = vn;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    if (i == r / RPI) {
                        kr[i] = kn;
                        vr[i] = vn;
                    }
                }
            }
        }
    }

    // scores in log2 units; the NC lanes of a row add their chunks' dot products
    float s[NI];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t kw = kr[i][p];  // a plain value: bit_cast of a vector element reads element 0
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kw), qh[p], acc, false);
        }
#pragma unroll
        for (int x = 1; x < NC; x <<= 1) acc += __shfl_xor(acc, x);
        s[i] = u0 + i * RPI + rl <= pos ? acc : -INFINITY;
        m = fmaxf(m, s[i]);
    }
#pragma unroll
    for (int x = NC; x < 64; x <<= 1) m = fmaxf(m, __shfl_xor(m, x));

    // p = 2^(s - m) (0 for rows past pos); l and o over this lane's rows
    float l = 0.f;
    float o[8] = {};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const float p = exp2_fast(s[i] - m);
        l += p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2 x = unpack2<E>(vr[i][e]);
            o[2 * e] += p * x[0];
            o[2 * e + 1] += p * x[1];
        }
    }
    // sum over the rows: the lanes that share chunk cc
#pragma unroll
    for (int x = NC; x < 64; x <<= 1) {
        l += __shfl_xor(l, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] += __shfl_xor(o[j], x);
    }
    float* dst = part + (size_t)gw * partial_stride<D>();
    if (rl == 0) {
        *reinterpret_cast<f32x4*>(dst + 8 * cc) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(dst + 8 * cc + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
    if (lane == 0) {
        dst[D] = m;
        dst[D + 1] = l;
    }
}

// Merge a head's slices; one thread per feature. Slices are taken CH at a time
// with all their loads issued together (one memory round trip per group; a
// loop with one dependent load per slice would pay the latency nsplit times),
// and merged online: the running sums are rescaled when the maximum grows.
template <int D, typename E>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part,
                                                           E* __restrict__ o,
                                                           float* __restrict__ lse, int nsplit) {
    constexpr int PS = partial_stride<D>();
    constexpr int CH = 32;
    const int bh = blockIdx.x, d = threadIdx.x;
    const float* P = part + (size_t)bh * nsplit * PS;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int c0 = 0; c0 < nsplit; c0 += CH) {
        float mi[CH], li[CH], oi[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int i = min(c0 + j, nsplit - 1);  // past the end: a repeat, skipped below
            mi[j] = P[i * PS + D];
            li[j] = P[i * PS + D + 1];
            oi[j] = P[i * PS + d];
        }
        float cm = M;
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (c0 + j < nsplit) cm = fmaxf(cm, mi[j]);
        const float r = exp2_fast(M - cm);  // 0 on the first group (M = -inf, cm finite)
        L *= r;
        O *= r;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (c0 + j < nsplit) {
                const float w = exp2_fast(mi[j] - cm);
                L += w * li[j];
                O += w * oi[j];
            }
        }
        M = cm;
    }
    o[(size_t)bh * D + d] = static_cast<E>(O / L);
    if (d == 0) lse[bh] = (M + log2f(L)) * kLn2;
}

// One workgroup per head, one wave per 64-key slice (a wave takes slices w,
// w + W, ... when a head has more than W = blockDim / 64 of them): every wave
// keeps the running (max, sum, unnormalised o) of its slices, rescaling them when
// its maximum grows, and the waves' results are merged through LDS by the same
// workgroup - the whole step in one launch, without the partials' round trip
// through memory. Used when there are enough heads to spread over the CUs.
template <int D, typename E, bool APPEND>
__global__ __launch_bounds__(64 * kHeadWaves<D>()) void decode_head_kernel(
    const E* __restrict__ q, f16* __restrict__ kc, E* __restrict__ vc,
    const float* __restrict__ cs, const float* __restrict__ sn, E* __restrict__ o,
    float* __restrict__ lse, const E* __restrict__ knew, const E* __restrict__ vnew, int Tmax,
    int pos, int nsplit, float qs) {
    constexpr int NC = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / NC;       // rows per load instruction
    constexpr int NI = kSlice / RPI;   // load instructions per operand
    constexpr int PS = partial_stride<D>();
    __shared__ float sp[kHeadWaves<D>() * PS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int bh = blockIdx.x;
    const int cc = lane % NC, rl = lane / NC;
    const uint32_t bytes = (uint32_t)(APPEND ? pos : pos + 1) * D * 2;
    const rsrc_t kb = make_rsrc(kc + (size_t)bh * Tmax * D, bytes);
    const rsrc_t vb = make_rsrc(vc + (size_t)bh * Tmax * D, bytes);
    // the K' and V rows of a slice: rows past the buffers' ends read as zeros
    u32x4 kr[NI], vr[NI];
    auto load_slice = [&](int u0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t off = (uint32_t)((u0 + i * RPI + rl) * D + 8 * cc) * 2;
            kr[i] = buf_load16(kb, off);
            vr[i] = buf_load16(vb, off);
        }
    };
    // the wave's first slice is requested before the query (a wave without
    // slices reads zeros and never uses them), so the two loads share one
    // memory round trip instead of taking two in turn
    load_slice(wave * kSlice);
    __builtin_amdgcn_sched_barrier(0);

    // this lane's chunk of the query: R_pos q scaled by log2(e)/sqrt(D), fp16
    const u32x4 wq = *reinterpret_cast<const u32x4*>(q + (size_t)bh * D + 8 * cc);
    const f32x4 c4 = *reinterpret_cast<const f32x4*>(cs + (size_t)pos * (D / 2) + 4 * cc);
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(sn + (size_t)pos * (D / 2) + 4 * cc);
    const u32x4 rq = rope_chunk_f16<E>(wq, c4, s4, qs);
    f16x2 qh[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t w = rq[p];  // a plain value: bit_cast of a vector element reads element 0
        qh[p] = __builtin_bit_cast(f16x2, w);
    }

    float M = -INFINITY, l = 0.f;  // M: the wave's running maximum (uniform)
    float oa[8] = {};
    for (int sl = wave; sl < nsplit; sl += nw) {
        const int u0 = sl * kSlice;
        if (sl != wave) load_slice(u0);
        if constexpr (APPEND) {
            if (pos - u0 < kSlice) {  // uniform: this slice holds the new row
                const int r = pos - u0;
                if (rl == r % RPI) {
                    const size_t cell = ((size_t)bh * Tmax + pos) * D + 8 * cc;
                    const u32x4 kn = rotate_key_chunk<E>(
                        *reinterpret_cast<const u32x4*>(knew + (size_t)bh * D + 8 * cc), c4, s4);
                    const u32x4 vn =
                        *reinterpret_cast<const u32x4*>(vnew + (size_t)bh * D + 8 * cc);
                    *reinterpret_cast<u32x4*>(kc + cell) = kn;
                    *reinterpret_cast<u32x4*>(vc + cell) = vn;
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        if (i == r / RPI) {
                            kr[i] = kn;
                            vr[i] = vn;
                        }
                    }
                }
            }
        }
        float s[NI];
        float m = M;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t kw = kr[i][p];
                acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kw), qh[p], acc, false);
            }
#pragma unroll
            for (int x = 1; x < NC; x <<= 1) acc += __shfl_xor(acc, x);
            s[i] = u0 + i * RPI + rl <= pos ? acc : -INFINITY;
            m = fmaxf(m, s[i]);
        }
#pragma unroll
        for (int x = NC; x < 64; x <<= 1) m = fmaxf(m, __shfl_xor(m, x));
        // m is finite: every slice holds row u0 <= pos
        const float alpha = exp2_fast(M - m);  // 0 on the wave's first slice
        l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) oa[j] *= alpha;
        M = m;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float p = exp2_fast(s[i] - m);
            l += p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x2 x = unpack2<E>(vr[i][e]);
                oa[2 * e] += p * x[0];
                oa[2 * e + 1] += p * x[1];
            }
        }
    }
    // sums over the wave's rows: the lanes that share chunk cc
#pragma unroll
    for (int x = NC; x < 64; x <<= 1) {
        l += __shfl_xor(l, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) oa[j] += __shfl_xor(oa[j], x);
    }
    float* dst = sp + wave * PS;
    if (rl == 0) {
        *reinterpret_cast<f32x4*>(dst + 8 * cc) = f32x4{oa[0], oa[1], oa[2], oa[3]};
        *reinterpret_cast<f32x4*>(dst + 8 * cc + 4) = f32x4{oa[4], oa[5], oa[6], oa[7]};
    }
    if (lane == 0) {
        dst[D] = M;  // -inf for a wave without slices (its weight below is 0)
        dst[D + 1] = l;
    }
    __syncthreads();
    float Mx = -INFINITY;
    for (int w = 0; w < nw; ++w) Mx = fmaxf(Mx, sp[w * PS + D]);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float L = 0.f, O = 0.f;
        for (int w = 0; w < nw; ++w) {
            const float r = exp2_fast(sp[w * PS + D] - Mx);
            L += r * sp[w * PS + D + 1];
            O += r * sp[w * PS + d];
        }
        o[(size_t)bh * D + d] = static_cast<E>(O / L);
        if (d == 0) lse[bh] = (Mx + log2f(L)) * kLn2;
    }
}

// Explicit instantiations: the host pass does not always emit the launch stub of
// a kernel template with a 16-bit element-type argument on its own.
#define ATTN_DEC_INST(D_, E_)                                                                \
    template __global__ void kv_append_kernel<D_, E_>(const E_*, const E_*, const float*,      \
                                                      const float*, f16*, E_*, int, int, int,  \
                                                      long long);                              \
    template __global__ void decode_partial_kernel<D_, E_, false>(                            \
        const E_*, f16*, E_*, const float*, const float*, float*, const E_*, const E_*, int, int, \
        int, int, float);                                                                      \
    template __global__ void decode_partial_kernel<D_, E_, true>(                             \
        const E_*, f16*, E_*, const float*, const float*, float*, const E_*, const E_*, int, int, \
        int, int, float);                                                                      \
    template __global__ void decode_combine_kernel<D_, E_>(const float*, E_*, float*, int);    \
    template __global__ void decode_head_kernel<D_, E_, false>(                                \
        const E_*, f16*, E_*, const float*, const float*, E_*, float*, const E_*, const E_*, int, \
        int, int, float);                                                                      \
    template __global__ void decode_head_kernel<D_, E_, true>(                                 \
        const E_*, f16*, E_*, const float*, const float*, E_*, float*, const E_*, const E_*, int, \
        int, int, float);
ATTN_DEC_INST(64, bf16) ATTN_DEC_INST(128, bf16) ATTN_DEC_INST(64, f16) ATTN_DEC_INST(128, f16)
#undef ATTN_DEC_INST

int decode_slices(int pos) { return (pos + kSlice) / kSlice; }

size_t decode_workspace_floats(int B, int H, int Tmax, int D) {
    return (size_t)B * H * decode_slices(Tmax - 1) * (D + 4);
}

template <int D, typename E>
static hipError_t launch_append_t(const void* k, const void* v, const float* cs,
                                  const float* sn, void* cache, int pos0, int n, int B, int H,
                                  int Tmax, hipStream_t st) {
    const long long chunks = (long long)B * H * n * (D / 8);
    const size_t kbytes = (size_t)B * H * Tmax * D * 2;
    f16* kc = static_cast<f16*>(cache);
    E* vc = reinterpret_cast<E*>(static_cast<char*>(cache) + kbytes);
    hipLaunchKernelGGL((kv_append_kernel<D, E>), dim3((unsigned)((chunks + 255) / 256)),
                       dim3(256), 0, st, (const E*)k, (const E*)v, cs, sn, kc, vc, n, pos0, Tmax,
                       chunks);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void* k, const void* v, const float* cs, const float* sn,
                            void* cache, int pos0, int n, int B, int H, int Tmax, int D,
                            bool f16_storage, hipStream_t st) {
    if (f16_storage)
        return D == 64 ? launch_append_t<64, f16>(k, v, cs, sn, cache, pos0, n, B, H, Tmax, st)
                       : launch_append_t<128, f16>(k, v, cs, sn, cache, pos0, n, B, H, Tmax, st);
    return D == 64 ? launch_append_t<64, bf16>(k, v, cs, sn, cache, pos0, n, B, H, Tmax, st)
                   : launch_append_t<128, bf16>(k, v, cs, sn, cache, pos0, n, B, H, Tmax, st);
}

template <int D, typename E>
static hipError_t launch_decode_t(const void* q, const void* knew, const void* vnew,
                                  const void* cache, const float* cs, const float* sn, void* o,
                                  float* lse, float* ws, int pos, int B, int H, int Tmax,
                                  hipStream_t st) {
    const int nsplit = decode_slices(pos);
    const int nwaves = B * H * nsplit;
    const size_t kbytes = (size_t)B * H * Tmax * D * 2;
    f16* kc = static_cast<f16*>(const_cast<void*>(cache));
    E* vc = reinterpret_cast<E*>(static_cast<char*>(const_cast<void*>(cache)) + kbytes);
    const float qs = kLog2e / sqrtf((float)D);
    if (B * H >= kHeadKernelMinHeads) {
        const dim3 hgrid((unsigned)(B * H)), hblock(64 * (nsplit < kHeadWaves<D>() ? nsplit : kHeadWaves<D>()));
        if (knew != nullptr)
            hipLaunchKernelGGL((decode_head_kernel<D, E, true>), hgrid, hblock, 0, st,
                               (const E*)q, kc, vc, cs, sn, (E*)o, lse, (const E*)knew,
                               (const E*)vnew, Tmax, pos, nsplit, qs);
        else
            hipLaunchKernelGGL((decode_head_kernel<D, E, false>), hgrid, hblock, 0, st,
                               (const E*)q, kc, vc, cs, sn, (E*)o, lse, (const E*)nullptr,
                               (const E*)nullptr, Tmax, pos, nsplit, qs);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (knew != nullptr)
        hipLaunchKernelGGL((decode_partial_kernel<D, E, true>), grid, block, 0, st, (const E*)q,
                           kc, vc, cs, sn, ws, (const E*)knew, (const E*)vnew, Tmax, pos, nsplit,
                           nwaves, qs);
    else
        hipLaunchKernelGGL((decode_partial_kernel<D, E, false>), grid, block, 0, st, (const E*)q,
                           kc, vc, cs, sn, ws, (const E*)nullptr, (const E*)nullptr, Tmax, pos,
                           nsplit, nwaves, qs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D, E>), dim3((unsigned)(B * H)), dim3(D), 0, st,
                       ws, (E*)o, lse, nsplit);
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* knew, const void* vnew, const void* cache,
                         const float* cs, const float* sn, void* o, float* lse, float* ws, int pos,
                         int B, int H, int Tmax, int D, bool f16_storage, hipStream_t st) {
    if (f16_storage)
        return D == 64 ? launch_decode_t<64, f16>(q, knew, vnew, cache, cs, sn, o, lse, ws, pos,
                                                  B, H, Tmax, st)
                       : launch_decode_t<128, f16>(q, knew, vnew, cache, cs, sn, o, lse, ws, pos,
                                                   B, H, Tmax, st);
    return D == 64 ? launch_decode_t<64, bf16>(q, knew, vnew, cache, cs, sn, o, lse, ws, pos, B,
                                               H, Tmax, st)
                   : launch_decode_t<128, bf16>(q, knew, vnew, cache, cs, sn, o, lse, ws, pos, B,
                                                H, Tmax, st);
}

}  // namespace attn
