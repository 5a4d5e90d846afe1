// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-bit packing, the RoPE-on-load loader and LDS tile staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32] with fp32 accumulation (bf16 or fp16 operands).
// Lane layout (wave64, l = lane, c = l & 31, h = l >> 5):
//   A: lane l holds row c, k = 8h .. 8h+7;  B: lane l holds column c, k = 8h .. 8h+7
//   D: lane l holds column c, rows 8*(i/4) + 4h + (i%4) for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to a 16-bit type (nearest-even) and pack them, first in the low half.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const T a = (T)lo, b = (T)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return pack2<bf16>(lo, hi); }

template <typename V>
__device__ __forceinline__ V as_vec8(u32x4 w) { return __builtin_bit_cast(V, w); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<f16> { typedef f16x8 type; };

// Eight consecutive features of row t of a [T, D] bf16 head starting at d0 (a
// multiple of 8), rotated by R_t with the fp32 cos/sin tables [T, D/2]:
// pair p becomes (x0 c - x1 s, x0 s + x1 c). Rows t >= T give zeros.
template <int D>
__device__ __forceinline__ void rope8(const bf16* __restrict__ x, int t, int d0,
                                      const float* __restrict__ cs,
                                      const float* __restrict__ sn, int T, float* r) {
    if (t >= T) {
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = 0.f;
        return;
    }
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + (size_t)t * D + d0);
    const f32x4 c = *reinterpret_cast<const f32x4*>(cs + (size_t)t * (D / 2) + d0 / 2);
    const f32x4 s = *reinterpret_cast<const f32x4*>(sn + (size_t)t * (D / 2) + d0 / 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x0 = bf16_lo(w[p]), x1 = bf16_hi(w[p]);
        r[2 * p] = x0 * c[p] - x1 * s[p];
        r[2 * p + 1] = x0 * s[p] + x1 * c[p];
    }
}

// rope8, rounded once to the 16-bit type T and packed as an MFMA operand.
template <int D, typename T>
__device__ __forceinline__ typename Vec8<T>::type load_rope8(const bf16* __restrict__ x, int t,
                                                             int d0, const float* __restrict__ cs,
                                                             const float* __restrict__ sn, int T_) {
    float r[8];
    rope8<D>(x, t, d0, cs, sn, T_, r);
    u32x4 w;
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = pack2<T>(r[2 * p], r[2 * p + 1]);
    return as_vec8<typename Vec8<T>::type>(w);
}

// Eight consecutive bf16 at (t, d0) of a [T, D] head without rotation; zero if t >= T.
template <int D>
__device__ __forceinline__ u32x4 load_row8(const bf16* __restrict__ x, int t, int d0, int T) {
    if (t >= T) return u32x4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4*>(x + (size_t)t * D + d0);
}

// Row permutation inside a 32-row MFMA block. When the A operand's row rho is
// taken from tile row key_perm(rho), item i of lane half h of the 32x32 result
// belongs to tile row 16*(i/8) + 8h + (i%8). Items 8j..8j+7 of a lane then form,
// after rounding to 16 bits, the B operand of a following MFMA whose contraction
// runs over those 32 rows in natural order (chunk j, lane half h <-> rows
// 16j + 8h .. 16j + 8h + 7).
__device__ __forceinline__ int key_perm(int rho) {
    const int g = rho >> 3, hh = (rho >> 2) & 1, i = rho & 3;
    return 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + i;
}

// Tile row (0..31) of result item i held by lane half h, for blocks computed
// with key_perm rows.
__device__ __forceinline__ int item_row(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

// Stage rows [r0, r0 + ROWS) of a [T, D] bf16 head into LDS as a row-major copy
// rm[ROWS][D + 8] of type RM and/or a transposed copy tr[D][ROWS + 8] of type TR
// (RM/TR = void: not written). With ROT the rows are rotated by RoPE in fp32 and
// rounded once to each copy's type; without ROT the bf16 values are copied as
// they are (RM and TR must then be bf16). Rows at or beyond T become zeros.
// Work unit: two rows times 8 features; NT threads share the units.
template <int D, int ROWS, int NT, bool ROT, typename RM, typename TR>
__device__ __forceinline__ void stage_rows(const bf16* __restrict__ x, int r0, int T,
                                           const float* __restrict__ cs,
                                           const float* __restrict__ sn, void* rm_, void* tr_,
                                           int tid) {
    constexpr bool HAS_RM = !__is_same(RM, void), HAS_TR = !__is_same(TR, void);
    constexpr int RS = D + 8, TS = ROWS + 8;
    constexpr int UNITS = (ROWS / 2) * (D / 8);
    uint16_t* rm = static_cast<uint16_t*>(rm_);
    uint16_t* tr = static_cast<uint16_t*>(tr_);
#pragma unroll
    for (int u0 = 0; u0 < UNITS; u0 += NT) {
        const int u = u0 + tid;
        if (UNITS % NT != 0 && u >= UNITS) break;
        const int kp = u % (ROWS / 2), dc = u / (ROWS / 2);
        const int ra = r0 + 2 * kp;
        u32x4 a_rm, b_rm;
        uint32_t t_w[8];
        if constexpr (ROT) {
            float a[8], b[8];
            rope8<D>(x, ra, 8 * dc, cs, sn, T, a);
            rope8<D>(x, ra + 1, 8 * dc, cs, sn, T, b);
            if constexpr (HAS_RM) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    a_rm[p] = pack2<RM>(a[2 * p], a[2 * p + 1]);
                    b_rm[p] = pack2<RM>(b[2 * p], b[2 * p + 1]);
                }
            }
            if constexpr (HAS_TR) {
#pragma unroll
                for (int e = 0; e < 8; ++e) t_w[e] = pack2<TR>(a[e], b[e]);
            }
        } else {
            a_rm = load_row8<D>(x, ra, 8 * dc, T);
            b_rm = load_row8<D>(x, ra + 1, 8 * dc, T);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t_w[2 * e] = (a_rm[e] & 0xffffu) | (b_rm[e] << 16);
                t_w[2 * e + 1] = (a_rm[e] >> 16) | (b_rm[e] & 0xffff0000u);
            }
        }
        if constexpr (HAS_RM) {
            *reinterpret_cast<u32x4*>(rm + (2 * kp) * RS + 8 * dc) = a_rm;
            *reinterpret_cast<u32x4*>(rm + (2 * kp + 1) * RS + 8 * dc) = b_rm;
        }
        if constexpr (HAS_TR) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint32_t*>(tr + (8 * dc + e) * TS + 2 * kp) = t_w[e];
        }
    }
}

}  // namespace attn
