// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-bit packing, lane exchanges, buffer resources, and the
// direct-to-LDS tile ring with its swizzled operand reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// A 32x32 accumulator with every entry equal to x. Used as the initial value
// of a score product, it subtracts a per-lane offset (a running maximum, a
// log-sum-exp, a row dot product) inside the MFMA instead of once per element.
__device__ __forceinline__ f32x16 splat16(float x) {
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = x;
    return r;
}

// Work item of workgroup `bid` when items are numbered heaviest first and the
// dispatcher hands workgroups to the ncu CUs in rounds (workgroup r*ncu + c
// lands on CU c in round r). Odd rounds take their items in reverse, so a CU
// that received a heavy item in one round receives a light one in the next
// and the per-CU sums of work even out. The reversal moves whole groups of 8
// workgroups, so item i still runs on XCD i mod 8 (the round-robin XCD of its
// workgroup id), which keeps one head's items on one L2 when the head count is
// a multiple of 8. Incomplete rounds, or CU counts that are not a multiple of
// 8, keep the identity order.
__device__ __forceinline__ int snake_item(int bid, int ncu, int n_items) {
    if (ncu <= 0 || (ncu & 7)) return bid;
    const int r = bid / ncu, c = bid - r * ncu;
    if (!(r & 1) || (r + 1) * ncu > n_items) return bid;
    return r * ncu + (((ncu >> 3) - 1 - (c >> 3)) << 3) + (c & 7);
}

// Row t of a head whose 16-bit rows are st elements apart. The in-head byte
// offset fits 32 bits (the entry points check it), so a lane needs one 32-bit
// offset register rather than a 64-bit address.
template <typename E>
__device__ __forceinline__ E* row_ptr(E* head, int t, int st) {
    return reinterpret_cast<E*>(reinterpret_cast<char*>(head) + (uint32_t)t * (uint32_t)st * 2u);
}

// True on every lane when the predicate holds on any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to a 16-bit type (nearest-even) and pack them, first in the low half.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef T T2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, T2));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return pack2<bf16>(lo, hi); }

// 16-bit storage types of the fast path (bf16 or fp16): 8-wide vectors,
// unpacking of a packed pair, and the sum of a packed pair.
template <typename E>
struct Vec8 {
    typedef E type __attribute__((ext_vector_type(8)));
};
template <typename E>
using vec8 = typename Vec8<E>::type;

template <typename E>
__device__ __forceinline__ f32x2 unpack2(uint32_t w) {
    typedef E E2 __attribute__((ext_vector_type(2)));
    return __builtin_convertvector(__builtin_bit_cast(E2, w), f32x2);
}

// acc + lo(w) + hi(w) for a packed pair w, one v_dot2c against (1, 1): two
// probabilities summed per instruction, exactly the rounded values that feed
// the following MFMA.
template <typename E>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    if constexpr (__is_same(E, bf16)) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                               __builtin_bit_cast(b2, 0x3f803f80u), acc, false);
    } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, 0x3c003c00u),
                                      acc, false);
    }
}

// RoPE on one 16-byte chunk of a row: the four adjacent feature pairs
// (x0, x1) of w (storage type E) become (x0 c - x1 s, x0 s + x1 c) for the
// pair's cosine c and sine s, times `scale`, rounded once to fp16. The
// arithmetic is spelled out (explicit fused multiply-adds) so that every kernel
// that rotates a row - the forward's loaders, the rotation pass, the cache
// append and the decode query - produces bitwise the same values.
template <typename E>
__device__ __forceinline__ u32x4 rope_chunk_f16(u32x4 w, f32x4 c, f32x4 s, float scale) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x2 x = unpack2<E>(w[p]);
        const float y0 = __builtin_fmaf(x[0], c[p], -(x[1] * s[p]));
        const float y1 = __builtin_fmaf(x[0], s[p], x[1] * c[p]);
        r[p] = pack2<f16>(y0 * scale, y1 * scale);
    }
    return r;
}

template <typename V>
__device__ __forceinline__ V as_vec8(u32x4 w) { return __builtin_bit_cast(V, w); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Row (0..31) of the 32x32 MFMA result held in item i of lane half h.
__device__ __forceinline__ int item_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

}  // namespace attn

namespace attn {

// Max (or sum) of x over the two lanes l and l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float max_across_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over `bytes` bytes at p: loads at byte offsets >= bytes
// return zeros, which is how the kernels read past the end of a sequence.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
}  // namespace attn

namespace attn {

// ---------------------------------------------------------------------------
// Direct global -> LDS tile streaming and LDS operand reads.
//
// Tiles of ROWS rows x D 16-bit values are stored row-major in LDS without
// padding; within a row the 16-byte chunks are permuted by an XOR swizzle of
// the row index so that the MFMA operand reads below hit distinct banks.
// Loads use buffer_load ... lds: lane l of a wave instruction writes its 16
// bytes at (wave base + 16 l), so one instruction fills 1 KB; each lane fetches
// the global chunk that belongs at its LDS position. Offsets past the end of
// the buffer (rows >= T) read as zeros.
// ---------------------------------------------------------------------------
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier for the LDS ring. Each wave first waits for its own LDS
// reads (lgkmcnt) - its direct-to-LDS loads were already waited for with
// wait_vmcnt - so a plain s_barrier both publishes the tiles those loads
// filled and guarantees the stage about to be refilled is no longer read.
// __syncthreads() would add a release fence that also waits for every
// direct-to-LDS load still in flight (vmcnt(0)), emptying the prefetch ring.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The LDS ring: every stage's tiles are separate __shared__ objects, so the
// compiler can tell that reading one stage does not depend on the
// direct-to-LDS loads still filling another (with one array it waits for every
// load in flight before each operand read). k and v are the two 64-row tiles of
// a stage, x an optional small extra block.
struct Ring {
    char* k[8];
    char* v[8];
    char* x[8];
};

// Calls f(std::integral_constant<int, S>) for S = 0 .. N-1, in order.
template <int N, typename F, int... S>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, S...>) {
    (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Swizzled 16-byte chunk position of chunk c in row r of a tile with D-element
// (2*D-byte) rows. LDS serves 256 bytes per cycle: 16 lanes of a 16-byte read,
// 32 lanes of an 8-byte read. The XOR pattern keeps both operand reads
// conflict-free: the row-operand read (16 consecutive rows, same chunk) and the
// transpose read (rows R..R+3, four consecutive chunks; R a multiple of 4).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (D == 64)
        return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    else
        return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
}

// Byte offset inside a tile of element (r, col) (col a multiple of 4).
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
    return r * (D * 2) + 16 * swz<D>(r, col >> 3) + 2 * (col & 7);
}

// Per-lane voffsets of the loads that fill one ROWS x D tile: NW waves share
// the tile, each issuing IPW 1 KB instructions; instruction i of this wave
// fills LDS bytes [1024 (wave IPW + i), +1024) of the tile and takes its
// global chunk at voff[i] from the tile's first row. Each tile gets its own
// buffer resource starting at that row and ending just after the last element
// of row T-1, so rows past the end of the sequence read as zeros (the range
// check covers the per-lane offset, not a scalar one) and nothing beyond the
// head's last element is touched.
template <int D, int ROWS, int NW>
struct TileLoads {
    static constexpr int NC = D / 8;                 // 16-byte chunks per row
    static constexpr int INSTR = ROWS * NC / 64;     // 1 KB instructions per tile
    static_assert(INSTR % NW == 0, "tile instructions must divide among waves");
    static constexpr int IPW = INSTR / NW;
    static constexpr int ROW_SHIFT = D == 64 ? 7 : 8;  // log2 of a row's 2*D bytes
    static_assert((2 * D) == (1 << ROW_SHIFT), "row bytes");
    uint32_t voff[IPW];
    __device__ __forceinline__ TileLoads(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (wave * IPW + i) * 64 + lane;  // LDS chunk index
            const int r = p / NC, pos = p % NC;
            voff[i] = (uint32_t)(r * D + 8 * swz<D>(r, pos)) * 2;
        }
    }
    // rows r0 .. r0+ROWS-1 of a [T, D] head -> LDS `tile`
    __device__ __forceinline__ void issue(const void* head, int T, int r0, char* tile,
                                          int wave) const {
        const int rows = T > r0 ? T - r0 : 0;
        const rsrc_t src = make_rsrc(static_cast<const char*>(head) + (size_t)r0 * D * 2,
                                     (uint32_t)rows * D * 2);
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, LDS_PTR(tile + (wave * IPW + i) * 1024),
                                                     16, voff[i], 0, 0, 0);
    }
    // The same for a head whose rows are `pitch` elements apart (its rows sit
    // inside token rows that hold other heads or tensors). The row of a chunk is
    // voff >> ROW_SHIFT (the swizzled column stays below one row), so its offset
    // gains row * (pitch - D) * 2 bytes; that is formed right before each load
    // (asm, so the compiler does not keep a second offset array live across the
    // tile loop).
    __device__ __forceinline__ void issue_strided(const void* head, int T, int r0, char* tile,
                                                  int wave, int pitch) const {
        const int rows = T > r0 ? T - r0 : 0;
        const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * pitch + D) * 2 : 0u;
        const rsrc_t src =
            make_rsrc(static_cast<const char*>(head) + (size_t)r0 * pitch * 2, bytes);
        const uint32_t extra = (uint32_t)(pitch - D) * 2;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            uint32_t off;
            asm volatile("v_lshrrev_b32 %0, %2, %1\n\tv_mad_u32_u24 %0, %0, %3, %1"
                         : "=&v"(off)
                         : "v"(voff[i]), "i"(ROW_SHIFT), "s"(extra));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, LDS_PTR(tile + (wave * IPW + i) * 1024),
                                                     16, off, 0, 0, 0);
        }
    }
};

// Byte offsets, inside a tile, of this lane's operand reads (see tile_off):
// k[c]     the row operand (A of a 32x32x16 MFMA contracting over the head
//          dimension) for head-dimension chunk c, row = lane & 31;
// v[b][h]  the two transpose reads of an X^T operand (A of an MFMA contracting
//          over tile rows) for head-dimension block b, see tr_pair.
// Moving 16 or 32 rows down a tile leaves the swizzle unchanged, so the other
// 16-key chunks and 32-key sub-blocks are these offsets plus a constant.
template <int D>
struct OperandOffs {
    int k[D / 16];
    int v[D / 32][2];
    __device__ __forceinline__ OperandOffs(int lane) {
        const int c32 = lane & 31, hf = lane >> 5, g = lane >> 4, m = lane & 15;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) k[c] = tile_off<D>(c32, 16 * c + 8 * hf);
        const int row = 4 * (g >> 1) + (m >> 2);
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
            const int col = 32 * b + 16 * (g & 1) + 4 * (m & 3);
            v[b][0] = tile_off<D>(row, col);
            v[b][1] = tile_off<D>(row + 8, col);
        }
    }
};

// A operand X^T for a 32x32x16 MFMA from a row-major tile X[rows][D], read at
// the two OperandOffs::v offsets of a block: lane (c = lane & 31, h = lane >> 5)
// receives X[8*(i>>2) + 4h + (i&3)][c] for items i = 0..7 (rows relative to the
// 16-row chunk, columns to the 32-wide block) - the row order of the items of a
// 32x32 result, so that rounded result items can be the B operand. Two
// ds_read_b64_tr_b16: within each 16-lane group, lane m gets element m&3 of the
// 8-byte reads of lanes 4j + (m>>2), j = 0..3.
template <typename V>
__device__ __forceinline__ V tr_pair(const char* lo, const char* hi) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lo);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)hi);
    const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(V, r);
}

}  // namespace attn
