// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-bit packing, the RoPE-on-load loader and LDS tile staging.
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

// acc + lo(w) + hi(w) for a packed bf16 pair w (v_dot2c_f32_bf16 against 1, 1):
// two probabilities summed per instruction, exactly the rounded values that
// feed the following MFMA.
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                           __builtin_bit_cast(b2, 0x3f803f80u), acc, false);
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

template <typename V>
__device__ __forceinline__ V as_vec8(u32x4 w) { return __builtin_bit_cast(V, w); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<f16> { typedef f16x8 type; };

// Row (0..31) of the 32x32 MFMA result held in item i of lane half h.
__device__ __forceinline__ int item_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Column order of transposed LDS tiles. Items 8j..8j+7 of a lane half h of a
// 32x32 result (rows 16j + 8g + 4h + i, g = 0..1, i = 0..3) are the B operand of
// a following MFMA that contracts over those rows. Storing row u of the
// contraction at column col_perm(u) (bits 2 and 3 swapped) puts those eight rows
// at columns 16j + 8h .. 16j + 8h + 7, so the matching A operand is one 16-byte
// LDS read.
__device__ __forceinline__ int col_perm(int u) {
    return (u & ~12) | ((u & 4) << 1) | ((u & 8) >> 1);
}

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
__device__ __forceinline__ f32x4 buf_load_f4(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Buffers of one [T, D] bf16 head and of the [T, D/2] fp32 RoPE tables.
template <int D>
struct HeadBufs {
    rsrc_t x, c, s;
    __device__ __forceinline__ HeadBufs(const bf16* head, const float* cs, const float* sn,
                                        int T)
        : x(make_rsrc(head, (uint32_t)T * D * 2)),
          c(make_rsrc(cs, (uint32_t)T * (D / 2) * 4)),
          s(make_rsrc(sn, (uint32_t)T * (D / 2) * 4)) {}
};

// Eight features d0 .. d0+7 of row t (zeros past the end), rotated by R_t in
// fp32 and rounded once to the 16-bit type T: pair p -> (x0 c - x1 s, x0 s + x1 c).
template <int D, typename T>
__device__ __forceinline__ typename Vec8<T>::type rope_operand(const HeadBufs<D>& hb, int t,
                                                               int d0) {
    const u32x4 w = buf_load16(hb.x, (uint32_t)(t * D + d0) * 2);
    const f32x4 c = buf_load_f4(hb.c, (uint32_t)(t * (D / 2) + d0 / 2) * 4);
    const f32x4 s = buf_load_f4(hb.s, (uint32_t)(t * (D / 2) + d0 / 2) * 4);
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x0 = bf16_lo(w[p]), x1 = bf16_hi(w[p]);
        r[p] = pack2<T>(x0 * c[p] - x1 * s[p], x0 * s[p] + x1 * c[p]);
    }
    return as_vec8<typename Vec8<T>::type>(r);
}

// Register-staged copy of rows [r0, r0 + ROWS) of a head, loaded by NT threads
// in units of two rows x 8 features (consecutive lanes take consecutive 16-byte
// pieces of a row, so eight lanes read one 128-byte row). load() issues the global reads (and, with
// ROT, those of the matching cos/sin entries) so they can complete while the
// caller computes; store() then rotates by RoPE in fp32 (if ROT), rounds once
// and writes a row-major copy rm[ROWS][D + 8] of type RM and/or a transposed
// copy tr[D][ROWS + 8] of type TR (void = not written) whose columns follow
// col_perm. Rows at or beyond T read as zeros.
template <int D, int ROWS, int NT, bool ROT>
struct RowStage {
    static constexpr int UNITS = (ROWS / 2) * (D / 8);
    static constexpr int U = UNITS / NT;
    static_assert(UNITS % NT == 0, "tile units must divide evenly among threads");
    u32x4 a[U], b[U];
    f32x4 ca[U], sa[U], cb[U], sb[U];

    __device__ __forceinline__ void load(const HeadBufs<D>& hb, int r0, int tid) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int u = j * NT + tid;
            const int dc = u % (D / 8), kp = u / (D / 8);
            const int ra = r0 + 2 * kp;
            a[j] = buf_load16(hb.x, (uint32_t)(ra * D + 8 * dc) * 2);
            b[j] = buf_load16(hb.x, (uint32_t)((ra + 1) * D + 8 * dc) * 2);
            if constexpr (ROT) {
                ca[j] = buf_load_f4(hb.c, (uint32_t)(ra * (D / 2) + 4 * dc) * 4);
                sa[j] = buf_load_f4(hb.s, (uint32_t)(ra * (D / 2) + 4 * dc) * 4);
                cb[j] = buf_load_f4(hb.c, (uint32_t)((ra + 1) * (D / 2) + 4 * dc) * 4);
                sb[j] = buf_load_f4(hb.s, (uint32_t)((ra + 1) * (D / 2) + 4 * dc) * 4);
            }
        }
    }

    template <typename RM, typename TR>
    __device__ __forceinline__ void store(void* rm_, void* tr_, int tid) const {
        constexpr bool HAS_RM = !__is_same(RM, void), HAS_TR = !__is_same(TR, void);
        constexpr int RS = D + 8, TS = ROWS + 8;
        uint16_t* rm = static_cast<uint16_t*>(rm_);
        uint16_t* tr = static_cast<uint16_t*>(tr_);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int u = j * NT + tid;
            const int dc = u % (D / 8), kp = u / (D / 8);
            u32x4 a_rm, b_rm;
            uint32_t t_w[8];
            if constexpr (ROT) {
                float fa[8], fb[8];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float a0 = bf16_lo(a[j][p]), a1 = bf16_hi(a[j][p]);
                    const float b0 = bf16_lo(b[j][p]), b1 = bf16_hi(b[j][p]);
                    fa[2 * p] = a0 * ca[j][p] - a1 * sa[j][p];
                    fa[2 * p + 1] = a0 * sa[j][p] + a1 * ca[j][p];
                    fb[2 * p] = b0 * cb[j][p] - b1 * sb[j][p];
                    fb[2 * p + 1] = b0 * sb[j][p] + b1 * cb[j][p];
                }
                if constexpr (HAS_RM) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        a_rm[p] = pack2<RM>(fa[2 * p], fa[2 * p + 1]);
                        b_rm[p] = pack2<RM>(fb[2 * p], fb[2 * p + 1]);
                    }
                }
                if constexpr (HAS_TR) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) t_w[e] = pack2<TR>(fa[e], fb[e]);
                }
            } else {
                a_rm = a[j];
                b_rm = b[j];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t_w[2 * e] = (a[j][e] & 0xffffu) | (b[j][e] << 16);
                    t_w[2 * e + 1] = (a[j][e] >> 16) | (b[j][e] & 0xffff0000u);
                }
            }
            if constexpr (HAS_RM) {
                *reinterpret_cast<u32x4*>(rm + (2 * kp) * RS + 8 * dc) = a_rm;
                *reinterpret_cast<u32x4*>(rm + (2 * kp + 1) * RS + 8 * dc) = b_rm;
            }
            if constexpr (HAS_TR) {
                const int col = col_perm(2 * kp);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint32_t*>(tr + (8 * dc + e) * TS + col) = t_w[e];
            }
        }
    }
};

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
// buffer resource starting at that row and ending at row T, so rows past the
// end of the sequence read as zeros (the range check covers the per-lane
// offset, not a scalar one).
template <int D, int ROWS, int NW>
struct TileLoads {
    static constexpr int NC = D / 8;                 // 16-byte chunks per row
    static constexpr int INSTR = ROWS * NC / 64;     // 1 KB instructions per tile
    static_assert(INSTR % NW == 0, "tile instructions must divide among waves");
    static constexpr int IPW = INSTR / NW;
    uint32_t voff[IPW];
    __device__ __forceinline__ TileLoads(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (wave * IPW + i) * 64 + lane;  // LDS chunk index
            const int r = p / NC, pos = p % NC;
            voff[i] = (uint32_t)(r * D + 8 * swz<D>(r, pos)) * 2;
        }
    }
    // rows r0 .. r0+ROWS-1 of a [T, D] 16-bit head -> LDS `tile`
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
};

// 8 consecutive 16-bit values of row r starting at column col (a multiple of 8).
template <int D, typename V>
__device__ __forceinline__ V lds_row8(const char* tile, int r, int col) {
    return *reinterpret_cast<const V*>(tile + tile_off<D>(r, col));
}

// A operand X^T for a 32x32x16 MFMA from a row-major tile X[rows][D]:
// lane (c = lane & 31, h = lane >> 5) receives X[row0 + 8*(i>>2) + 4h + (i&3)][col0 + c]
// for items i = 0..7 - the row order of the items of a 32x32 result (item i of
// lane half h is row 8*(i>>2) + 4h + (i&3)), so that rounded result items can be
// the B operand. Two ds_read_b64_tr_b16: within each 16-lane group, lane m gets
// element m&3 of the 8-byte reads of lanes 4j + (m>>2), j = 0..3.
template <int D, typename V>
__device__ __forceinline__ V lds_tr8(const char* tile, int row0, int col0, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, m = lane & 15;
    const int row = row0 + 4 * (g >> 1) + (m >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (m & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(tile + tile_off<D>(row, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(tile + tile_off<D>(row + 8, col)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(V, r);
}

// Byte offsets, inside a tile, of this lane's operand reads (see tile_off):
// k[c]     the row operand (A of a 32x32x16 MFMA contracting over the head
//          dimension) for head-dimension chunk c, row = lane & 31;
// v[b][h]  the two transpose reads of an X^T operand (A of an MFMA contracting
//          over tile rows) for head-dimension block b, see lds_tr8.
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
