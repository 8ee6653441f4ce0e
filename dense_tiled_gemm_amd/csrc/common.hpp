// common.hpp -- types and small device helpers shared by the gemm_bt kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_bt.h"

namespace gbt {

typedef unsigned short u16;
typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Cache policy of the C stores: non-temporal (the `nt` bit, aux bit 1).  C
// is written once and not read back by the kernel; streaming it past the L2
// shortens the write burst at the end of the kernel (1000x3000x2050 fp32:
// 32.7 -> 29.7 us; 1024x4096x4096: 40.5 -> 39.7 us).
constexpr int kStoreNT = 2;

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1.
// Used where a body must be replicated whatever its size: the unroll pragma
// gives up above a size limit, and a loop left rolled turns the accumulator
// array's constant indices into dynamic ones, which moves it to scratch.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Buffer-resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle, no index stride).  With stride 0 the hardware range-checks each
// access against num_records bytes: an out-of-range load returns zero and an
// out-of-range store is dropped.  The kernels rely on this for the rows past
// M or N of a ragged tile and as a safety net for everything else.
constexpr int kRsrcWord3 = 0x00020000;
// A byte offset that is always out of range (num_records is kept below 2^31).
constexpr u32 kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Whole-value reinterpretations.  Arguments are taken by value on purpose:
// __builtin_bit_cast applied directly to an element of an ext_vector_type
// reads the vector's first element in this compiler, so always go through a
// plain local.
__device__ inline float as_f32(u32 u) { return __builtin_bit_cast(float, u); }
__device__ inline u32 as_u32(float f) { return __builtin_bit_cast(u32, f); }

// fp32 -> 16-bit, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32),
// two values packed into one dword, the first in the low half.
template <int OUT>
__device__ inline u32 pack2(float a, float b);
template <>
__device__ inline u32 pack2<GEMM_BT_BF16>(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(u32, p);
}
template <>
__device__ inline u32 pack2<GEMM_BT_F16>(float a, float b) {
    f16x2 p = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(u32, p);
}

// Batch item z of a batched product: its A, B and C start z byte strides
// after the base pointers.  A stride of 0 shares the operand between all
// items; a single product is item 0 with zero strides.
template <class PA, class PB, class PC>
__device__ inline void batch_item(long long z, PA& A, PB& B, PC& C, long long sa, long long sb, long long sc) {
    A = (PA)((const char*)A + z * sa);
    B = (PB)((const char*)B + z * sb);
    C = (PC)((char*)C + z * sc);
}

// MFMA wrappers over raw 16-byte operands (8 elements of the input type).
template <int IN>
struct Mfma;
template <>
struct Mfma<GEMM_BT_BF16> {
    __device__ static inline f32x16 m32x32x16(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 m16x16x32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma<GEMM_BT_F16> {
    __device__ static inline f32x16 m32x32x16(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 m16x16x32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// OCP 8-bit float inputs: v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales
// (exponent 127, i.e. 2^0) on both operands.  Each lane supplies 32 bytes of
// one row (the same k bytes of A and of B, so any lane order of k gives the
// full sum); the accumulator layout is that of the 16-bit 32x32 MFMAs.
template <int FMT>
struct MfmaF8 {
    __device__ static inline f32x16 m32x32x64(u32x8 a, u32x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                               c, FMT, FMT, 0, 127, 0, 127);
    }
};
template <>
struct Mfma<GEMM_BT_FP8_E4M3> : MfmaF8<0> {};  // operand format 0: E4M3
template <>
struct Mfma<GEMM_BT_FP8_E5M2> : MfmaF8<1> {};  // operand format 1: E5M2

// 8-bit integer inputs: v_mfma_i32_32x32x32_i8 takes 16 bytes of one row per
// lane, so the 32-byte fragment of a 64-element substep is two instructions,
// one per 16-byte half, each pairing the same half of A and of B (the same k
// bytes, so the sum over both is the full one).  The int32 sums are exact and
// live in the fp32 accumulator registers as raw bits; the int32 output path
// copies those bits unchanged.
template <>
struct Mfma<GEMM_BT_INT8> {
    // half H (0 or 1) of the fragment pair: bytes 16*H .. 16*H+15 of each lane
    template <int H>
    __device__ static inline f32x16 half(u32x8 a, u32x8 b, f32x16 c) {
        const i32x8 ai = __builtin_bit_cast(i32x8, a), bi = __builtin_bit_cast(i32x8, b);
        return __builtin_bit_cast(
            f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{ai[4 * H], ai[4 * H + 1], ai[4 * H + 2], ai[4 * H + 3]},
                                                          i32x4{bi[4 * H], bi[4 * H + 1], bi[4 * H + 2], bi[4 * H + 3]},
                                                          __builtin_bit_cast(i32x16, c), 0, 0, 0));
    }
    __device__ static inline f32x16 m32x32x64(u32x8 a, u32x8 b, f32x16 c) { return half<1>(a, b, half<0>(a, b, c)); }
};

// Bytes per input element, and the per-lane MFMA operand fragment: 8 elements
// (16 bytes) of 16-bit data, 32 elements (32 bytes) of 8-bit data.
constexpr int in_size(int in) {
    return in == GEMM_BT_FP8_E4M3 || in == GEMM_BT_FP8_E5M2 || in == GEMM_BT_INT8 ? 1 : 2;
}
// int32 results are stored exactly as fp32 ones: 4 bytes of accumulator bits.
constexpr int store_type(int out) { return out == GEMM_BT_INT32 ? GEMM_BT_F32 : out; }
template <int ESZ>
struct FragT {
    typedef u32x4 type;
};
template <>
struct FragT<1> {
    typedef u32x8 type;
};

// 8 consecutive 16-bit elements of one row, starting at byte offset `off`
// inside the buffer `r`, with every element at index >= `valid` (0..8)
// replaced by zero.  VEC is the widest access the alignment allows:
// 8 -> one 16-byte load (then `valid` is 0 or 8), 2 -> four 4-byte loads,
// 1 -> eight 2-byte loads.
template <int VEC>
__device__ inline u32x4 load8(__amdgpu_buffer_rsrc_t r, u32 off, int valid);

template <>
__device__ inline u32x4 load8<8>(__amdgpu_buffer_rsrc_t r, u32 off, int valid) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, valid > 0 ? off : kOutOfRange, 0, 0);
}
template <>
__device__ inline u32x4 load8<2>(__amdgpu_buffer_rsrc_t r, u32 off, int valid) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32 d = __builtin_amdgcn_raw_buffer_load_b32(r, 2 * i < valid ? off + 4 * i : kOutOfRange, 0, 0);
        v[i] = d;
    }
    return v;
}
template <>
__device__ inline u32x4 load8<1>(__amdgpu_buffer_rsrc_t r, u32 off, int valid) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32 lo = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * i < valid ? off + 4 * i : kOutOfRange, 0, 0);
        const u32 hi = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * i + 1 < valid ? off + 4 * i + 2 : kOutOfRange, 0, 0);
        v[i] = lo | (hi << 16);
    }
    return v;
}

// One bf16 / f16 bit pattern (low 16 bits of v) to fp32, exactly.
template <int IN>
__device__ inline float decode16(u32 v) {
    if constexpr (IN == GEMM_BT_BF16) return __uint_as_float(v << 16);
    else return (float)__builtin_bit_cast(_Float16, (u16)v);
}

// Workgroup pid of a grid of `total` is dispatched to die (XCD) pid % 8.
// xcd_seq renumbers the grid so that die x holds the contiguous run
// [start_x, start_x + count_x) of the result: a bijection of [0, total).
__host__ __device__ inline int64_t xcd_seq(int64_t pid, int64_t total) {
    constexpr int64_t kXcd = 8;
    const int64_t q = total / kXcd, rem = total % kXcd;
    const int64_t x = pid % kXcd, i = pid / kXcd;
    return x * q + (x < rem ? x : rem) + i;
}

// Banded order over the tile grid: position seq of the sequence is tile
// (tm, tn), with bands of group_m tile-rows walked column by column, rows
// fastest inside a band.
__host__ __device__ inline void band_coord(int64_t seq, int64_t tiles_m, int64_t tiles_n, int group_m, int64_t* tm,
                                           int64_t* tn) {
    const int64_t band_tiles = (int64_t)group_m * tiles_n;
    const int64_t band = seq / band_tiles;
    const int64_t first_m = band * group_m;
    const int64_t rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int64_t in_band = seq - band * band_tiles;
    *tm = first_m + in_band % rows;
    *tn = in_band / rows;
}

// Tile order: XCD regrouping followed by banded (grouped) order.  Identical
// on host and device so the host can verify it is a bijection.
__host__ __device__ inline void tile_coord(int64_t pid, int64_t tiles_m, int64_t tiles_n, int group_m,
                                           int64_t* tm, int64_t* tn) {
    band_coord(xcd_seq(pid, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

// Accumulator blocks of the tiled kernels.  The MFMA takes the B tile as its
// first operand, so block (i, j) of a wave holds a block of C^T, and each
// lane owns 4 consecutive columns of one row of C per group of 4 registers:
//   MF = 32 (v_mfma_f32_32x32x16, 16 registers): register r of lane l is
//     C[mw + 32j + l%32][nw + 32i + 8(r/4) + 4(l/32) + r%4];
//   MF = 16 (v_mfma_f32_16x16x32, 4 registers): register r of lane l is
//     C[mw + 16j + l%16][nw + 16i + 4(l/16) + r].
template <int MF>
struct AccBlock {
    typedef f32x16 type;
    static constexpr int regs = 16;
    __device__ static int row(int lane) { return lane & 31; }
    // first column of register group g (registers 4g .. 4g+3), relative to the block
    __device__ static int col(int lane, int g) { return 8 * g + 4 * (lane >> 5); }
};
template <>
struct AccBlock<16> {
    typedef f32x4 type;
    static constexpr int regs = 4;
    __device__ static int row(int lane) { return lane & 15; }
    __device__ static int col(int lane, int g) { return 4 * (lane >> 4) + 0 * g; }
};

// Store a wave's FN x FM grid of MF x MF accumulator blocks directly: each
// lane writes the 4 consecutive outputs of a register group with one 16-byte
// (fp32) or 8-byte (16-bit) store when vec_store, else element by element.
// Rows >= M and columns >= N are not written.  The fp32 -> 16-bit conversion
// rounds to nearest even, once.
template <int OUT, int FN, int FM, int MF = 32>
__device__ inline void store_tile(const typename AccBlock<MF>::type (&acc)[FN][FM], void* C, int M, int N, int m0,
                                  int n0, int mw, int nw, int lane, int vec_store) {
    typedef AccBlock<MF> AB;
    constexpr int OSZ = OUT == GEMM_BT_F32 ? 4 : 2;
    const size_t c_origin = (size_t)m0 * N + n0;
    const size_t c_rest = (size_t)M * N - c_origin;
    const u32 c_bytes = (u32)min(c_rest * OSZ, (size_t)0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const char*)C + c_origin * OSZ, c_bytes);
    const int mlim = M - m0, nlim = N - n0;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int ml = mw + MF * j + AB::row(lane);
            if (ml >= mlim) continue;
#pragma unroll
            for (int g = 0; g < AB::regs / 4; ++g) {
                const int nl = nw + MF * i + AB::col(lane, g);
                const u32 off = ((u32)ml * (u32)N + (u32)nl) * OSZ;
                const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                if (vec_store) {
                    if (nl < nlim) {
                        if constexpr (OUT == GEMM_BT_F32) {
                            u32x4 w = {as_u32(v0), as_u32(v1), as_u32(v2), as_u32(v3)};
                            __builtin_amdgcn_raw_buffer_store_b128(w, rc, off, 0, kStoreNT);
                        } else {
                            u32x2 w = {pack2<OUT>(v0, v1), pack2<OUT>(v2, v3)};
                            __builtin_amdgcn_raw_buffer_store_b64(w, rc, off, 0, kStoreNT);
                        }
                    }
                } else {
                    const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (nl + e < nlim) {
                            if constexpr (OUT == GEMM_BT_F32) {
                                __builtin_amdgcn_raw_buffer_store_b32(as_u32(vv[e]), rc, off + 4u * e, 0, kStoreNT);
                            } else {
                                const u32 p = pack2<OUT>(vv[e], 0.0f);
                                __builtin_amdgcn_raw_buffer_store_b16((u16)(p & 0xFFFFu), rc, off + 2u * e, 0, kStoreNT);
                            }
                        }
                    }
                }
            }
        }
    }
}

// Physical 16-byte chunk of logical chunk c in row r of the parked output
// tile (rows of CPR chunks).  The 16 rows of one parking pass (16-byte
// writes of fp32 outputs 16 lanes per pass, 8-byte writes of 16-bit outputs
// 32 lanes per pass) must fill all 64 banks, so rows that start at the same
// bank offset get different chunks: c ^ (r mod min(32, CPR)) for rows of 256
// bytes or more; for 128- and 384-byte rows (CPR 8 and 24, two bank offsets,
// rows r and r + 2 alike) row bits 1..3 are XORed into the chunk's low 3
// bits; for 192-byte rows (CPR 12, four bank offsets) row bits 2..3 into its
// low 2 bits.  Each form permutes chunks inside aligned groups of 8 or 4, so
// it is a bijection on the row.
__host__ __device__ inline int epi_chunk(int c, int r, int cpr) {
    if (cpr == 8 || cpr == 24) return c ^ ((r >> 1) & 7);
    if (cpr == 12) return c ^ ((r >> 2) & 3);
    return c ^ (r & ((cpr < 32 ? cpr : 32) - 1));
}

// Bytes 16 - ph .. 31 - ph of the 32 bytes lo:hi (ph even, 0 <= ph < 16):
// the 16 bytes that start ph bytes before hi.  A right shift of the 256-bit
// value by 16 - ph bytes, done on named 64-bit words (no indexed array, which
// the compiler would place in scratch memory).
__device__ inline u32x4 window16(const u32x4 lo, const u32x4 hi, int ph) {
    const uint64_t l0 = lo[0] | ((uint64_t)lo[1] << 32), l1 = lo[2] | ((uint64_t)lo[3] << 32);
    const uint64_t h0 = hi[0] | ((uint64_t)hi[1] << 32), h1 = hi[2] | ((uint64_t)hi[3] << 32);
    const int sh = 16 - ph;                 // bytes, 2 .. 16
    const int q = sh >> 3, b = (sh & 7) * 8;  // whole words, then bits
    const uint64_t x = q == 0 ? l0 : (q == 1 ? l1 : h0);
    const uint64_t y = q == 0 ? l1 : (q == 1 ? h0 : h1);
    const uint64_t z = q == 0 ? h0 : (q == 1 ? h1 : 0ull);
    const uint64_t o0 = b ? (x >> b) | (y << (64 - b)) : x;
    const uint64_t o1 = b ? (y >> b) | (z << (64 - b)) : y;
    return u32x4{(u32)o0, (u32)(o0 >> 32), (u32)o1, (u32)(o1 >> 32)};
}

// Store the workgroup's BM x BN tile through LDS so that each global store
// instruction writes whole rows: every wave first parks its accumulator
// blocks (rounded to OUT) in LDS as a row-major tile, then the NT threads of
// the workgroup copy rows to C with 16 bytes per lane, so 64 lanes write 1 KiB
// of consecutive row bytes (full cache lines instead of 16-byte pieces from
// 32 rows at a time).  The 16-byte chunk c of tile row r sits at physical
// chunk c ^ (r mod min(32, chunks per row)): the column-wise parking
// writes of 16 or 32 rows then spread over the banks, and the row-wise reads
// stay whole chunks.  A tile larger than LDS_BYTES goes in WM passes of one
// wave row each.  Unless `shifted`, requires 16-byte aligned rows of C
// (N * sizeof(OUT) a multiple of 16 and C 16-byte aligned).  With `shifted`
// (rows of any element alignment) each lane writes one 16-byte chunk that is
// aligned in C: a tile row that starts `ph` bytes past a 16-byte boundary
// touches one chunk more than it holds, chunk j taking the last ph bytes of
// parked chunk j - 1 and the first 16 - ph of parked chunk j; the row's first
// and last chunks, shared with the neighbouring tiles, and any chunk cut by
// column N, go out element by element.  Rows >= M and columns >= N are not
// written.  The caller guarantees that no wave still reads or fills `lds`.
template <int OUT, int FN, int FM, int BM, int BN, int WM, int NT, int LDS_BYTES, int MF = 32>
__device__ inline void store_tile_lds(const typename AccBlock<MF>::type (&acc)[FN][FM], unsigned char* lds, void* C,
                                      int M, int N, int m0, int n0, int mw, int nw, int wm, int tid,
                                      bool shifted = false) {
    typedef AccBlock<MF> AB;
    constexpr int OSZ = OUT == GEMM_BT_F32 ? 4 : 2;
    constexpr int ROWB = BN * OSZ;  // bytes per tile row
    constexpr int CPR = ROWB / 16;  // 16-byte chunks per tile row
    constexpr int P = BM * ROWB <= LDS_BYTES ? 1 : WM;
    constexpr int RP = BM / P;  // tile rows per pass
    static_assert(CPR == 12 || CPR == 24 || (CPR >= 8 && (CPR & (CPR - 1)) == 0), "row chunks");
    static_assert(RP * ROWB <= LDS_BYTES, "a pass must fit in LDS");
    static_assert((RP * CPR) % NT == 0, "the row copy covers a pass in whole rounds of NT threads");
    const size_t c_origin = (size_t)m0 * N + n0;
    const size_t c_rest = (size_t)M * N - c_origin;
    const u32 c_bytes = (u32)min(c_rest * OSZ, (size_t)0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const char*)C + c_origin * OSZ, c_bytes);
    const int mlim = M - m0, nlim = N - n0;
    const int lane = tid & 63;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        if (P == 1 || wm == p) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int r = mw + MF * j + AB::row(lane) - p * RP;  // tile row within the pass
#pragma unroll
                    for (int g = 0; g < AB::regs / 4; ++g) {
                        const int col = nw + MF * i + AB::col(lane, g);
                        const int c = col * OSZ / 16;
                        unsigned char* dst = lds + r * ROWB + (epi_chunk(c, r, CPR) * 16) + (OSZ == 2 ? 8 * ((col >> 2) & 1) : 0);
                        const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                        if constexpr (OUT == GEMM_BT_F32)
                            *(u32x4*)dst = u32x4{as_u32(v0), as_u32(v1), as_u32(v2), as_u32(v3)};
                        else
                            *(u32x2*)dst = u32x2{pack2<OUT>(v0, v1), pack2<OUT>(v2, v3)};
                    }
                }
        }
        __syncthreads();
        if (!shifted) {
#pragma unroll
            for (int q0 = 0; q0 < RP * CPR; q0 += NT) {
                const int q = q0 + tid;
                const int r = q / CPR, c = q % CPR;
                const u32x4 v = *(const u32x4*)(lds + r * ROWB + (epi_chunk(c, r, CPR) * 16));
                const int row = p * RP + r, col = c * (16 / OSZ);
                if (row < mlim && col < nlim)
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, ((u32)row * (u32)N + (u32)col) * OSZ, 0, kStoreNT);
            }
        } else {
            constexpr int CH = CPR + 1;  // aligned chunks of C one tile row can touch
            const int row_end = (nlim < BN ? nlim : BN) * OSZ;  // tile-row bytes inside C
#pragma unroll
            for (int q0 = 0; q0 < RP * CH; q0 += NT) {
                const int q = q0 + tid;
                const int r = q / CH, j = q % CH;
                const int row = p * RP + r;
                if (q >= RP * CH || row >= mlim) continue;
                const u32 row_off = (u32)row * (u32)N * OSZ;  // tile row start, from the tile origin
                const int ph = (int)(((uintptr_t)C + (c_origin * OSZ) + row_off) & 15u);
                const int b0 = 16 * j - ph;  // tile-row byte at the start of aligned chunk j
                if (b0 >= row_end || b0 + 16 <= 0) continue;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 lo = j > 0 ? *(const u32x4*)(lds + r * ROWB + (epi_chunk(j - 1, r, CPR) * 16)) : z;
                const u32x4 hi = j < CPR ? *(const u32x4*)(lds + r * ROWB + (epi_chunk(j, r, CPR) * 16)) : z;
                const u32x4 v = window16(lo, hi, ph);
                if (b0 >= 0 && b0 + 16 <= row_end) {
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, row_off + (u32)b0, 0, kStoreNT);
                } else {
#pragma unroll
                    for (int e = 0; e < 16 / OSZ; ++e) {
                        const int b = b0 + e * OSZ;
                        if (b < 0 || b >= row_end) continue;
                        if constexpr (OSZ == 4)
                            __builtin_amdgcn_raw_buffer_store_b32(v[e], rc, row_off + (u32)b, 0, kStoreNT);
                        else
                            __builtin_amdgcn_raw_buffer_store_b16((u16)(v[e >> 1] >> (16 * (e & 1))), rc,
                                                                  row_off + (u32)b, 0, kStoreNT);
                    }
                }
            }
        }
        if (p + 1 < P) __syncthreads();
    }
}

}  // namespace gbt
