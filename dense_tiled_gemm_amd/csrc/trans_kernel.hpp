// trans_kernel.hpp -- C = A * B^T on gfx950 with either 16-bit operand stored
// K-outer: A as K x M (M contiguous) and/or B as K x N (N contiguous).
//
// The MMA contract of "Writing Mosaic GPU kernels with Pallas", section "MMA
// (TensorCore)", lets 16-bit operands arrive transposed (an A reference of
// shape (K, M), likewise for B).  Here a K-outer operand is copied to LDS as
// it lies in memory, one 256-byte row per k, and transposed on the way out of
// LDS by ds_read_b64_tr_b16: inside each group of 16 lanes, lane i's element
// e is the i-th of the 16 values that lanes 4e .. 4e+3 address (measured on
// the device).  Lanes 4e+a of group g pointing at T[8g + 4h + e][x + 4a]
// therefore receive T[8g + 4h + 0..3][x + i], and the reads h = 0, 1 together
// give each lane the 8 consecutive k of one row of the MFMA operand, exactly
// what the K-inner layout gives with one 16-byte read.
//
// One workgroup computes one 128 x 128 tile of C with 4 waves (2 x 2, each
// 64 x 64 as 4 x 4 blocks of v_mfma_f32_16x16x32).  Per K step of 64:
//   * loader: every thread moves 4 16-byte chunks of each operand through
//     registers (buffer loads; rows past M or N, k >= K, and chunks past the
//     edge of a K-outer row read as zero);
//   * LDS, per operand and stage 16 KiB:
//       K-inner: 128 rows x 128 bytes, chunk c of row r at c ^ ((r >> 1) & 7);
//       K-outer: 64 rows x 256 bytes, chunk c of row r at c ^ 2 s(r) with
//       s(r) = (r & 3) | ((r >> 3) & 1) << 2, so the 16 rows x 32 bytes that
//       one transpose read touches fall in distinct bank ranges;
//   * pipeline: two stages; the loads for step k+1 are issued before the
//     MFMAs of step k and written to the other stage after them, one barrier
//     per step (the register-staged scheme of tiled_kernel.hpp);
//   * epilogue: the shared store_tile / store_tile_lds.
// Requirements checked by the host: bf16 or f16 inputs, every operand row in
// 16-byte chunks (K % 8 == 0 for a K-inner operand, M % 8 == 0 for a K-outer
// A, N % 8 == 0 for a K-outer B) and 16-byte aligned A and B.
#pragma once

#include "common.hpp"

namespace gbt {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// transpose read of 4 16-bit values (see the header comment)
__device__ inline u32x2 lds_read_tr16(const unsigned char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// pair swizzle of a K-outer row (in units of 16-byte chunks: always even)
__device__ inline int kouter_swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

template <int IN, int OUT, bool TA, bool TB>
__global__ __launch_bounds__(256) void trans_kernel(const u16* __restrict__ A, const u16* __restrict__ B,
                                                    void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                    int tiles_n, int group_m, int vec_store) {
    constexpr int BM = 128, BN = 128, BK = 64, WN = 2, T = 256;
    constexpr int TM = 64, TN = 64, FM = TM / 16, FN = TN / 16;
    constexpr int OPB = BM * BK * 2;  // bytes of one operand tile (either layout)
    constexpr int STAGE = 2 * OPB;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int64_t tm64, tn64;
    tile_coord(blockIdx.x, tiles_m, tiles_n, group_m, &tm64, &tn64);
    const int m0 = (int)tm64 * BM, n0 = (int)tn64 * BN;

    // Global geometry of one operand: base x0 (its tile's first row or
    // column), extent X (M or N), K-outer or not.
    struct Src {
        __amdgpu_buffer_rsrc_t r;
        u32 ld_bytes;  // bytes between consecutive k (K-outer) or rows (K-inner)
        int lim;       // valid rows (K-inner) or elements of a k-row (K-outer) from x0
    };
    auto make_src = [&](const u16* X, int x0, int ext, bool kouter) {
        Src s;
        if (kouter) {
            // K x ext matrix: rows k, element x at k * ext + x; the range ends at
            // the matrix end, so rows k >= K read as zero
            s.r = make_rsrc(X + x0, (u32)min(((size_t)K * ext - x0) * 2, (size_t)0x7FFFFFFF));
            s.ld_bytes = (u32)ext * 2u;
            s.lim = ext - x0;
        } else {
            const int rows = min(BM, ext - x0);
            s.r = make_rsrc(X + (size_t)x0 * K, (u32)rows * (u32)K * 2u);
            s.ld_bytes = (u32)K * 2u;
            s.lim = rows;
        }
        return s;
    };
    const Src sa = make_src(A, m0, M, TA);
    const Src sb = make_src(B, n0, N, TB);

    // Loader: 4 chunks per operand per thread.  K-inner: chunk column
    // tid & 7 of tile rows (tid >> 3) + 32 i; K-outer: chunk column tid & 15
    // of k-rows (tid >> 4) + 16 i.  Either way the swizzle term is the same
    // for a thread's 4 rows.
    const int in_c = tid & 7, in_r = tid >> 3;
    const int out_c = tid & 15, out_r = tid >> 4;
    const int in_phys = in_c ^ ((in_r >> 1) & 7);
    const int out_phys = out_c ^ kouter_swz(out_r);

    u32x4 ga[4], gb[4];
    auto gload_op = [&](const Src& s, bool kouter, int kt, u32x4 (&g)[4]) {
        if (kouter) {
            const bool col_ok = out_c * 8 < s.lim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32 off = col_ok ? (u32)(kt * BK + out_r + 16 * i) * s.ld_bytes + (u32)out_c * 16u : kOutOfRange;
                g[i] = load8<8>(s.r, off, 8);
            }
        } else {
            const int kc = kt * BK + in_c * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                g[i] = load8<8>(s.r, (u32)(in_r + 32 * i) * s.ld_bytes + (u32)kc * 2u, kc < K ? 8 : 0);
        }
    };
    auto swrite_op = [&](unsigned char* dst, bool kouter, const u32x4 (&g)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (kouter)
                *(u32x4*)(dst + (out_r + 16 * i) * 256 + out_phys * 16) = g[i];
            else
                *(u32x4*)(dst + (in_r + 32 * i) * 128 + in_phys * 16) = g[i];
        }
    };

    // Fragment reads for k-substep ks (32 k) of the 16-row/column block at
    // x (a multiple of 16) within the operand tile.
    const int q = lane & 15, g = lane >> 4;
    const int f_in_phys_base = (q >> 1) & 7;  // K-inner: swizzle of row x + q
    const int e = q >> 2, a4 = q & 3;
    const int f_out_swz = 2 * (e | ((g & 1) << 2));  // K-outer: s(r) of the rows this lane addresses
    auto frag = [&](const unsigned char* src, bool kouter, int x, int ks) -> u32x4 {
        if (kouter) {
            const int c = (x >> 3) + (a4 >> 1);
            const int col = ((c ^ f_out_swz) * 16) + (a4 & 1) * 8;
            const int r0 = 32 * ks + 8 * g + e;
            const u32x2 lo = lds_read_tr16(src + r0 * 256 + col);
            const u32x2 hi = lds_read_tr16(src + (r0 + 4) * 256 + col);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        const int chunk = 4 * ks + g;
        return *(const u32x4*)(src + (x + q) * 128 + ((chunk ^ f_in_phys_base) * 16));
    };

    typedef AccBlock<16> AB;
    typename AB::type acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < AB::regs; ++r) acc[i][j][r] = 0.0f;

    auto compute = [&](int stage) {
        const unsigned char* sA = lds + stage * STAGE;
        const unsigned char* sB = sA + OPB;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            u32x4 fb[FN], fa[FM];
#pragma unroll
            for (int i = 0; i < FN; ++i) fb[i] = frag(sB, TB, wn * TN + 16 * i, ks);
#pragma unroll
            for (int j = 0; j < FM; ++j) fa[j] = frag(sA, TA, wm * TM + 16 * j, ks);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = Mfma<IN>::m16x16x32(fb[i], fa[j], acc[i][j]);
        }
    };

    const int nk = (K + BK - 1) / BK;
    gload_op(sa, TA, 0, ga);
    gload_op(sb, TB, 0, gb);
    swrite_op(lds, TA, ga);
    swrite_op(lds + OPB, TB, gb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            gload_op(sa, TA, kt + 1, ga);
            gload_op(sb, TB, kt + 1, gb);
        }
        compute(cur);
        if (more) {
            unsigned char* nxt = lds + (cur ^ 1) * STAGE;
            swrite_op(nxt, TA, ga);
            swrite_op(nxt + OPB, TB, gb);
        }
        __syncthreads();
    }

    // the loop ended on a barrier: LDS is free for the whole-row epilogue
    if (vec_store == 2)
        store_tile_lds<OUT, FN, FM, BM, BN, 2, T, 2 * STAGE, 16>(acc, lds, C, M, N, m0, n0, wm * TM, wn * TN, wm, tid);
    else
        store_tile<OUT, FN, FM, 16>(acc, C, M, N, m0, n0, wm * TM, wn * TN, lane, vec_store);
}

}  // namespace gbt
