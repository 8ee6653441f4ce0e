// trans_kernel.hpp -- C = A * B^T on gfx950 with either 16-bit operand stored
// K-outer: A as K x M (M contiguous) and/or B as K x N (N contiguous).
//
// The MMA contract of "Writing Mosaic GPU kernels with Pallas", section "MMA
// (TensorCore)", lets 16-bit operands arrive transposed (an A reference of
// shape (K, M), likewise for B).  Here a K-outer operand is copied to LDS as
// it lies in memory, one row of its tile's columns per k, and transposed on the way out of
// LDS by ds_read_b64_tr_b16: inside each group of 16 lanes, lane i's element
// e is the i-th of the 16 values that lanes 4e .. 4e+3 address (measured on
// the device).  Lanes 4e+a of group g pointing at T[8g + 4h + e][x + 4a]
// therefore receive T[8g + 4h + 0..3][x + i], and the reads h = 0, 1 together
// give each lane the 8 consecutive k of one row of the MFMA operand, exactly
// what the K-inner layout gives with one 16-byte read.
//
// One workgroup computes one BM x BN tile of C (256 x 256 with 8 waves as
// 2 x 4, or 128 x 128 with 4 waves as 2 x 2), each wave (BM/WM) x (BN/WN) as
// 16 x 16 blocks of v_mfma_f32_16x16x32.  Per K step of 64:
//   * loader: LDS DMA (buffer_load ... lds), one 1 KiB block of tile rows
//     per wave instruction, the swizzle applied by choosing which global
//     chunk each lane fetches; rows past M or N, k >= K, and chunks past the
//     edge of a K-outer row land as zeros;
//   * LDS, per operand and stage BX x 64 x 2 bytes (BX = BM or BN):
//       K-inner: BX rows x 128 bytes, chunk c of row r at c ^ ((r >> 1) & 7);
//       K-outer: 64 rows x 2*BX bytes, chunk c of row r at c ^ 2 s(r) with
//       s(r) = (r & 3) | ((r >> 3) & 1) << 2, so the 16 rows x 32 bytes that
//       one transpose read touches fall in distinct bank ranges;
//   * pipeline: two stages; the transfers for step k+1 go out before the
//     MFMAs of step k, one s_waitcnt vmcnt(0) and one barrier per step;
//   * epilogue: the shared whole-row store_tile_lds.
// Requirements checked by the host: bf16 or f16 inputs, every operand row in
// 16-byte chunks (K % 8 == 0 for a K-inner operand, M % 8 == 0 for a K-outer
// A, N % 8 == 0 for a K-outer B) and 16-byte aligned A and B.
#pragma once

#include "common.hpp"
#include "dma_kernel.hpp"  // dma16, rsrc_words, wait_vmcnt, barrier_no_fence

namespace gbt {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// transpose read of 4 16-bit values (see the header comment)
__device__ inline u32x2 lds_read_tr16(const unsigned char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// pair swizzle of a K-outer row (in units of 16-byte chunks: always even)
__host__ __device__ inline int kouter_swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

// Geometry of one operand tile of BX rows/columns by 64 k in LDS.
//   K-inner: BX rows of 128 bytes (8 chunks), chunk c of row r at c ^ ((r >> 1) & 7);
//   K-outer: 64 rows of 2*BX bytes (BX/8 chunks), chunk c of row r at c ^ kouter_swz(r).
template <int BX, bool KOUTER>
struct OpGeom {
    static constexpr int ROWB = KOUTER ? 2 * BX : 128;  // bytes per LDS row
    static constexpr int CR = ROWB / 16;                 // chunks per row
    static constexpr int ROWS = KOUTER ? 64 : BX;
    static constexpr int BYTES = ROWS * ROWB;
};

template <int IN, int OUT, bool TA, bool TB, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void trans_kernel(const u16* __restrict__ A, const u16* __restrict__ B,
                                                             void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                             int tiles_n, int group_m, int vec_store, int item_tiles_m,
                                                             long long sa, long long sb, long long sc) {
    constexpr int T = 64 * WM * WN, BK = 64;
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    typedef OpGeom<BM, TA> GA;
    typedef OpGeom<BN, TB> GB;
    constexpr int STAGE = GA::BYTES + GB::BYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS-DMA base)
    const int wm = wave / WN, wn = wave % WN;

    int64_t tm64, tn64;
    tile_coord(blockIdx.x, tiles_m, tiles_n, group_m, &tm64, &tn64);
    if (tiles_m != item_tiles_m) {
        // batch items are stacked along the tile rows, as in dma_kernel
        const int z = (int)tm64 / item_tiles_m;
        tm64 -= (int64_t)z * item_tiles_m;
        batch_item(z, A, B, C, sa, sb, sc);
    }
    const int m0 = (int)tm64 * BM, n0 = (int)tn64 * BN;

    // Global view of one operand as four buffer-resource words: rows past the
    // extent (K-inner) or the matrix end (K-outer) read as zero.
    auto make_src = [&](const u16* X, int x0, int ext, bool kouter, int bx) {
        if (kouter)
            return rsrc_words(X + x0, (u32)min(((size_t)K * ext - x0) * 2, (size_t)0x7FFFFFFF));
        return rsrc_words(X + (size_t)x0 * K, (u32)min(bx, ext - x0) * (u32)K * 2u);
    };
    const i32x4 ra = make_src(A, m0, M, TA, BM);
    const i32x4 rb = make_src(B, n0, N, TB, BN);
    const int lim_a = M - m0, lim_b = N - n0;

    // Loader: LDS-DMA, one 1 KiB block (RPI = 1024 / ROWB rows) per wave
    // instruction; this wave fills blocks wave + W*i.  Lane L writes row
    // (block * RPI + L / CR) at physical chunk L % CR, so it fetches the
    // logical chunk (L % CR) ^ swizzle(row); chunks at k >= K (K-inner: whole
    // chunks, K % 8 == 0) or past the edge of a K-outer row are sent out of
    // range and land as zeros.
    constexpr int W = WM * WN;
    auto issue_op = [&](const i32x4& r, unsigned char* dst, auto geom, auto kouter_c, int kt, int lim, u32 ld_bytes) {
        typedef decltype(geom) G;
        constexpr bool KO = decltype(kouter_c)::value;
        constexpr int RPI = 1024 / G::ROWB, NI = G::BYTES / 1024 / W;
        static_assert(NI * W * 1024 == G::BYTES, "blocks split evenly over waves");
        const int lc = lane % G::CR;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int blk = wave + W * i;
            const int row = blk * RPI + lane / G::CR;
            u32 off;
            if constexpr (KO) {
                // row = k within the step; ld_bytes = the operand's row pitch (2 * M or 2 * N)
                const int c = lc ^ kouter_swz(row);
                const int k = kt * BK + row;
                off = (k < K && c * 8 < lim) ? (u32)k * ld_bytes + (u32)c * 16u : kOutOfRange;
            } else {
                // row = tile row; ld_bytes = 2 * K
                const int c = lc ^ ((row >> 1) & 7);
                const int kc = kt * BK + c * 8;
                off = kc < K ? (u32)row * ld_bytes + (u32)kc * 2u : kOutOfRange;
            }
            dma16(r, dst + blk * 1024, off, 0u);
        }
    };
    typedef std::integral_constant<bool, TA> KA;
    typedef std::integral_constant<bool, TB> KB;
    auto issue = [&](int stage, int kt) {
        unsigned char* base = lds + stage * STAGE;
        issue_op(ra, base, GA(), KA(), kt, lim_a, TA ? (u32)M * 2u : (u32)K * 2u);
        issue_op(rb, base + GA::BYTES, GB(), KB(), kt, lim_b, TB ? (u32)N * 2u : (u32)K * 2u);
    };

    // Fragment reads for k-substep ks (32 k) of the 16-row/column block at x
    // (a multiple of 16) within an operand tile.
    const int q = lane & 15, g4 = lane >> 4;
    const int f_in_swz = (q >> 1) & 7;  // K-inner: swizzle of row x + q
    const int e = q >> 2, a4 = q & 3;
    const int f_out_swz = 2 * (e | ((g4 & 1) << 2));  // K-outer: kouter_swz of the rows this lane addresses
    auto frag = [&](const unsigned char* src, auto geom, auto kouter_c, int x, int ks) -> u32x4 {
        typedef decltype(geom) G;
        if constexpr (decltype(kouter_c)::value) {
            const int c = (x >> 3) + (a4 >> 1);
            const int col = ((c ^ f_out_swz) * 16) + (a4 & 1) * 8;
            const int r0 = 32 * ks + 8 * g4 + e;
            const u32x2 lo = lds_read_tr16(src + r0 * G::ROWB + col);
            const u32x2 hi = lds_read_tr16(src + (r0 + 4) * G::ROWB + col);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            const int chunk = 4 * ks + g4;
            return *(const u32x4*)(src + (x + q) * 128 + ((chunk ^ f_in_swz) * 16));
        }
    };

    typedef AccBlock<16> AB;
    typename AB::type acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < AB::regs; ++r) acc[i][j][r] = 0.0f;

    // Both k-substeps' fragments are read before their MFMAs, so the second
    // substep's reads run under the first substep's MFMAs.
    auto compute = [&](int stage) {
        const unsigned char* sA = lds + stage * STAGE;
        const unsigned char* sB = sA + GA::BYTES;
        u32x4 fb[BK / 32][FN], fa[BK / 32][FM];
        static_for<0, BK / 32>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            static_for<0, FN>([&](auto ic) { fb[ks][ic] = frag(sB, GB(), KB(), wn * TN + 16 * ic, ks); });
            static_for<0, FM>([&](auto jc) { fa[ks][jc] = frag(sA, GA(), KA(), wm * TM + 16 * jc, ks); });
        });
        static_for<0, BK / 32>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            static_for<0, FN * FM>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                acc[t / FM][t % FM] = Mfma<IN>::m16x16x32(fb[ks][t / FM], fa[ks][t % FM], acc[t / FM][t % FM]);
            });
        });
    };

    // Two LDS stages: the transfers of tile kt+1 go out into the other stage
    // (free since the last barrier) before tile kt is multiplied; each wave
    // then waits for its own transfers and the barrier makes all of them,
    // and the end of every wave's reads of stage kt, visible.
    const int nk = (K + BK - 1) / BK;
    issue(0, 0);
    wait_vmcnt<0>();
    barrier_no_fence();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) issue(cur ^ 1, kt + 1);
        compute(cur);
        wait_vmcnt<0>();
        barrier_no_fence();
    }

    // the loop ended on a barrier: LDS is free for the whole-row epilogue
    // (shifted when rows of C are not 16-byte aligned)
    store_tile_lds<OUT, FN, FM, BM, BN, WM, T, 2 * STAGE, 16>(acc, lds, C, M, N, m0, n0, wm * TM, wn * TN, wm, tid,
                                                             vec_store != 2);
}

}  // namespace gbt
