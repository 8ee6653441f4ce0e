// tiled_kernel.hpp -- LDS-tiled, double-buffered MFMA kernel for C = A * B^T (gfx950),
// register-staged variant used when rows are not 16-byte aligned (K % 8 != 0
// or operands offset by 2 or 4 bytes); the aligned fast path is dma_kernel.hpp.
//
// One workgroup computes one BM x BN tile of C.  Per K step of BK = 64:
//   * loader: every thread moves 16-byte chunks of the A tile (BM x 64) and
//     the B tile (BN x 64) from HBM/L2 into registers with buffer loads (8
//     threads cover one 128-byte K-row, so reads coalesce: B is stored N x K
//     for exactly this reason, "Optimizing Blackwell matrix multiplication in
//     Mojo (part 2)", section "Kernel 2: TMA and Tensor Core"), then into LDS;
//   * LDS layout: 128 bytes per tile row, the 16-byte chunk index XORed with
//     bits of the row index (the XOR swizzle of the same page, section
//     "Kernel 3: Swizzling" and its appendix on the swizzle math, applied at
//     16-byte granularity to 128-byte rows), so both the loader's row writes
//     and the MFMA operand reads (32 rows, one chunk each) spread over all
//     LDS banks;
//   * pipeline: two LDS stages; the global loads for step k+1 are issued
//     before the MFMAs of step k and written to the other stage after them,
//     one barrier per step ("Writing Mosaic GPU kernels with Pallas", section
//     "Hopper (wgmma)" / waiting for completion: refill a slot while the MMA
//     on the other runs);
//   * MFMA: each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32 x 32
//     blocks and issues v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulators
//     kept in registers for the whole K loop, zero-initialised ("Chapter 7:
//     Writing custom kernels with Pallas", section 4.1: zero the accumulator
//     on the first K step; section 4.1': accumulate in fp32);
//   * K tail: chunks at k >= K load as zero on BOTH operands (same chapter,
//     section 4.3: mask A's columns and B's rows); rows past M or N load as
//     zero through the buffer range check and are never stored;
//   * epilogue: fp32 -> output type once, round to nearest even, stores
//     masked to i < M, j < N (section 4.3: out-of-range writes dropped); when
//     rows of C are whole 16-byte chunks the tile goes out through LDS as
//     whole rows (store_tile_lds).
//
// Operand roles: the MFMA's first operand is taken from the B tile and the
// second from the A tile, so the MFMA computes a block of C^T.  Its
// accumulator layout then gives each lane 4 consecutive columns of one row of
// C, which become one 16-byte (fp32) or 8-byte (16-bit) store.
//
// MFMA 32x32x16 lane maps used here (gfx950): operand lane l holds row l % 32,
// elements 8*(l/32) .. 8*(l/32)+7 of a 32 x 16 slice; accumulator register r
// of lane l is D[8*(r/4) + 4*(l/32) + r%4][l % 32].
#pragma once

#include "common.hpp"

namespace gbt {

template <int SWZ>
__device__ inline int swz(int row) {
    if constexpr (SWZ == 0) return 0;
    else if constexpr (SWZ == 1) return row & 7;
    else return (row >> 1) & 7;
}

template <int IN, int OUT, int BM, int BN, int WM, int WN, int VEC, int SWZ>
__global__ __launch_bounds__(64 * WM * WN) void staged_kernel(const u16* __restrict__ A,
                                                            const u16* __restrict__ B,
                                                            void* __restrict__ C, int M, int N, int K,
                                                            int tiles_m, int tiles_n, int group_m,
                                                            int vec_store, int item_tiles_m, long long sa, long long sb,
                                                          long long sc) {
    constexpr int T = 64 * WM * WN;  // threads
    constexpr int BK = 64;           // K elements per step = 128 bytes = 8 chunks
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int LA = BM * 8 / T, LB = BN * 8 / T;  // 16-byte chunks per thread per step
    constexpr int ROWS_PER_PASS = T / 8;
    constexpr int STAGE = (BM + BN) * 8;  // chunks per LDS stage
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert((BM * 8) % T == 0 && (BN * 8) % T == 0, "tile rows must split evenly over threads");
    static_assert(ROWS_PER_PASS % 16 == 0, "row step must keep the swizzle phase");

    __shared__ u32x4 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int64_t tm64, tn64;
    tile_coord(blockIdx.x, tiles_m, tiles_n, group_m, &tm64, &tn64);
    if (tiles_m != item_tiles_m) {
        // batch items are stacked along the tile rows (tiles_m counts all of
        // them), so the XCD regrouping gives each die whole items
        const int z = (int)tm64 / item_tiles_m;
        tm64 -= (int64_t)z * item_tiles_m;
        batch_item(z, A, B, C, sa, sb, sc);
    }
    const int m0 = (int)tm64 * BM, n0 = (int)tn64 * BN;
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (u32)rows_a * (u32)K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (u32)rows_b * (u32)K * 2u);

    // Loader geometry: thread tid always handles chunk column lc of rows
    // lr, lr + T/8, lr + 2T/8, ...; because T/8 is a multiple of 16 the
    // swizzle term of those rows is the same for all of them.
    const int lc = tid & 7;
    const int lr = tid >> 3;
    const int lsw = lc ^ swz<SWZ>(lr);
    const u32 row_bytes = (u32)K * 2u;
    const u32 ld_off0 = (u32)lr * row_bytes + (u32)lc * 16u;
    const u32 ld_step = (u32)ROWS_PER_PASS * row_bytes;

    // Operand-read geometry: lane reads row (lane % 32) of each 32-row block,
    // chunk 2*s + lane/32 for k-substep s.  Block bases are multiples of 8
    // (of 16 for SWZ 2), so the swizzle term depends on the lane only.
    const int fr = lane & 31;
    const int fhi = lane >> 5;
    const int fsw = swz<SWZ>(fr);
    const int a_row0 = wm * TM + fr;
    const int b_row0 = BM + wn * TN + fr;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 ga[LA], gb[LB];
    const int nk = (K + BK - 1) / BK;

    auto gload = [&](int kt) {
        const int kc = kt * BK + lc * 8;  // first K index of this thread's chunk
        const int valid = min(8, K - kc);
        const u32 kb = (u32)kt * (BK * 2u);
#pragma unroll
        for (int i = 0; i < LA; ++i) ga[i] = load8<VEC>(ra, ld_off0 + (u32)i * ld_step + kb, valid);
#pragma unroll
        for (int i = 0; i < LB; ++i) gb[i] = load8<VEC>(rb, ld_off0 + (u32)i * ld_step + kb, valid);
    };
    auto swrite = [&](int stage) {
        u32x4* s = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < LA; ++i) s[(lr + i * ROWS_PER_PASS) * 8 + lsw] = ga[i];
#pragma unroll
        for (int i = 0; i < LB; ++i) s[(BM + lr + i * ROWS_PER_PASS) * 8 + lsw] = gb[i];
    };
    auto compute = [&](int stage) {
        const u32x4* s = lds + stage * STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = (2 * ks + fhi) ^ fsw;
            u32x4 fb[FN], fa[FM];
#pragma unroll
            for (int i = 0; i < FN; ++i) fb[i] = s[(b_row0 + 32 * i) * 8 + ch];
#pragma unroll
            for (int j = 0; j < FM; ++j) fa[j] = s[(a_row0 + 32 * j) * 8 + ch];
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = Mfma<IN>::m32x32x16(fb[i], fa[j], acc[i][j]);
        }
    };

    gload(0);
    swrite(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) gload(kt + 1);
        compute(cur);
        if (more) swrite(cur ^ 1);
        __syncthreads();
    }

    // the loop ended on a barrier: LDS is free for the whole-row epilogue
    if (vec_store == 2)
        store_tile_lds<OUT, FN, FM, BM, BN, WM, T, 2 * STAGE * 16>(acc, (unsigned char*)lds, C, M, N, m0, n0, wm * TM,
                                                                  wn * TN, wm, tid);
    else
        store_tile<OUT, FN, FM>(acc, C, M, N, m0, n0, wm * TM, wn * TN, lane, vec_store);
}

}  // namespace gbt
