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
// One workgroup computes one BM x BN tile of C (256 x 256 with 8 waves as
// 2 x 4, or 128 x 128 with 4 waves as 2 x 2), each wave (BM/WM) x (BN/WN) as
// 16 x 16 blocks of v_mfma_f32_16x16x32.  Per K step of 64:
//   * loader: every thread moves 16-byte chunks of each operand through
//     registers (buffer loads; rows past M or N, k >= K, and chunks past the
//     edge of a K-outer row read as zero);
//   * LDS, per operand and stage BX x 64 x 2 bytes (BX = BM or BN):
//       K-inner: BX rows x 128 bytes, chunk c of row r at c ^ ((r >> 1) & 7);
//       K-outer: 64 rows x 2*BX bytes, chunk c of row r at c ^ 2 s(r) with
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

// Geometry of one operand tile of BX rows/columns by 64 k in LDS.
//   K-inner: BX rows of 128 bytes (8 chunks), chunk c of row r at c ^ ((r >> 1) & 7);
//   K-outer: 64 rows of 2*BX bytes (BX/8 chunks), chunk c of row r at c ^ kouter_swz(r).
// Loader: T threads, 16-byte chunks; thread t takes chunk column t % CR of rows
// t / CR + (T / CR) * i, so its swizzle term is the same for all its rows.
template <int BX, bool KOUTER, int T>
struct OpGeom {
    static constexpr int ROWB = KOUTER ? 2 * BX : 128;  // bytes per LDS row
    static constexpr int CR = ROWB / 16;                 // chunks per row
    static constexpr int ROWS = KOUTER ? 64 : BX;
    static constexpr int STEP = T / CR;                  // rows between a thread's chunks
    static constexpr int NCH = ROWS * CR / T;            // chunks per thread per K step
    static constexpr int BYTES = ROWS * ROWB;
    static_assert(STEP % 16 == 0 && NCH * T == ROWS * CR, "loader rows must keep the swizzle phase");
};

template <int IN, int OUT, bool TA, bool TB, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void trans_kernel(const u16* __restrict__ A, const u16* __restrict__ B,
                                                             void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                             int tiles_n, int group_m, int vec_store) {
    constexpr int T = 64 * WM * WN, BK = 64;
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    typedef OpGeom<BM, TA, T> GA;
    typedef OpGeom<BN, TB, T> GB;
    constexpr int STAGE = GA::BYTES + GB::BYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int64_t tm64, tn64;
    tile_coord(blockIdx.x, tiles_m, tiles_n, group_m, &tm64, &tn64);
    const int m0 = (int)tm64 * BM, n0 = (int)tn64 * BN;

    // Global view of one operand: rows past the extent (K-inner) or k >= K
    // (K-outer: the range ends at the matrix end) read as zero.
    struct Src {
        __amdgpu_buffer_rsrc_t r;
        u32 ld_bytes;  // bytes between consecutive k (K-outer) or rows (K-inner)
        int lim;       // elements of a k-row from x0 (K-outer)
    };
    auto make_src = [&](const u16* X, int x0, int ext, bool kouter, int bx) {
        Src s;
        if (kouter) {
            s.r = make_rsrc(X + x0, (u32)min(((size_t)K * ext - x0) * 2, (size_t)0x7FFFFFFF));
            s.ld_bytes = (u32)ext * 2u;
        } else {
            s.r = make_rsrc(X + (size_t)x0 * K, (u32)min(bx, ext - x0) * (u32)K * 2u);
            s.ld_bytes = (u32)K * 2u;
        }
        s.lim = ext - x0;
        return s;
    };
    const Src sa = make_src(A, m0, M, TA, BM);
    const Src sb = make_src(B, n0, N, TB, BN);

    u32x4 ga[GA::NCH], gb[GB::NCH];
    auto gload_op = [&](const Src& s, auto geom, auto kouter_c, int kt, auto& g) {
        typedef decltype(geom) G;
        constexpr bool KO = decltype(kouter_c)::value;
        const int c = tid % G::CR, r = tid / G::CR;
        if constexpr (KO) {
            const bool col_ok = c * 8 < s.lim;
#pragma unroll
            for (int i = 0; i < G::NCH; ++i) {
                const int k = kt * BK + r + G::STEP * i;
                g[i] = load8<8>(s.r, (u32)k * s.ld_bytes + (u32)c * 16u, col_ok && k < K ? 8 : 0);
            }
        } else {
            const int kc = kt * BK + c * 8;
#pragma unroll
            for (int i = 0; i < G::NCH; ++i)
                g[i] = load8<8>(s.r, (u32)(r + G::STEP * i) * s.ld_bytes + (u32)kc * 2u, kc < K ? 8 : 0);
        }
    };
    auto swrite_op = [&](unsigned char* dst, auto geom, auto kouter_c, const auto& g) {
        typedef decltype(geom) G;
        constexpr bool KO = decltype(kouter_c)::value;
        const int c = tid % G::CR, r = tid / G::CR;
        const int phys = c ^ (KO ? kouter_swz(r) : ((r >> 1) & 7));
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) *(u32x4*)(dst + (r + G::STEP * i) * G::ROWB + phys * 16) = g[i];
    };
    typedef std::integral_constant<bool, TA> KA;
    typedef std::integral_constant<bool, TB> KB;

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

    auto compute = [&](int stage) {
        const unsigned char* sA = lds + stage * STAGE;
        const unsigned char* sB = sA + GA::BYTES;
        static_for<0, BK / 32>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            u32x4 fb[FN], fa[FM];
            static_for<0, FN>([&](auto ic) { fb[ic] = frag(sB, GB(), KB(), wn * TN + 16 * ic, ks); });
            static_for<0, FM>([&](auto jc) { fa[jc] = frag(sA, GA(), KA(), wm * TM + 16 * jc, ks); });
            static_for<0, FN * FM>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                acc[t / FM][t % FM] = Mfma<IN>::m16x16x32(fb[t / FM], fa[t % FM], acc[t / FM][t % FM]);
            });
        });
    };

    const int nk = (K + BK - 1) / BK;
    gload_op(sa, GA(), KA(), 0, ga);
    gload_op(sb, GB(), KB(), 0, gb);
    swrite_op(lds, GA(), KA(), ga);
    swrite_op(lds + GA::BYTES, GB(), KB(), gb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            gload_op(sa, GA(), KA(), kt + 1, ga);
            gload_op(sb, GB(), KB(), kt + 1, gb);
        }
        compute(cur);
        if (more) {
            unsigned char* nxt = lds + (cur ^ 1) * STAGE;
            swrite_op(nxt, GA(), KA(), ga);
            swrite_op(nxt + GA::BYTES, GB(), KB(), gb);
        }
        __syncthreads();
    }

    // the loop ended on a barrier: LDS is free for the whole-row epilogue
    if (vec_store == 2)
        store_tile_lds<OUT, FN, FM, BM, BN, WM, T, 2 * STAGE, 16>(acc, lds, C, M, N, m0, n0, wm * TM, wn * TN, wm, tid);
    else
        store_tile<OUT, FN, FM, 16>(acc, C, M, N, m0, n0, wm * TM, wn * TN, lane, vec_store);
}

}  // namespace gbt
