// skinny_dma.hpp -- streaming MFMA kernel for C = A * B^T with M <= 16
// (gfx950).
//
// With at most 16 rows in A the product is bound by reading B once from HBM
// (2 bytes per multiply-add pair): a 16-row tile has an arithmetic intensity
// of about 16 FLOP per byte ("Chapter 7: Writing custom kernels with Pallas",
// section 6.3, intensity bm*bn/(bm+bn) per tile), far below the MI355X
// MFMA/HBM ridge.  So this kernel is organised around keeping enough bytes of
// B in flight, not around data reuse:
//   * each workgroup owns BN rows of B and the whole K range; B and the 16
//     rows of A stream through an STAGES-deep LDS ring, KB elements of K per
//     stage, with buffer_load_dwordx4 ... lds (no register staging), so about
//     (STAGES-1) * (16 + BN) * KB * 2 bytes per workgroup are in flight.  HBM
//     streams B fastest when each workgroup walks few rows at a time, so BN
//     may be 8: the MFMA's first operand then repeats those 8 rows and the
//     repeated outputs are never stored (the matrix cores have ample slack
//     here), and LDS holds only the 8 real rows, so more workgroups fit;
//   * rows are 2*KB bytes long in LDS; the 16-byte chunk index is XORed with
//     the low 4 row bits so the 16 rows read by one MFMA operand load fall
//     in 16 different bank groups of the 64-bank LDS (the same swizzle idea as
//     the tiled kernel, "Optimizing Blackwell matrix multiplication in Mojo
//     (part 2)", section "Kernel 3: Swizzling");
//   * the W waves split each stage's 32-element k-blocks; each runs
//     v_mfma_f32_16x16x32_{bf16,f16} with B as first operand (rows = columns
//     of C) and A as second, fp32 accumulators; at the end the W partial sums
//     are added through LDS in a fixed order, rounded once and stored masked
//     to i < M, j < N;
//   * rows of A past M and of B past N, and chunks at k >= K, read as zero
//     through the buffer range check ("Chapter 7", section 4.3: zero the K
//     overhang of both operands);
//   * rows need only 2-byte alignment: the LDS DMA moves the whole 16-byte
//     chunks below Kf = K & ~7 from any even address, and the last K - Kf
//     (1 to 7) elements of each row, fetched with 16-bit loads before the
//     loop, form one more zero-padded k-block multiplied after it, so each
//     sum still runs over k in increasing order.
#pragma once

#include "common.hpp"
#include "dma_kernel.hpp"

namespace gbt {

template <int IN, int OUT, int BN, int KB, int STAGES, int W, int ROT = 0>
__global__ __launch_bounds__(64 * W) void skinny_dma_kernel(const u16* __restrict__ A, const u16* __restrict__ B,
                                                           void* __restrict__ C, int M, int N, int K,
                                                           int vec_store, long long sa, long long sb, long long sc) {
    batch_item(blockIdx.y, A, B, C, sa, sb, sc);  // one grid row per batch item
    constexpr int AR = 16;                 // rows of A held (M <= 16)
    constexpr int CPR = KB / 8;            // 16-byte chunks per row per stage
    constexpr int ROWB = KB * 2;           // bytes per row per stage
    constexpr int RPI = 1024 / ROWB;       // rows per wave load instruction
    constexpr int BR = BN < 16 ? BN : 16;   // distinct B rows under one 16-row MFMA operand
    constexpr int BNP = BN;                 // B rows held in LDS
    constexpr int A_LOADS = AR / RPI, B_LOADS = BN / RPI;
    constexpr int LOADS = (A_LOADS + B_LOADS) / W;  // per wave per stage
    constexpr int STAGE_BYTES = (AR + BNP) * ROWB;
    constexpr int KBLK = KB / 32;          // MFMA k-blocks per stage
    constexpr int KPW = KBLK / W;          // k-blocks per wave per stage
    constexpr int NBLK = BN < 16 ? 1 : BN / 16;
    constexpr int PEND = (STAGES - 2) * LOADS;
    constexpr int OSZ = OUT == GEMM_BT_F32 ? 4 : 2;
    static_assert(RPI >= 1 && ROWB * RPI == 1024, "stage rows must tile 1 KiB loads");
    static_assert(BN % RPI == 0 && (BN % 16 == 0 || BN < 16), "B rows per workgroup");
    static_assert((A_LOADS + B_LOADS) % W == 0, "loads split evenly over waves");
    static_assert(KBLK % W == 0, "k-blocks split evenly over waves");
    static_assert(CPR >= 16, "swizzle needs 16 chunks per row");
    static_assert(PEND < 64, "vmcnt range");
    static_assert(STAGES * STAGE_BYTES + W * NBLK * 64 * 16 <= 160 * 1024, "LDS budget");
    static_assert(16 % BR == 0, "B rows repeat evenly under a 16-row operand");
    static_assert(LOADS * W == A_LOADS + B_LOADS, "loads split evenly");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * STAGE_BYTES];
    __shared__ f32x4 red[W][NBLK][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * BN;
    const int rows_a = min(AR, M), rows_b = min(BN, N - n0);
    const i32x4 ra = rsrc_words(A, (u32)rows_a * (u32)K * 2u);
    const i32x4 rb = rsrc_words(B + (size_t)n0 * K, (u32)rows_b * (u32)K * 2u);
    const u32 row_bytes = (u32)K * 2u;

    // Loads: stage rows 0..15 hold A, rows 16..16+BN-1 hold B.  Load
    // instruction j (j = wave + i*W) fills stage rows j*RPI .. j*RPI+RPI-1;
    // lane L writes row j*RPI + L/CPR at physical chunk L%CPR, fetching the
    // logical chunk (L%CPR) ^ (row & 15) of that row.
    const int lrow = lane / CPR, lphys = lane % CPR;
    u32 off[LOADS];
    int kc[LOADS];
    bool is_a[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int j = wave + i * W;
        const int srow = j * RPI + lrow;  // stage row
        const int c = lphys ^ (srow & 15);
        const bool a = srow < AR;
        const int grow = a ? srow : srow - AR;  // row within A or within this block of B
        off[i] = (u32)grow * row_bytes + (u32)c * 16u;
        kc[i] = c * 8;
        is_a[i] = a;
    }
    const int Kf = K & ~7;  // whole 16-byte chunks: through the LDS DMA
    const int nk = (Kf + KB - 1) / KB;
    // ROT > 0: workgroup g walks the K steps starting at (g * ROT) mod nk and
    // wraps around, so that concurrent workgroups read different K offsets
    const int k0 = ROT > 0 && nk > 0 ? (int)(((long long)blockIdx.x * ROT) % nk) : 0;
    auto issue = [&](int stage, int kstep) {
        const int kt = ROT > 0 ? (kstep + k0 >= nk ? kstep + k0 - nk : kstep + k0) : kstep;
        unsigned char* sbase = lds + stage * STAGE_BYTES;
        const u32 kbytes = (u32)kt * (u32)ROWB;
        const int kleft = Kf - kt * KB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int j = wave + i * W;
            const u32 o = kc[i] < kleft ? off[i] : kOutOfRange;
            // whether load i reads A or B is fixed per (wave, i) and uniform
            // B is read exactly once: non-temporal; A is re-read by every
            // workgroup and should stay in L2
            if (is_a[i]) dma16<false>(ra, sbase + j * 1024, o, kbytes);
            else dma16<true>(rb, sbase + j * 1024, o, kbytes);
        }
    };

    // Operand reads: lane (r = l%16, q = l/16) reads row r of a 16-row block,
    // logical chunk 4*kb + q.
    const int r16 = lane & 15, q = lane >> 4;
    // K tail: in the extra k-block, lanes with q = 0 hold elements Kf ..
    // Kf + 7 of their row (zeros past K and for rows past M or N); the other
    // lanes' chunks are zero.  Fetched now so the loads hide behind the loop.
    const int tail = K - Kf;
    u32x4 ta = {0u, 0u, 0u, 0u}, tb[NBLK];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) tb[b] = u32x4{0u, 0u, 0u, 0u};
    if (tail > 0 && wave == 0 && q == 0) {
        auto fetch = [&](const u16* src) {
            u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 7; ++e)
                if (e < tail) v[e >> 1] |= (u32)__builtin_nontemporal_load(src + e) << (16 * (e & 1));
            return v;
        };
        if (r16 < rows_a) ta = fetch(A + (size_t)r16 * K + Kf);
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int br = 16 * b + (r16 % BR);  // B row of the operand's row r16 within this block
            if (br < rows_b) tb[b] = fetch(B + (size_t)(n0 + br) * K + Kf);
        }
    }
    f32x4 acc[NBLK];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int stage) {
        const unsigned char* s = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < KPW; ++t) {
            const int kb = wave * KPW + t;
            const int ch = ((4 * kb + q) ^ r16) * 16;  // A rows 0..15: swizzle term r16
            const u32x4 fa = *(const u32x4*)(s + r16 * ROWB + ch);
#pragma unroll
            for (int b = 0; b < NBLK; ++b) {
                // with BN < 16 the operand's rows r16 and r16 + BN repeat B row r16 % BN;
                // the repeated output columns are never stored
                const int brow = AR + 16 * b + (r16 % BR);
                const int chb = ((4 * kb + q) ^ (brow & 15)) * 16;
                const u32x4 fb = *(const u32x4*)(s + brow * ROWB + chb);
                acc[b] = Mfma<IN>::m16x16x32(fb, fa, acc[b]);
            }
        }
    };

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s, s);
    int cs = 0, ls = STAGES - 1;
    for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt<PEND>();
        barrier_no_fence();
        issue(ls, kt + STAGES - 1);
        compute(cs);
        cs = cs + 1 == STAGES ? 0 : cs + 1;
        ls = ls + 1 == STAGES ? 0 : ls + 1;
    }
    wait_vmcnt<0>();
    if (tail > 0 && wave == 0)
#pragma unroll
        for (int b = 0; b < NBLK; ++b) acc[b] = Mfma<IN>::m16x16x32(tb[b], ta, acc[b]);

#pragma unroll
    for (int b = 0; b < NBLK; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    if (wave != 0) return;
    const int m = lane & 15;  // accumulator lane l holds D[4*(l/16) + e][l % 16]: column m of C^T
    if (m >= M) return;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (u32)min((size_t)M * N * OSZ, (size_t)0x7FFFFFFF));
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
        f32x4 sum = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[w][b][lane];
        const int nl = 16 * b + 4 * q;  // padding rows (nl >= BN) are not stored
        const int n = n0 + nl;
        const u32 o = ((u32)m * (u32)N + (u32)n) * OSZ;
        const float v0 = sum[0], v1 = sum[1], v2 = sum[2], v3 = sum[3];
        if (nl >= BN) continue;
        if (vec_store) {
            if (n < N) {
                if constexpr (OUT == GEMM_BT_F32) {
                    u32x4 w4 = {as_u32(v0), as_u32(v1), as_u32(v2), as_u32(v3)};
                    __builtin_amdgcn_raw_buffer_store_b128(w4, rc, o, 0, 0);
                } else {
                    u32x2 w2 = {pack2<OUT>(v0, v1), pack2<OUT>(v2, v3)};
                    __builtin_amdgcn_raw_buffer_store_b64(w2, rc, o, 0, 0);
                }
            }
        } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e < N) {
                    if constexpr (OUT == GEMM_BT_F32) {
                        __builtin_amdgcn_raw_buffer_store_b32(as_u32(vv[e]), rc, o + 4u * e, 0, 0);
                    } else {
                        const u32 p = pack2<OUT>(vv[e], 0.0f);
                        __builtin_amdgcn_raw_buffer_store_b16((u16)(p & 0xFFFFu), rc, o + 2u * e, 0, 0);
                    }
                }
            }
        }
    }
}

}  // namespace gbt
