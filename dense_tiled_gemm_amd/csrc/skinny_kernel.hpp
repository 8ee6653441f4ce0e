// skinny_kernel.hpp -- streaming MFMA kernel for C = A * B^T when M <= 16 (gfx950).
//
// With at most 16 rows in A the product is bound by reading B once from HBM
// (2 bytes per multiply-add pair), not by the matrix cores.  The tile
// roofline of "Chapter 7: Writing custom kernels with Pallas", section 6.3,
// puts a 16-row tile at an intensity of about 16 FLOP per byte, far below the
// MI355X ridge, so this kernel is organised around keeping enough bytes of B
// in flight rather than around LDS reuse:
//   * each workgroup owns 16*NB rows of B (NB blocks of 16) and KS waves
//     split K between them; every wave streams its rows of B straight from
//     HBM into registers with 16-byte buffer loads, two k-blocks ahead of use
//     (register double buffering), and reads the matching slice of A (small
//     and shared by all workgroups, so it stays in L2);
//   * v_mfma_f32_16x16x32_{bf16,f16}, first operand from B, second from A,
//     fp32 accumulators (lane l holds D[4*(l/16) + r][l % 16]: 4 consecutive
//     output columns of row l % 16 of C);
//   * the KS partial sums are added through LDS in a fixed order, rounded
//     once to the output type and stored masked to i < M, j < N.
// Rows of A past M and rows of B past N read as zero through the buffer
// range check; k >= K reads as zero on both operands.
#pragma once

#include "common.hpp"

namespace gbt {

template <int IN, int OUT, int NB, int KS, int VEC>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(const u16* __restrict__ A,
                                                         const u16* __restrict__ B,
                                                         void* __restrict__ C, int M, int N, int K,
                                                         int vec_store, long long sa, long long sb, long long sc) {
    batch_item(blockIdx.y, A, B, C, sa, sb, sc);  // one grid row per batch item
    constexpr int U = 4;  // k-blocks of 32 per batch
    constexpr int OSZ = OUT == GEMM_BT_F32 ? 4 : 2;
    __shared__ f32x4 red[KS][NB][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16 * NB;
    const int rows_b = min(16 * NB, N - n0);
    const int rows_a = min(16, M);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (u32)rows_a * (u32)K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (u32)rows_b * (u32)K * 2u);

    // K range of this wave, in whole 32-element k-blocks.
    const int kblocks = (K + 31) / 32;
    const int per = (kblocks + KS - 1) / KS;
    const int kb_begin = wave * per;
    const int kb_end = min(kblocks, kb_begin + per);
    const int k_end = min(K, kb_end * 32);  // elements at or past this read as zero

    const int r = lane & 15;   // row inside a 16-row block
    const int q = lane >> 4;   // which 8-element slice of a 32-element k-block
    const u32 row_bytes = (u32)K * 2u;
    const u32 a_off = (u32)r * row_bytes + (u32)q * 16u;
    const u32 b_off = (u32)r * row_bytes + (u32)q * 16u;
    const u32 b_blk = 16u * row_bytes;

    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4 fa[2][U], fb[2][U][NB];
    auto load_batch = [&](int buf, int kb0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (kb0 + u) * 32 + q * 8;
            const int valid = min(8, k_end - k);
            const u32 kbytes = (u32)(kb0 + u) * 64u;
            fa[buf][u] = load8<VEC>(ra, a_off + kbytes, valid);
#pragma unroll
            for (int b = 0; b < NB; ++b) fb[buf][u][b] = load8<VEC>(rb, b_off + (u32)b * b_blk + kbytes, valid);
        }
    };
    auto mma_batch = [&](int buf) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = Mfma<IN>::m16x16x32(fb[buf][u][b], fa[buf][u], acc[b]);
    };

    // The loop is unrolled by two so that the register buffer index is a
    // constant: indexed by a variable, fa/fb would be placed in scratch.
    int kb = kb_begin;
    if (kb < kb_end) {
        load_batch(0, kb);
        for (;;) {
            if (kb + U >= kb_end) {
                mma_batch(0);
                break;
            }
            load_batch(1, kb + U);
            mma_batch(0);
            kb += U;
            if (kb + U >= kb_end) {
                mma_batch(1);
                break;
            }
            load_batch(0, kb + U);
            mma_batch(1);
            kb += U;
        }
    }

#pragma unroll
    for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    if (wave != 0) return;

    const int m = lane & 15;
    if (m >= M) return;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (u32)min((size_t)M * N * OSZ, (size_t)0x7FFFFFFF));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        f32x4 s = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) s += red[w][b][lane];
        const int n = n0 + 16 * b + 4 * q;
        const u32 off = ((u32)m * (u32)N + (u32)n) * OSZ;
        const float v0 = s[0], v1 = s[1], v2 = s[2], v3 = s[3];
        if (vec_store) {
            if (n < N) {
                if constexpr (OUT == GEMM_BT_F32) {
                    u32x4 w = {as_u32(v0), as_u32(v1), as_u32(v2), as_u32(v3)};
                    __builtin_amdgcn_raw_buffer_store_b128(w, rc, off, 0, 0);
                } else {
                    u32x2 w = {pack2<OUT>(v0, v1), pack2<OUT>(v2, v3)};
                    __builtin_amdgcn_raw_buffer_store_b64(w, rc, off, 0, 0);
                }
            }
        } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e < N) {
                    if constexpr (OUT == GEMM_BT_F32) {
                        __builtin_amdgcn_raw_buffer_store_b32(as_u32(vv[e]), rc, off + 4u * e, 0, 0);
                    } else {
                        const u32 p = pack2<OUT>(vv[e], 0.0f);
                        __builtin_amdgcn_raw_buffer_store_b16((u16)(p & 0xFFFFu), rc, off + 2u * e, 0, 0);
                    }
                }
            }
        }
    }
}

}  // namespace gbt
