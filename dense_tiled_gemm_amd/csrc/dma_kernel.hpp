// dma_kernel.hpp -- LDS-tiled MFMA kernel for C = A * B^T with direct
// global->LDS loads and a multi-stage LDS ring (gfx950).
//
// Same computation and lane maps as staged_kernel (tiled_kernel.hpp); what
// changes is how tiles reach LDS:
//   * loader: buffer_load_dwordx4 ... lds (16 bytes per lane, new on gfx950)
//     moves each 16-byte chunk from global memory straight into LDS with no
//     register staging.  One wave instruction fills 1 KiB of LDS, i.e. 1024 /
//     (2*BK) whole tile rows; lane L writes LDS bytes [16L, 16L+16) of that
//     KiB, so the XOR swizzle is applied on the global side: lane L fetches the
//     logical chunk (L mod CPR) XOR swz(row), which lands where the MFMA reads
//     expect it ("Optimizing Blackwell matrix multiplication in Mojo (part
//     2)", section "Kernel 3: Swizzling" and the appendix's swizzle math: XOR
//     bits of the row into the 16-byte-chunk bits of the address);
//   * pipeline: STAGES LDS buffers in a ring.  Tile kt+STAGES-1 is requested
//     while tile kt is multiplied, so STAGES-1 K steps of MFMA work cover the
//     load latency ("Writing Mosaic GPU kernels with Pallas", section "Hopper
//     (wgmma)": multi-buffered pipeline that refills a slot as soon as the MMA
//     reading it has finished).  Per step: wait until this wave's loads of
//     tile kt have landed (s_waitcnt vmcnt(N) with N = loads of the younger
//     tiles), one s_barrier so every wave's loads have landed and every wave
//     is done reading the slot about to be refilled, refill, compute.  The
//     barrier is issued without a memory fence (a fence would force
//     vmcnt(0) and drain the ring); compiler-only fences keep LDS accesses on
//     their side of it;
//   * K tail and ragged edges: rows past M or N and chunks at k >= K are
//     fetched with an out-of-range offset, which the buffer unit turns into
//     zeros in LDS ("Chapter 7: Writing custom kernels with Pallas", section
//     4.3: zero the K overhang of both operands).  The ring always issues the
//     same number of loads per step (out-of-range ones past the last tile) so
//     the vmcnt bound is a compile-time constant.
#pragma once

#include "common.hpp"

namespace gbt {

// 16-byte-chunk swizzle for tile rows of CPR chunks.  SWZ 0 disables it (for
// measuring bank conflicts); SWZ 1 and 2 XOR 3 (CPR 8) or 2 (CPR 4) row bits
// into the chunk index, starting at row bit 0/1 (CPR 8) or 1/2 (CPR 4), and
// for CPR 16 row bits 0..2 or 0..3.
// gfx950's LDS has 64 four-byte banks (256 bytes per cycle): a ds_read_b128
// is served 16 lanes at a time, so the 16 lanes of one MFMA operand read
// (16 rows, same logical chunk) must hit 16 different 16-byte bank groups.
// With 128-byte rows, row r starts at bank group 8*(r%2); XORing bits 1..3
// of r into the chunk (SWZ 2) spreads rows r..r+15 over all 16 groups, while
// bits 0..2 (SWZ 1, the form that suits 32 banks) leaves 2-way conflicts.
// A 256-byte row covers all 64 banks, so every row starts at group 0 and
// SWZ 2 XORs bits 0..3.
template <int CPR, int SWZ>
__host__ __device__ inline int swz_row(int row) {
    if constexpr (SWZ == 0) return 0;
    else if constexpr (CPR == 16) return SWZ == 1 ? (row & 7) : (row & 15);
    else if constexpr (CPR == 8) return SWZ == 1 ? (row & 7) : ((row >> 1) & 7);
    else return SWZ == 1 ? ((row >> 1) & 3) : ((row >> 2) & 3);
}

// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ inline void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource as four SGPRs for inline assembly (same fields as
// make_rsrc: base address, stride 0, num_records bytes, word 3).
__device__ inline i32x4 rsrc_words(const void* base, u32 bytes) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(u32)p;
    r[1] = (int)((u32)(p >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = kRsrcWord3;
    return r;
}

// One 16-byte-per-lane global->LDS transfer: lane L's 16 bytes from buffer
// offset voff + soff land at LDS byte address m0 + 16 L, where m0 = `dst`
// (wave-uniform).  Written as inline assembly on purpose: the instruction
// then stays invisible to the compiler's wait-count insertion, which would
// otherwise treat every in-flight transfer as aliasing the ds_reads of the
// stage being computed and drain the whole ring (s_waitcnt vmcnt(0)) before
// them.  The kernels order these transfers with explicit s_waitcnt vmcnt(N)
// and barriers instead.  The s_nop covers the M0-write -> LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: the clobber documents the write
// NT = true marks the load non-temporal (streaming data read once: it should
// not displace reusable lines in L2).
template <bool NT = false>
__device__ inline void dma16(const i32x4& r, unsigned char* dst, u32 voff, u32 soff) {
    const u32 m0 = (u32)(uintptr_t)(lds_ptr_t)dst;
    if constexpr (NT) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
            :
            : "s"(m0), "v"(voff), "s"(r), "s"(soff)
            : "memory", "m0");
    } else {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen lds"
            :
            : "s"(m0), "v"(voff), "s"(r), "s"(soff)
            : "memory", "m0");
    }
}
// 4 bytes per lane into LDS at m0 + 4 L: used only to pull cache lines into
// L2 ahead of the 16-byte loads that will need them (the LDS bytes are not
// read).
__device__ inline void dma4_touch(const i32x4& r, unsigned char* dst, u32 voff, u32 soff) {
    const u32 m0 = (u32)(uintptr_t)(lds_ptr_t)dst;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, %3 offen lds"
        :
        : "s"(m0), "v"(voff), "s"(r), "s"(soff)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// SCHED 0: every wave loads fragments and multiplies in the same K step
//          (fragment reads double-buffered in registers);
// SCHED 2-5: early barrier (the default): as SCHED 0, but the barrier of a
//          K step sits before the MFMAs of the tile's last k-substep(s), which
//          then cover the first LDS reads of the next tile and the refill
//          loads; 3 and 4 spread the refill over 2 or all substeps, 5 also
//          reads fragments two substeps ahead (see the SCHED >= 2 branch);
// SCHED 6-8: as 2-4, with each substep's fragment reads spread over the
//          MFMAs of the one before instead of issued as a burst;
// SCHED 1: ping-pong.  The two wave rows (wm = 0, 1) are offset by one
//          barrier: waves w and w+4 share a SIMD, so on every SIMD one wave
//          issues its whole K step of MFMAs from registers while the other
//          reads its next fragments from LDS (and the wm = 0 group issues the
//          next tile's global->LDS loads); the roles swap at each barrier.
//
// PF > 0 (SCHED 0 only): L2 prefetch.  With each refill the waves also touch
// the 128-byte lines of tile kt + STAGES - 1 + PF (one line per tile row when
// BK = 64) with 4-byte LDS-DMA loads into a scratch corner of LDS, so that the
// refill PF steps later finds its lines in L2 instead of paying the full
// HBM / Infinity-Cache latency with only STAGES - 1 steps of cover.
//
// SK = 1: split-K, the work-splitting step of stream-K ("Writing Mosaic GPU
// kernels with Pallas", section "Cluster launch control": the grid walks the
// work itself, so that no core idles while a few tiles finish).  Each of the
// sk.tiles tiles is split along K into sk.pieces = S pieces, one per
// workgroup of a grid of tiles * S.  A tile is finished by the last of its S
// workgroups to arrive: every piece writes its fp32 sums to its own slot of
// sk.partials with device-scope (write-through) stores, waits until they are
// written, and counts itself in the tile's counter; the one that sees the
// other S - 1 already counted reads their sums back with device-scope loads,
// adds the pieces in K order (piece 0 + 1 + 2 ..., whatever the arrival
// order, so the result is the same bits on every run), resets the counter to
// zero and stores the tile.  No workgroup ever waits for another.
struct SkArgs {
    int tiles;           // tiles, each split along K into `pieces` pieces (grid = tiles * pieces)
    int pieces;          // S >= 2
    int nk;              // K steps of BK per tile (over the whole 16-byte chunks of K)
    unsigned* counters;  // one arrival counter per tile, zero between calls
    float* partials;     // one slot of BM * BN floats per workgroup
};

template <int IN, int OUT, int BM, int BN, int BK, int STAGES, int WM, int WN, int SWZ, int SCHED = 0, int PF = 0,
          int MF = 32, int LDW = 0, int RING5 = 0, int SK = 0, int PH = 0>
__global__ __launch_bounds__(64 * WM * WN) void dma_kernel(const u16* __restrict__ A, const u16* __restrict__ B,
                                                          void* __restrict__ C, int M, int N, int K,
                                                          int tiles_m, int tiles_n, int group_m,
                                                          int vec_store, int item_tiles_m, long long sa, long long sb,
                                                          long long sc, const SkArgs sk) {
    constexpr int W = WM * WN;
    constexpr int ESZ = in_size(IN);     // bytes per input element (2, or 1 for 8-bit floats)
    constexpr int EPC = 16 / ESZ;        // elements per 16-byte chunk
    constexpr int ROWB = BK * ESZ;       // bytes per tile row
    constexpr int CPR = ROWB / 16;       // 16-byte chunks per tile row
    constexpr int RPI = 1024 / ROWB;     // tile rows per wave load instruction
    constexpr int LA = BM / (RPI * W);   // A load instructions per wave per stage
    constexpr int LB = BN / (RPI * W);
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / MF, FN = TN / MF;
    // K per MFMA: 16-bit inputs 16 (32x32x16) or 32 (16x16x32); 8-bit inputs 64 (32x32x64)
    constexpr int KSUB = (512 / MF) * (ESZ == 2 ? 1 : 4);
    typedef typename FragT<ESZ>::type Frag;
    constexpr int STAGE_BYTES = (BM + BN) * ROWB;
    constexpr int PFI = PF > 0 ? (BM + BN) / (64 * W) : 0;  // prefetch instructions per wave per step
    constexpr int PEND = (STAGES - 2) * (LA + LB + PFI) + PFI;
    static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "tile rows of 64, 128 or 256 bytes");
    static_assert(ESZ == 2 || MF == 32, "8-bit inputs use the 32x32x64 MFMA");
    static_assert((64 / MF) * (2 / ESZ) * 16 == KSUB * ESZ, "the lanes' fragments cover one substep's bytes once");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(LA * RPI * W == BM && LB * RPI * W == BN, "tile rows must split evenly over waves");
    static_assert(MF == 32 || MF == 16, "MFMA 32x32x16 or 16x16x32");
    static_assert(TM % MF == 0 && TN % MF == 0, "wave tile must be whole MFMA blocks");
    static_assert(BK % (2 * KSUB) == 0, "two or more MFMA k-substeps per K step");
    static_assert(PEND < 64, "vmcnt range");
    static_assert(PF == 0 || (BK == 64 && (BM + BN) % (64 * W) == 0 && SCHED == 0), "prefetch layout");
    // RING5: five slots of one operand tile each instead of STAGES stages
    constexpr int SLOT_BYTES = BM * ROWB;
    constexpr int RING_BYTES = RING5 ? 5 * SLOT_BYTES : STAGES * STAGE_BYTES;
    static_assert(!RING5 || (BM == BN && STAGES == 2 && SCHED == 6 && PF == 0 && RING5 <= 2), "five-slot ring layout");
    static_assert(RING_BYTES + (PF > 0 ? W * 256 : 0) <= 160 * 1024, "LDS budget");
    // PH: the line ring for rows that are 16-byte but not 128-byte aligned
    // (see the loader below)
    static_assert(!PH || (ESZ == 2 && CPR == 8 && !RING5 && SCHED >= 2 && PF == 0 && STAGES >= 3 && LDW == 0),
                  "line ring: 16-bit inputs, 128-byte tile rows, an early-barrier ring of 3 or more stages, "
                  "every wave loading");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[RING_BYTES + (PF > 0 ? W * 256 : 0)];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const u32 row_bytes = (u32)K * (u32)ESZ;
    // Only whole 16-byte chunks go through the LDS DMA: k < Kf.  Rows need no
    // more than 2-byte alignment: the buffer unit accepts 16-byte loads at
    // any even address (a chunk that straddles a 16-byte boundary costs a
    // second access).  When K % 8 != 0, the last K - Kf (1 to 7) elements of
    // every row are added after the loop (see the tail below).
    const int Kf = K & ~(EPC - 1);
    const int nk_all = (Kf + BK - 1) / BK;  // K steps of a whole tile
    static_assert(64 * W >= BM + BN, "one thread per tile row of the K tail");
    typedef AccBlock<MF> AB;
    typedef typename AB::type Acc[FN][FM];

    // The pipeline over K steps kb .. ke-1 of the tile whose A rows start at
    // row m0 of Ap and whose B rows start at row n0 of Bp, added into acc.
    // When ke is the tile's last step and K % 8 != 0, the K tail follows.
    // Leaves every LDS DMA landed; other waves may still read LDS.
    auto run = [&](const u16* Ap, const u16* Bp, int m0, int n0, int kb, int ke, Acc& acc) {
    // The per-lane geometry below is derived from a copy of the lane index
    // that the compiler must treat as new on every call: in the stream-K form
    // (one call per piece) it is then recomputed per piece (a few VALU
    // operations) instead of being kept live, and spilled, across the pieces.
    int lane_r = lane;
    asm volatile("" : "+v"(lane_r));
    // Loader geometry.  Wave instruction i of this wave fills row block
    // j = wave + i*W (rows j*RPI .. j*RPI+RPI-1 of the tile); lane L writes
    // row j*RPI + L/CPR at physical chunk L%CPR and so fetches logical chunk
    // (L%CPR) ^ swz(row).
    const int lrow = lane_r / CPR, lphys = lane_r % CPR;
    // The rows of a wave's instructions are W * RPI apart, a multiple of the
    // swizzle period (16 rows), so all of them fetch the same logical chunk
    // and instruction i only adds i * W * RPI rows to the byte offset.  A and
    // B tiles use the same row mapping.  The offsets are recomputed per load
    // rather than held in registers (they are one add each).
    static_assert((W * RPI) % 16 == 0, "a wave's row blocks share one swizzle");
    const int lchunk = lphys ^ swz_row<CPR, SWZ>(wave * RPI + lrow);
    const int l_kc = lchunk * EPC;  // first K index (within a tile) of the lane's chunk
    u32 l_off = (u32)(wave * RPI + lrow) * row_bytes + (u32)lchunk * 16u;
    const u32 i_stride = (u32)(W * RPI) * row_bytes;
    auto ld_off = [&](int i) { return l_off + (u32)i * i_stride; };

    // Operand reads: row (lane % MF) of each MF-row block, logical chunk
    // (KSUB/8)*ks + lane/MF for k-substep ks; block bases are multiples of MF
    // (>= 16), so the swizzle term depends on the lane only.
    const int fr = lane_r % MF, fhi = lane_r / MF;
    const int fsw = swz_row<CPR, SWZ>(fr);
    const int a_base = (wm * TM + fr) * ROWB;
    const int b_base = BM * ROWB + (wn * TN + fr) * ROWB;
    const int b_base0 = (wn * TN + fr) * ROWB;  // relative to the B tile
    // PH (rows 16-byte aligned, row_bytes % 128 != 0): every 128-byte K
    // segment of such a row straddles two cache lines.  The line ring loads
    // whole aligned lines instead: stage kt holds line kt of each row, the
    // aligned 128 bytes from the row's start rounded down to a line, plus
    // kt * 128.  A row whose start lies ph 16-byte chunks into its line has
    // logical chunk c of K segment kt in line kt (c + ph < 8) or kt + 1
    // (c + ph >= 8).  The loader's lane that owns physical chunk P fetches
    // logical chunk c = P ^ swz of segment kt, or of segment kt - 1 when
    // c + ph >= 8 (its "carry"): that is line chunk (c + ph) % 8 of line kt,
    // so every logical chunk sits at P = c ^ swz of the stage of its line and
    // the operand reads stay one conflict-free ds_read_b128, from stage kt or
    // kt + 1.  Rows 8 apart have the same phase (8 * row_bytes % 128 == 0),
    // so a lane's phase is fixed for all its loads and fragment rows.
    auto phase = [&](const u16* X, int64_t row) {
        return (int)((((uintptr_t)X + (uint64_t)row * row_bytes) & 127u) >> 4);
    };
    const int ld_row = wave * RPI + lrow;  // this lane's first tile row in each load
    const int carry_a = PH ? (lchunk + phase(Ap, (int64_t)m0 + ld_row)) >> 3 : 0;
    const int carry_b = PH ? (lchunk + phase(Bp, (int64_t)n0 + ld_row)) >> 3 : 0;
    const int ph_fa = PH ? phase(Ap, (int64_t)m0 + wm * TM + fr) : 0;
    const int ph_fb = PH ? phase(Bp, (int64_t)n0 + wn * TN + fr) : 0;

    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const i32x4 ra = rsrc_words((const unsigned char*)Ap + (size_t)m0 * row_bytes, (u32)rows_a * row_bytes);
    const i32x4 rb = rsrc_words((const unsigned char*)Bp + (size_t)n0 * row_bytes, (u32)rows_b * row_bytes);
    // k < Ke: the whole chunks of this K range (loads past it come back as zeros)
    const int Ke = min(Kf, ke * BK);
    const bool with_tail = ESZ == 2 && Kf != K && ke == nk_all;
    // K tail (see after the loop): thread t fetches the last K - Kf (1 to 7)
    // elements of tile row t (A rows first, then B rows) now, one 16-bit
    // load each (rows may be only 2-byte aligned), so that their latency
    // hides behind the main loop.  Being older than every ring load, they are
    // also covered by each of the ring's vmcnt waits.
    u32 tail_v[4] = {0u, 0u, 0u, 0u};
    if (with_tail) {
        const int r = threadIdx.x;
        const bool in_a = r < BM;
        const bool valid = in_a ? r < rows_a : (r < BM + BN && r - BM < rows_b);
        if (valid) {
            const u16* src = in_a ? Ap + (size_t)(m0 + r) * K + Kf : Bp + (size_t)(n0 + r - BM) * K + Kf;
            const int t = K - Kf;
#pragma unroll
            for (int e = 0; e < 7; ++e)
                if (e < t) tail_v[e >> 1] |= (u32)__builtin_nontemporal_load(src + e) << (16 * (e & 1));
        }
    }

    auto issue = [&](int stage, int kt) {
        unsigned char* sbase = lds + stage * STAGE_BYTES;
        const u32 kbytes = (u32)(kb + kt) * (u32)ROWB;
        const int kleft = Ke - (kb + kt) * BK;  // valid K elements in this tile (may be <= 0)
        if (kleft >= BK) {
#pragma unroll
            for (int i = 0; i < LA; ++i)
                dma16(ra, sbase + (wave + i * W) * 1024, ld_off(i), kbytes);
#pragma unroll
            for (int i = 0; i < LB; ++i)
                dma16(rb, sbase + BM * ROWB + (wave + i * W) * 1024, ld_off(i), kbytes);
        } else {
#pragma unroll
            for (int i = 0; i < LA; ++i)
                dma16(ra, sbase + (wave + i * W) * 1024, l_kc < kleft ? ld_off(i) : kOutOfRange, kbytes);
#pragma unroll
            for (int i = 0; i < LB; ++i)
                dma16(rb, sbase + BM * ROWB + (wave + i * W) * 1024, l_kc < kleft ? ld_off(i) : kOutOfRange,
                      kbytes);
        }
    };

    // L2 prefetch: lane l of instruction p of this wave touches tile row
    // (wave * PFI + p) * 64 + l (A rows first, then B rows), first line of the
    // tile's 128-byte K segment.
    auto prefetch = [&](int kt) {
        if constexpr (PF > 0) {
            unsigned char* pbase = lds + STAGES * STAGE_BYTES + wave * 256;
            const u32 kbytes = (u32)(kb + kt) * (u32)ROWB;
            const bool live = (kb + kt) * BK < Ke;
#pragma unroll
            for (int p = 0; p < PFI; ++p) {
                const int row = (wave * PFI + p) * 64 + lane;
                if (row < BM)
                    dma4_touch(ra, pbase, live ? (u32)row * row_bytes : kOutOfRange, kbytes);
                else
                    dma4_touch(rb, pbase, live ? (u32)(row - BM) * row_bytes : kOutOfRange, kbytes);
            }
        }
    };

    // Operand fragments are double-buffered in registers: the LDS reads for
    // k-substep ks+1 are issued before the MFMAs of substep ks, so their
    // latency hides behind 8 MFMAs instead of stalling the wave.
    // The lane's fragment of k-substep ks from the row at `rowp`: one 16-byte
    // chunk (16-bit inputs) or two consecutive ones (8-bit inputs), logical
    // chunks (KSUB*ESZ/16)*ks + fhi*CPL + j, stored at chunk ^ fsw.
    // PH: the lane's chunk lies in the next stage (next - this bytes on) when
    // its logical chunk plus the row's phase passes the line's end.
    auto ld_frag = [&](const unsigned char* rowp, int ks, int ph = 0, int next = 0) -> Frag {
        constexpr int CPL = 2 / ESZ;  // chunks per lane per fragment
        const int c0 = (KSUB * ESZ / 16) * ks + fhi * CPL;
        if constexpr (PH) {
            return *(const u32x4*)(rowp + (c0 + ph >= 8 ? next : 0) + ((c0 ^ fsw) * 16));
        } else if constexpr (CPL == 1) {
            return *(const u32x4*)(rowp + ((c0 ^ fsw) * 16));
        } else {
            const u32x4 lo = *(const u32x4*)(rowp + ((c0 ^ fsw) * 16));
            const u32x4 hi = *(const u32x4*)(rowp + (((c0 + 1) ^ fsw) * 16));
            return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // bytes from a stage (or its B tile) to the same place in the next stage
    auto next_stage = [&](const unsigned char* s) -> int {
        return s + STAGE_BYTES < lds + STAGES * STAGE_BYTES ? STAGE_BYTES : -(STAGES - 1) * STAGE_BYTES;
    };
    auto read_frags = [&](const unsigned char* s, int ks, Frag (&fb)[FN], Frag (&fa)[FM]) {
        const int nx = PH ? next_stage(s) : 0;
#pragma unroll
        for (int i = 0; i < FN; ++i) fb[i] = ld_frag(s + b_base + MF * ROWB * i, ks, ph_fb, nx);
#pragma unroll
        for (int j = 0; j < FM; ++j) fa[j] = ld_frag(s + a_base + MF * ROWB * j, ks, ph_fa, nx);
    };
    auto mfma1 = [&](const Frag& b, const Frag& a, typename AB::type& c) {
        if constexpr (ESZ == 1) c = Mfma<IN>::m32x32x64(b, a, c);
        else if constexpr (MF == 32) c = Mfma<IN>::m32x32x16(b, a, c);
        else c = Mfma<IN>::m16x16x32(b, a, c);
    };
    auto mma = [&](const Frag (&fb)[FN], const Frag (&fa)[FM]) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) mfma1(fb[i], fa[j], acc[i][j]);
    };
    auto compute = [&](int stage) {
        const unsigned char* s = lds + stage * STAGE_BYTES;
        constexpr int KS = BK / KSUB;
        Frag fb0[FN], fa0[FM], fb1[FN], fa1[FM];
        read_frags(s, 0, fb0, fa0);
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            read_frags(s, ks + 1, fb1, fa1);
            mma(fb0, fa0);
            if (ks + 2 < KS) read_frags(s, ks + 2, fb0, fa0);
            mma(fb1, fa1);
        }
    };

    const int nk = ke - kb;  // K steps of this range
    if constexpr (SCHED >= 2) {
        // Early barrier: each wave reads the fragments of a tile's last FD
        // k-substeps, then waits for the next tile and joins the barrier
        // before issuing those substeps' MFMAs.  After the barrier these
        // MFMAs run from registers while the first FD fragment sets of the
        // next tile come out of LDS.  The refill of the freed stage is
        // spread over SPREAD substeps (the FD after the barrier and the
        // first SPREAD - FD of the next tile), one or two global->LDS loads
        // after each MFMA, so the load queues and the L2 see a steady stream
        // instead of one burst per K step.  FD = 2 (fragments read two
        // substeps ahead) is for one wave per SIMD, where no second wave
        // covers the LDS latency.  The sched_barrier pins keep the compiler
        // from regrouping the LDS reads, loads and MFMAs.
        constexpr int KS = BK / KSUB;
        // LDW > 0: only waves 0 .. LDW-1 issue the global->LDS loads (each a
        // W/LDW times larger share); the others only read LDS and multiply.
        constexpr int LW = LDW > 0 ? LDW : W;
        static_assert(W % LW == 0 && (LW * RPI) % 16 == 0, "loader waves share the swizzle");
        constexpr int LAW = BM / (RPI * LW), LBW = BN / (RPI * LW);
        static_assert(LAW * RPI * LW == BM && LBW * RPI * LW == BN, "tile rows split evenly over loader waves");
        constexpr int L = LAW + LBW;
        const bool loader = LW == W || wave < LW;
        const u32 lw_stride = (u32)(LW * RPI) * row_bytes;
        constexpr int NMMA = FN * FM;
        constexpr bool ILR = SCHED >= 6;  // fragment reads interleaved with the MFMAs
        constexpr int BASE = ILR ? SCHED - 4 : SCHED;
        static_assert(BASE >= 2 && BASE <= 5 && !(ILR && BASE == 5), "schedule");
        constexpr int FD = BASE == 5 ? 2 : 1;
        constexpr int NSLOT = 2 * FD;  // fragment buffers, used round robin
        constexpr int SPREAD = BASE == 2 ? 1 : (BASE == 3 ? 2 : KS);
        // ILR: the FN + FM fragment reads of the next substep go out one
        // every RS MFMAs over the first half of the current substep, in the
        // order the next substep consumes them (b0, a0 .. a[FM-1], b1 ..), so
        // that with one wave per SIMD the MFMA pipe is not left idle while a
        // burst of reads issues.
        constexpr int NRD = FN + FM;
        constexpr int RS = NMMA / (2 * NRD) > 0 ? NMMA / (2 * NRD) : 1;
        constexpr int CH = L / SPREAD;  // loads per chunk
        constexpr int HEADC = FD < SPREAD ? FD : SPREAD;  // chunks issued after the barrier
        static_assert(KS % NSLOT == 0 && KS > FD && PF == 0, "fragment buffers rotate per substep");
        static_assert(L % SPREAD == 0 && SPREAD <= KS, "refill chunks");
        Frag fb[NSLOT][FN], fa[NSLOT][FM];
        // load d of this wave's share of tile kt into stage `stage` (A rows
        // first), k >= K masked as in issue()
        auto load_one = [&](int stage, int kt, int d) {
            if (!loader) return;
            unsigned char* sbase = lds + stage * STAGE_BYTES;
            if constexpr (PH) {
                // K segment (kb + kt - carry) of the lane's row; its full byte
                // offset in the per-lane operand (none before the first segment)
                const int carry = d < LAW ? carry_a : carry_b;
                const int seg = kb + kt - carry;
                const u32 base = l_off + (u32)(d < LAW ? d : d - LAW) * lw_stride;
                const u32 off = seg >= 0 && seg * BK + l_kc < Ke ? base + (u32)seg * (u32)ROWB : kOutOfRange;
                if (d < LAW)
                    dma16(ra, sbase + (wave + d * LW) * 1024, off, 0u);
                else
                    dma16(rb, sbase + BM * ROWB + (wave + (d - LAW) * LW) * 1024, off, 0u);
                return;
            }
            const u32 kbytes = (u32)(kb + kt) * (u32)ROWB;
            const int kleft = Ke - (kb + kt) * BK;
            if (d < LAW)
                dma16(ra, sbase + (wave + d * LW) * 1024, l_kc < kleft ? l_off + (u32)d * lw_stride : kOutOfRange,
                      kbytes);
            else
                dma16(rb, sbase + BM * ROWB + (wave + (d - LAW) * LW) * 1024,
                      l_kc < kleft ? l_off + (u32)(d - LAW) * lw_stride : kOutOfRange, kbytes);
        };
        // fragment r of substep ks in consumption order: b0, a0 .. a[FM-1], b1 ..
        // (sta, stb: the A and B tiles)
        auto read_one = [&](const unsigned char* sta, const unsigned char* stb, int ks, auto rc, Frag (&fb)[FN],
                            Frag (&fa)[FM]) {
            constexpr int r = decltype(rc)::value;
            const int nx = PH ? next_stage(sta) : 0;
            if constexpr (r == 0)
                fb[0] = ld_frag(stb + b_base0, ks, ph_fb, nx);
            else if constexpr (r <= FM)
                fa[r - 1] = ld_frag(sta + a_base + MF * ROWB * (r - 1), ks, ph_fa, nx);
            else
                fb[r - FM] = ld_frag(stb + b_base0 + MF * ROWB * (r - FM), ks, ph_fb, nx);
        };
        // the NMMA MFMAs of one substep; after MFMA t it issues load d of the
        // refill if d * NMMA / CH == t (when do_load), and with ILR fragment
        // read r of the next substep if r * RS == t.  An int8 fragment pair
        // takes NH = 2 MFMAs of half the length (one per 16-byte half): the
        // first halves of all NMMA pairs go before the second halves, so no
        // MFMA waits for the accumulator of the one just before it, and the
        // reads and loads follow every second one, at the same points in time.
        constexpr int NH = IN == GEMM_BT_INT8 ? 2 : 1;
        auto mma_step = [&](const Frag (&b)[FN], const Frag (&a)[FM], bool do_load, auto&& load_d, auto&& read_r) {
            static_for<0, NMMA * NH>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                constexpr int t = u % NMMA;
                if constexpr (NH == 1)
                    mfma1(b[t / FM], a[t % FM], acc[t / FM][t % FM]);
                else
                    acc[t / FM][t % FM] = Mfma<IN>::template half<u / NMMA>(b[t / FM], a[t % FM], acc[t / FM][t % FM]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (u % NH == NH - 1) {
                    constexpr int p = u / NH;  // issue point, in units of full fragment pairs
                    if constexpr (ILR)
                        static_for<0, NRD>([&](auto rc) {
                            if constexpr (decltype(rc)::value * RS == p) read_r(rc);
                        });
                    static_for<0, CH>([&](auto dc) {
                        constexpr int d = decltype(dc)::value;
                        if constexpr (d * NMMA / CH == p)
                            if (do_load) load_d(d);
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // chunk c of the refill of stage `stage` with tile kt, and with ILR
        // the reads of substep rks of stage rst into rfb/rfa
        auto mma_refill = [&](const Frag (&b)[FN], const Frag (&a)[FM], int stage, int kt, int c,
                              const unsigned char* rst, int rks, Frag (&rfb)[FN], Frag (&rfa)[FM]) {
            mma_step(b, a, c >= 0, [&](int d) { load_one(stage, kt, c * CH + d); },
                     [&](auto rc) { read_one(rst, rst + BM * ROWB, rks, rc, rfb, rfa); });
        };
        if constexpr (RING5) {
        // Five slots of one operand tile each: A(j) sits in slot 2j mod 5 and
        // B(j) in slot 2j + 1 mod 5.  After the barrier of step kt the slots
        // of A(kt) and B(kt) are free; the refill then issues B(kt + 2) into
        // A(kt)'s slot first and A(kt + 3) into B(kt)'s slot after it, so the
        // next wait needs only the first half of the burst (the A loads are
        // requested one step earlier than in the two-stage ring).
        auto slot = [&](int sl) { return lds + sl * SLOT_BYTES; };
        auto load_a = [&](int sl, int kt, int d) {
            if (!loader) return;
            const int kleft = Ke - (kb + kt) * BK;
            dma16(ra, slot(sl) + (wave + d * LW) * 1024, l_kc < kleft ? l_off + (u32)d * lw_stride : kOutOfRange,
                  (u32)(kb + kt) * (u32)ROWB);
        };
        auto load_b = [&](int sl, int kt, int d) {
            if (!loader) return;
            const int kleft = Ke - (kb + kt) * BK;
            dma16(rb, slot(sl) + (wave + d * LW) * 1024, l_kc < kleft ? l_off + (u32)d * lw_stride : kOutOfRange,
                  (u32)(kb + kt) * (u32)ROWB);
        };
        static_assert(SPREAD == 1 && FD == 1 && CH == LAW + LBW, "one refill burst per step");
        // RING5 == 2: A(kt + 2) goes out during the first substep of step kt
        // instead of with the refill burst after the barrier of step kt - 1
        constexpr bool SPLIT = RING5 == 2;
#pragma unroll
        for (int j = 0; j < (SPLIT ? 2 : 3); ++j) {  // A0 B0 A1 B1 (A2)
#pragma unroll
            for (int d = 0; d < LAW; ++d) load_a(2 * j, j, d);
            if (j < 2)
#pragma unroll
                for (int d = 0; d < LBW; ++d) load_b(2 * j + 1, j, d);
        }
        wait_vmcnt<(SPLIT ? 1 : 2) * LAW + LBW>();  // A0 and B0 have landed
        barrier_no_fence();
        static_for<0, NRD>([&](auto rc) { read_one(slot(0), slot(1), 0, rc, fb[0], fa[0]); });
        __builtin_amdgcn_s_waitcnt(0xC07F);
        int sa = 0;  // slot of A(kt); B(kt) is in the next slot
        for (int kt = 0; kt < nk; ++kt) {
            const int sb = sa == 4 ? 0 : sa + 1;
            const int na = sa >= 3 ? sa - 3 : sa + 2, nb = sb >= 3 ? sb - 3 : sb + 2;
            __builtin_amdgcn_sched_barrier(0);
            const int sp = sa == 0 ? 4 : sa - 1;  // slot of B(kt - 1), free since the last barrier
            mma_step(fb[0], fa[0], SPLIT, [&](int d) { if (d < LAW) load_a(sp, kt + 2, d); },
                     [&](auto rc) { read_one(slot(sa), slot(sb), 1, rc, fb[1], fa[1]); });
            wait_vmcnt<LAW>();                   // A(kt + 1), B(kt + 1) have landed; A(kt + 2) may not
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading A(kt), B(kt)
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            // the post-barrier substep (MFMAs with the refill loads and the next
            // tile's first reads among them) runs at raised wave priority, so
            // the SIMD's arbiter favours it over the other wave's pre-barrier
            // substep (4096^3: 97.8 -> 96.3 us)
            __builtin_amdgcn_s_setprio(1);
            mma_step(fb[1], fa[1], true,
                     [&](int d) {
                         if (d < LBW) load_b(sa, kt + 2, d);
                         else if (!SPLIT) load_a(sb, kt + 3, d - LBW);
                     },
                     [&](auto rc) { read_one(slot(na), slot(nb), 0, rc, fb[0], fa[0]); });
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);
            sa = na;
        }
        } else {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
            for (int d = 0; d < L; ++d) load_one(s, s, d);
        // tile 0 has landed (PH: tiles 0 and 1, the lines K segment 0 spans)
        wait_vmcnt<(STAGES - 2 - (PH ? 1 : 0)) * L>();
        barrier_no_fence();
#pragma unroll
        for (int d = 0; d < CH * HEADC; ++d) load_one(STAGES - 1, STAGES - 1, d);  // head chunks of tile STAGES - 1
#pragma unroll
        for (int j = 0; j < FD; ++j) read_frags(lds, j, fb[j], fa[j]);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // both ways into the loop carry no pending LDS reads
        // stage cs holds tile kt; the head chunks of tile kt + STAGES - 1
        // (stage ps) are issued, its other chunks go out during this tile's
        // first substeps
        int cs = 0, ps = STAGES - 1;
        for (int kt = 0; kt < nk; ++kt) {
            const unsigned char* s = lds + cs * STAGE_BYTES;
            const int ns = cs + 1 == STAGES ? 0 : cs + 1;
#pragma unroll
            for (int ks = 0; ks < KS - FD; ++ks) {
                if constexpr (!ILR) read_frags(s, ks + FD, fb[(ks + FD) % NSLOT], fa[(ks + FD) % NSLOT]);
                __builtin_amdgcn_sched_barrier(0);
                mma_refill(fb[ks % NSLOT], fa[ks % NSLOT], ps, kt + STAGES - 1, ks + FD < SPREAD ? ks + FD : -1,
                           s, ks + FD, fb[(ks + FD) % NSLOT], fa[(ks + FD) % NSLOT]);
            }
            // this wave's part of tile kt + 1 has landed (PH: of kt + 2 too,
            // the second line of K segment kt + 1)
            wait_vmcnt<(STAGES - 2 - (PH ? 1 : 0)) * L>();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading stage cs
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!ILR)
#pragma unroll
                for (int j = 0; j < FD; ++j) read_frags(lds + ns * STAGE_BYTES, j, fb[j], fa[j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FD; ++j)  // head chunks of the refill of stage cs
                mma_refill(fb[(KS - FD + j) % NSLOT], fa[(KS - FD + j) % NSLOT], cs, kt + STAGES, j < SPREAD ? j : -1,
                           lds + ns * STAGE_BYTES, j, fb[j], fa[j]);
            // the next tile's first fragments arrived behind those MFMAs;
            // saying so here keeps the next iteration from waiting on the
            // reads it issues first
            __builtin_amdgcn_s_waitcnt(0xC07F);
            ps = cs;
            cs = ns;
        }
        }
    } else if constexpr (SCHED == 1) {
        static_assert(W == 8 && WM == 2, "ping-pong pairs the two wave rows");
        constexpr int KS = BK / KSUB;
        constexpr int L2 = 2 * (LA + LB);  // loads of one whole tile, issued by one wm = 0 wave
        const int grp = wm;  // waves 0..3 and 4..7; wave w and w + 4 share a SIMD
        // The wm = 0 group issues every load of a tile (block rows `wave` and
        // `wave + 4`); the wm = 1 group never loads from global memory.
        auto issue_g0 = [&](int stage, int kt) {
            unsigned char* sbase = lds + stage * STAGE_BYTES;
            const u32 kbytes = (u32)(kb + kt) * (u32)ROWB;
            const int kleft = Ke - (kb + kt) * BK;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int blk = wave + 4 * h;
#pragma unroll
                for (int i = 0; i < LA; ++i) {
                    const int row = (blk + i * W) * RPI + lrow;
                    const int c = lphys ^ swz_row<CPR, SWZ>(row);
                    const u32 o = (u32)row * row_bytes + (u32)c * 16u;
                    dma16(ra, sbase + (blk + i * W) * 1024, c * 8 < kleft ? o : kOutOfRange, kbytes);
                }
#pragma unroll
                for (int i = 0; i < LB; ++i) {
                    const int row = (blk + i * W) * RPI + lrow;
                    const int c = lphys ^ swz_row<CPR, SWZ>(row);
                    const u32 o = (u32)row * row_bytes + (u32)c * 16u;
                    dma16(rb, sbase + BM * ROWB + (blk + i * W) * 1024, c * 8 < kleft ? o : kOutOfRange, kbytes);
                }
            }
        };
        // Tile t lives in stage t % STAGES.  Barriers alternate between the
        // groups' phases: between barriers 2t+1 and 2t+2 the wm = 0 group
        // reads tile t while the wm = 1 group multiplies tile t-1; between
        // 2t+2 and 2t+3 the roles swap.  The refill of stage (t-1) % STAGES
        // with tile t + STAGES - 1 is issued by wm = 0 right after barrier
        // 2t+1, when both groups are done reading tile t-1; wm = 0 waits for
        // tile t+1 (allowing STAGES-2 younger tiles in flight) before barrier
        // 2t+3, after which it reads tile t+1.
        Frag fb[KS][FN], fa[KS][FM];
        if (grp == 0) {
#pragma unroll
            for (int t = 0; t < STAGES - 1; ++t) issue_g0(t, t);
            wait_vmcnt<(STAGES - 2) * L2>();
        }
        barrier_no_fence();
        if (grp == 1) barrier_no_fence();
        int cs = 0;              // stage of tile kt
        int ls = STAGES - 1;     // stage refilled during tile kt's read phase
        for (int kt = 0; kt < nk; ++kt) {
            // memory phase: this group's fragments of tile kt (+ a refill)
            const unsigned char* sc = lds + cs * STAGE_BYTES;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) read_frags(sc, ks, fb[ks], fa[ks]);
            if (grp == 0) issue_g0(ls, kt + STAGES - 1);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading stage cs
            barrier_no_fence();
            // compute phase: the whole K step from registers
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(fb[ks], fa[ks]);
            if (grp == 0) wait_vmcnt<(STAGES - 2) * L2>();  // tile kt + 1 has landed
            barrier_no_fence();
            cs = cs + 1 == STAGES ? 0 : cs + 1;
            ls = ls + 1 == STAGES ? 0 : ls + 1;
        }
        if (grp == 0) barrier_no_fence();
    } else {
    // Every step issues the same pair, (refill of tile t, prefetch of tile
    // t + PF), prologue included, so the loads younger than tile kt's are
    // always PEND instructions.
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
        issue(s, s);
        prefetch(s + PF);
    }
    int cs = 0;               // stage holding tile kt
    int ls = STAGES - 1;      // stage receiving tile kt + STAGES - 1
    for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt<PEND>();
        barrier_no_fence();
        issue(ls, kt + STAGES - 1);
        prefetch(kt + STAGES - 1 + PF);
        compute(cs);
        cs = cs + 1 == STAGES ? 0 : cs + 1;
        ls = ls + 1 == STAGES ? 0 : ls + 1;
    }
    }
    wait_vmcnt<0>();  // the ring's last (out-of-range) loads still write LDS

    if (with_tail) {
        // K tail: the last K - Kf (1 to 7) elements of every row form one
        // more K tile, zero-padded, written into LDS stage 0 in the same
        // swizzled layout and multiplied like the others.  It comes after all
        // whole chunks, so each sum still runs over k in order.
        barrier_no_fence();  // every wave is past its last read of the ring
        const int r = threadIdx.x;  // tile row r: A rows 0 .. BM-1, then B rows
        if (r < BM + BN) {
            // chunk 0 holds elements Kf .. Kf+7 (the fetched elements, zeros
            // past K and for rows past M or N); the other chunks are zero
#pragma unroll
            for (int c = 0; c < CPR; ++c)
                *(u32x4*)(lds + r * ROWB + ((c ^ swz_row<CPR, SWZ>(r)) * 16)) =
                    c == 0 ? u32x4{tail_v[0], tail_v[1], tail_v[2], tail_v[3]} : u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        Frag tb[FN], ta[FM];
#pragma unroll
        for (int ks = 0; ks < BK / KSUB; ++ks) {
            read_frags(lds, ks, tb, ta);
            mma(tb, ta);
        }
    }
    };  // run

    auto zero = [&](Acc& acc) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r = 0; r < AB::regs; ++r) acc[i][j][r] = 0.0f;
    };
    // the finished tile at rows m0.., columns n0.. of Cp
    // (tid_r: the thread index, recomputed per call for the same reason as
    // lane_r in run)
    // the whole-row epilogue takes tile rows of 8, 12, 16, 24 or 2^n 16-byte
    // chunks (epi_chunk), for rows of C of any alignment (shifted when not
    // 16-byte aligned: vec_store < 2); other tile widths store directly
    constexpr int OCPR = BN * (store_type(OUT) == GEMM_BT_F32 ? 4 : 2) / 16;
    constexpr bool WHOLE_ROWS = OCPR == 12 || OCPR == 24 || (OCPR >= 8 && (OCPR & (OCPR - 1)) == 0);
    auto store_c = [&](void* Cp, int m0, int n0, Acc& acc) {
        int tid_r = threadIdx.x;
        asm volatile("" : "+v"(tid_r));
        if constexpr (!WHOLE_ROWS) {
            store_tile<store_type(OUT), FN, FM, MF>(acc, Cp, M, N, m0, n0, wm * TM, wn * TN, tid_r & 63, vec_store);
        } else {
            // every wave is past its last LDS read and its loads have landed
            barrier_no_fence();
            store_tile_lds<store_type(OUT), FN, FM, BM, BN, WM, 64 * W, STAGES * STAGE_BYTES, MF>(
                acc, lds, Cp, M, N, m0, n0, wm * TM, wn * TN, wm, tid_r, vec_store != 2);
        }
    };

    if constexpr (!SK) {
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
        Acc acc;
        zero(acc);
        run(A, B, m0, n0, 0, nk_all, acc);
        store_c(C, m0, n0, acc);
    } else {
        // Split-K (one item; the host sends batches to the plain grid): the
        // workgroups are renumbered die by die (xcd_seq, so that the pieces of
        // a tile sit on one die); rank v computes piece j = v % S, K steps
        // [j*nk/S, (j+1)*nk/S), of tile v / S of the banded order.  The
        // bookkeeping is wave-uniform: readfirstlane pins each value to a
        // scalar register, so none of it competes with the accumulators.
        constexpr int NT = 64 * W;
        constexpr int Q = AB::regs / 4;  // 16-byte groups per accumulator block
        static_assert(W * 64 * 4 * FN * FM * AB::regs == BM * BN * 4, "a partial slot holds one fp32 tile");
        auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
        const int S = sk.pieces, nk = sk.nk;
        const int v = uni((int)xcd_seq(blockIdx.x, (int64_t)sk.tiles * S));
        const int s = uni(v / S), j = uni(v - s * S);
        const int kb = uni((int)((int64_t)j * nk / S)), ke = uni((int)((int64_t)(j + 1) * nk / S));
        // slot of piece jj of this tile: the partial sums of rank s * S + jj;
        // thread t owns 16-byte group e at byte (t + e * NT) * 16 of it
        auto slot = [&](int jj) {
            return make_rsrc(sk.partials + (int64_t)(s * S + jj) * (BM * BN), BM * BN * 4);
        };
        // Cache policy of the partial sums: sc1, device scope.  Stores are
        // written through the die's L2 to device memory, and loads miss any
        // die-local copy, so pieces computed on different dies (each with its
        // own L2) see each other's sums.  (The agent-scope release/acquire
        // fences would write back and invalidate the whole L2 instead: 93 us
        // against 34 us for 1000x3000x2050 split 192 ways.)
        constexpr int kCoherent = 16;
        // acc = P (overwrite) or acc += P, in place, elementwise.  The loads go
        // out in batches of CHUNK 16-byte groups ahead of their adds (the
        // sched_barrier keeps the compiler from pairing each load with its add
        // and waiting for it), so a slot costs NE / CHUNK memory latencies;
        // the batch is smaller when the accumulators already fill half the
        // registers.
        constexpr int NE = FN * FM * Q;
        constexpr int CHUNK = NE <= 16 ? NE : (NE * 4 * 2 > 256 ? 8 : 16);
        static_assert(NE % CHUNK == 0, "whole load batches");
        auto add_slot = [&](__amdgpu_buffer_rsrc_t p, bool overwrite, Acc& acc) {
            int tid_r = threadIdx.x;
            asm volatile("" : "+v"(tid_r));
            static_for<0, NE / CHUNK>([&](auto cc) {
                constexpr int c0 = decltype(cc)::value * CHUNK;
                u32x4 x[CHUNK];
                static_for<0, CHUNK>([&](auto ec) {
                    constexpr int e = c0 + decltype(ec)::value;
                    x[e - c0] = __builtin_amdgcn_raw_buffer_load_b128(p, (u32)(tid_r + e * NT) * 16u, 0, kCoherent);
                });
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, CHUNK>([&](auto ec) {
                    constexpr int e = c0 + decltype(ec)::value;
                    constexpr int i = e / (FM * Q), jf = (e / Q) % FM, q = e % Q;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][jf][4 * q + r] =
                            overwrite ? as_f32(x[e - c0][r]) : acc[i][jf][4 * q + r] + as_f32(x[e - c0][r]);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        int64_t tm, tn;
        band_coord(s, tiles_m, tiles_n, group_m, &tm, &tn);
        const int m0 = uni((int)tm * BM), n0 = uni((int)tn * BN);
        Acc acc;
        zero(acc);
        run(A, B, m0, n0, kb, ke, acc);
        // publish this piece: its partial sums, written through, then counted
        {
            const __amdgpu_buffer_rsrc_t mine = slot(j);
            int tid_r = threadIdx.x;
            asm volatile("" : "+v"(tid_r));
            static_for<0, FN * FM * Q>([&](auto ec) {
                constexpr int e = decltype(ec)::value;
                constexpr int i = e / (FM * Q), jf = (e / Q) % FM, q = e % Q;
                const u32x4 w = {as_u32(acc[i][jf][4 * q]), as_u32(acc[i][jf][4 * q + 1]),
                                 as_u32(acc[i][jf][4 * q + 2]), as_u32(acc[i][jf][4 * q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(w, mine, (u32)(tid_r + e * NT) * 16u, 0, kCoherent);
            });
        }
        wait_vmcnt<0>();  // this wave's sums have reached device memory
        __syncthreads();
        if (threadIdx.x == 0) {
            // every wave of this workgroup is past its wait (the barrier
            // above), so the count follows all of the piece's stores
            const unsigned seen = __hip_atomic_fetch_add(sk.counters + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = seen == (unsigned)(S - 1);
            if (last) __hip_atomic_store(sk.counters + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *(volatile int*)lds = last;
        }
        __syncthreads();
        if (!*(volatile int*)lds) return;
        // last to arrive: sum piece 0 + 1 + ... + S-1 in that order
        int jn;
        if (j == 0) {
            jn = 1;  // acc is piece 0
        } else if (j == 1) {
            add_slot(slot(0), false, acc);  // piece 1 + piece 0 == piece 0 + piece 1
            jn = 2;
        } else {
            add_slot(slot(0), true, acc);  // piece 0; ours is read back in its turn
            jn = 1;
        }
        for (int jj = jn; jj < S; ++jj) add_slot(slot(jj), false, acc);
        store_c(C, m0, n0, acc);
    }
}

}  // namespace gbt
