// gemm_bt.hip -- C-ABI entry points of libgemm_bt.so: argument checks, launch
// planning and kernel dispatch for C = A * B^T on gfx950.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "common.hpp"
#include "dma_kernel.hpp"
#include "skinny_dma.hpp"
#ifdef GEMM_BT_TUNING
// measured alternatives: register streaming for M <= 16, register-staged
// loads for the tiled kernel
#include "skinny_kernel.hpp"
#include "tiled_kernel.hpp"
#endif
#include "trans_kernel.hpp"

namespace gbt {

// Zero fill of C for K == 0 (every entry is an empty sum); batch item
// blockIdx.y starts `sc` bytes after the previous one.
__global__ void zero_fill_kernel(u16* __restrict__ c, size_t n16, long long sc) {
    c = (u16*)((char*)c + (long long)blockIdx.y * sc);
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) c[i] = 0;
}

enum Kind { KIND_NONE = 0, KIND_FILL = 1, KIND_TILED = 2, KIND_SKINNY = 3, KIND_DMA = 4, KIND_TRANS = 5 };

// Kernels.  Products with M > 16 run dma_kernel (direct global->LDS loads of
// 16-byte chunks, from rows of any even alignment) in one of the tile shapes
// of dma_variants(); through gemm_bt_ws and gemm_bt_noalloc, products that
// leave half the CUs without a tile run its split-K form instead (128 x 128
// tiles, or for M <= 64 thin tiles of 256-byte rows, see plan_split_rule).
// Skinny products (M <= 16) run skinny_dma_kernel (8 rows
// of B per single-wave workgroup, 256-element K stages in a 3-deep LDS ring,
// rows of any even alignment too).  The tuning build also has the
// register-streaming skinny_kernel (GEMM_BT_FORCE_SKINNY=REG: 32 rows, K split
// over 4 waves) and the register-staged tiled kernel (GEMM_BT_FORCE_TILE=STAGED):
//   staged L: 256 x 256, 8 waves as 2 x 4 (each wave 128 x 64), BK 64, 2 stages.
//   staged M: 128 x 128, 4 waves as 2 x 2 (each wave 64 x 64), BK 64, 2 stages.
struct TileCfg {
    int bm, bn, wm, wn;
};
constexpr TileCfg kCfgL = {256, 256, 2, 4};
constexpr TileCfg kCfgM = {128, 128, 2, 2};
constexpr int kSkinnyNB = 2, kSkinnyKS = 4;
constexpr int kGroupM = 4;

// DMA-kernel variants: [in][out] entry points.
struct DmaVariant {
    const char* name;
    int bm, bn, bk, stages, wm, wn, swz;
    int lds_bytes;  // the ring: `stages` A+B stages, or five operand-tile slots
    const void* fn[5][4];  // [bf16, f16, e4m3, e5m2, int8][f32, bf16, f16, int32]
};

static bool is_fp8(int in_dtype) { return in_dtype == GEMM_BT_FP8_E4M3 || in_dtype == GEMM_BT_FP8_E5M2; }
// 8-bit inputs of either kind: 128-element K steps, whole 16-byte rows
static bool is_8bit(int in_dtype) { return is_fp8(in_dtype) || in_dtype == GEMM_BT_INT8; }
static int in_index(int in_dtype) {
    switch (in_dtype) {
        case GEMM_BT_BF16: return 0;
        case GEMM_BT_F16: return 1;
        case GEMM_BT_FP8_E4M3: return 2;
        case GEMM_BT_FP8_E5M2: return 3;
        default: return 4;
    }
}
static int out_index(int out_dtype) {
    switch (out_dtype) {
        case GEMM_BT_F32: return 0;
        case GEMM_BT_BF16: return 1;
        case GEMM_BT_F16: return 2;
        default: return 3;
    }
}
static int out_size(int out_dtype) { return out_dtype == GEMM_BT_F32 || out_dtype == GEMM_BT_INT32 ? 4 : 2; }

template <int BM, int BN, int BK, int S, int WM, int WN, int SWZ, int SCHED = 0, int PF = 0, int MF = 32,
          bool ALL = false, int LDW = 0, int RING5 = 0, bool F8 = false, int PH = 0>
static DmaVariant dma_variant(const char* name) {
    DmaVariant v = {name, BM, BN, BK, RING5 ? 5 : S, WM, WN, SWZ, 0, {}};
    // LDS: BK elements of 1 (8-bit inputs) or 2 bytes per tile row
    const int rowb = BK * (F8 ? 1 : 2);
    v.lds_bytes = RING5 ? 5 * BM * rowb : S * (BM + BN) * rowb;
    if constexpr (F8) {
        // tuning forms: E4M3 -> bf16 only
        v.fn[2][1] = (const void*)&dma_kernel<GEMM_BT_FP8_E4M3, GEMM_BT_BF16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
        if constexpr (ALL) {
            v.fn[2][0] = (const void*)&dma_kernel<GEMM_BT_FP8_E4M3, GEMM_BT_F32, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
            v.fn[2][2] = (const void*)&dma_kernel<GEMM_BT_FP8_E4M3, GEMM_BT_F16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
            v.fn[3][0] = (const void*)&dma_kernel<GEMM_BT_FP8_E5M2, GEMM_BT_F32, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
            v.fn[3][1] = (const void*)&dma_kernel<GEMM_BT_FP8_E5M2, GEMM_BT_BF16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
            v.fn[3][2] = (const void*)&dma_kernel<GEMM_BT_FP8_E5M2, GEMM_BT_F16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
            v.fn[4][3] = (const void*)&dma_kernel<GEMM_BT_INT8, GEMM_BT_INT32, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5>;
        }
    } else {
        v.fn[0][1] = (const void*)&dma_kernel<GEMM_BT_BF16, GEMM_BT_BF16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
        v.fn[1][2] = (const void*)&dma_kernel<GEMM_BT_F16, GEMM_BT_F16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
        if constexpr (ALL) {
            v.fn[0][0] = (const void*)&dma_kernel<GEMM_BT_BF16, GEMM_BT_F32, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
            v.fn[0][2] = (const void*)&dma_kernel<GEMM_BT_BF16, GEMM_BT_F16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
            v.fn[1][0] = (const void*)&dma_kernel<GEMM_BT_F16, GEMM_BT_F32, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
            v.fn[1][1] = (const void*)&dma_kernel<GEMM_BT_F16, GEMM_BT_BF16, BM, BN, BK, S, WM, WN, SWZ, SCHED, PF, MF, LDW, RING5, 0, PH>;
        }
    }
    return v;
}

// Geometry of a tile form that runs only split along K (its kernels are the
// split forms in sk_fn_t): no data-parallel entry points.
template <int BM, int BN, int BK, int S, int WM, int WN, int SWZ>
static DmaVariant split_only_variant(const char* name) {
    DmaVariant v = {name, BM, BN, BK, S, WM, WN, SWZ, S * (BM + BN) * BK * 2, {}};
    return v;
}

// Index 0 is the default for large grids, 7, 1, 8 and 9 for smaller ones, 2
// and 6 for the smallest (see plan_impl), 3..5 the same for 8-bit inputs, float or integer
// (128-element K steps: 128-byte tile rows, as for the 16-bit kernels; 32x32
// MFMAs over 64-element substeps); 10 and 11 run only split along K, for thin
// products (plan_split_rule), with 128-element K steps of 16-bit inputs
// (256-byte tile rows); 12..15 are 1, 8, 9 and 2 with the line ring.
// A build with GEMM_BT_TUNING defined adds the measured alternatives after
// them (selected with GEMM_BT_FORCE_TILE=<name>, bf16->bf16 and f16->f16
// only); the default library holds the production tile shapes only.
constexpr int kFp8Variants = 3;
constexpr int kTiny16 = 6;  // 32 x 64 tiles (16-bit inputs), when even 64 x 64 tiles leave half the CUs idle
constexpr int kWide16 = 7;  // 128 x 256 tiles (16-bit inputs, 8 waves of 64 x 64), see plan_impl
constexpr int kShort16 = 8;  // 96 x 128 tiles (16-bit inputs, 4 waves of 48 x 64), see plan_impl
constexpr int kNarrow16 = 9;  // 128 x 96 tiles (16-bit inputs, 4 waves of 64 x 48), see plan_impl
constexpr int kThin64 = 10;   // 64 x 64 tiles of 256-byte rows, split along K only (thin products)
constexpr int kThin32 = 11;   // 32 x 64 tiles of 256-byte rows, split along K only (thin products)
// The line-ring twins of the 128 x 128, 96 x 128, 128 x 96 and 64 x 64 tiers
// (dma_kernel PH = 1), for rows that are 16-byte but not 128-byte aligned.
constexpr int kRing128 = 12, kRingShort = 13, kRingNarrow = 14, kRing64 = 15;
static const DmaVariant* dma_variants(int* count) {
    static const DmaVariant v[] = {
        dma_variant<256, 256, 64, 2, 2, 4, 2, 6, 0, 16, true, 0, 2>("L64E16iR5s"),
        dma_variant<128, 128, 64, 4, 2, 2, 2, 8, 0, 16, true>("M64E4s4i"),
        dma_variant<64, 64, 64, 4, 2, 2, 2, 4, 0, 16, true>("Q64E4m16"),
        dma_variant<256, 256, 128, 2, 2, 4, 2, 6, 0, 32, true, 0, 2, true>("L128F8R5s"),
        dma_variant<128, 128, 128, 4, 2, 2, 2, 8, 0, 32, true, 0, 0, true>("M128F8s4i"),
        dma_variant<64, 64, 128, 4, 2, 2, 2, 4, 0, 32, true, 0, 0, true>("Q128F8"),
        dma_variant<32, 64, 64, 4, 2, 2, 2, 2, 0, 16, true>("T32x64"),
        dma_variant<128, 256, 64, 3, 2, 4, 2, 8, 0, 16, true>("H128x256s3"),
        dma_variant<96, 128, 64, 4, 2, 2, 2, 6, 0, 16, true>("M96x128s4"),
        dma_variant<128, 96, 64, 4, 2, 2, 2, 6, 0, 16, true>("M128x96s4"),
        split_only_variant<64, 64, 128, 4, 2, 2, 2>("Q64B128s4"),
        split_only_variant<32, 64, 128, 4, 2, 2, 2>("T32x64B128s4"),
        // the line ring (PH) twins of indices 1, 8 and 9
        dma_variant<128, 128, 64, 4, 2, 2, 2, 8, 0, 16, true, 0, 0, false, 1>("M64E4s4iP"),
        dma_variant<96, 128, 64, 4, 2, 2, 2, 6, 0, 16, true, 0, 0, false, 1>("M96x128s4P"),
        dma_variant<128, 96, 64, 4, 2, 2, 2, 6, 0, 16, true, 0, 0, false, 1>("M128x96s4P"),
        dma_variant<64, 64, 64, 4, 2, 2, 2, 4, 0, 16, true, 0, 0, false, 1>("Q64E4m16P"),
#ifdef GEMM_BT_TUNING
        dma_variant<256, 256, 64, 2, 2, 4, 2, 2, 0, 16>("L64E16"),
        dma_variant<128, 128, 64, 4, 2, 2, 2, 4, 0, 16>("M64E4s4m16"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 6, 0, 16>("L64E16i"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 6, 0, 16, false, 4>("L64E16iL4"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 6, 0, 16, false, 0, 1>("L64E16iR5"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 6, 0, 16, false, 4, 2>("L64E16iL4R5s"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 2>("L64E"),
        dma_variant<128, 128, 64, 4, 2, 2, 2, 4>("M64E4s4"),
        dma_variant<128, 128, 64, 4, 2, 2, 2, 5>("M64E4f2"),
        dma_variant<256, 256, 64, 2, 2, 4, 2>("L64S2"),
        dma_variant<256, 256, 64, 2, 2, 4, 0>("L64S2X0"),
        dma_variant<256, 256, 32, 4, 2, 4, 2>("L32S4"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 1>("L64PP"),
        dma_variant<256, 256, 64, 2, 2, 4, 2, 0, 2>("L64P2"),
        dma_variant<256, 128, 64, 3, 4, 2, 2, 8, 0, 16>("H256x128s3"),
        dma_variant<128, 256, 64, 2, 2, 4, 2, 8, 0, 16>("H128x256s2"),
        dma_variant<128, 128, 64, 2, 2, 2, 2, 8, 0, 16>("M64s2"),
        dma_variant<128, 96, 64, 5, 2, 2, 2, 6, 0, 16, true, 0, 0, false, 1>("M128x96s5P"),

#endif
    };
    *count = (int)(sizeof(v) / sizeof(v[0]));
    return v;
}

// Split-K forms (16-bit inputs, one item): a grid that splits the K range of
// every tile over several workgroups.  The 128 x 128 tier (M64E4s4i,
// dma_variants() index 1), and for thin products 64 x 64 and 32 x 64 tiles
// with 128-element K steps (indices 10 and 11): each piece then streams 256
// contiguous bytes of every B row per step instead of 128 (same box, us, 64-
// against 128-element steps: 64x8192x8192 35.5 vs 34.8, 24x8192x8192 35.3 vs
// 34.4, 32x4096x4096 15.5 vs 14.8, 64x4096x16384 f16 38.6 vs 37.8); and the
// 128 x 128 tier's line-ring twin (index 12) for rows 16-byte but not
// 128-byte aligned (us, plain vs line ring: 1000x1000x8200 -> f32 39.4 vs
// 32.8, 1024x1024x16392 68.0 vs 53.5, 512x1024x32776 f16 76.4 vs 60.5,
// 256x4096x8200 42.5 vs 37.5).  A tuning build also has the split form of the
// 128 x 256 tier (index 7; measured no faster: 1024x4096x4096 f16 43.1 us
// split 2 ways against 42.9 us unsplit on 128 x 128 tiles).
constexpr int kSkVariant = 1;
template <int IN, int OUT>
static const void* sk_fn_t(int variant) {
#ifdef GEMM_BT_TUNING
    if (variant == 7) return (const void*)&dma_kernel<IN, OUT, 128, 256, 64, 3, 2, 4, 2, 8, 0, 16, 0, 0, 1>;
#endif
    if (variant == kSkVariant) return (const void*)&dma_kernel<IN, OUT, 128, 128, 64, 4, 2, 2, 2, 8, 0, 16, 0, 0, 1>;
    if (variant == kRing128) return (const void*)&dma_kernel<IN, OUT, 128, 128, 64, 4, 2, 2, 2, 8, 0, 16, 0, 0, 1, 1>;
    if (variant == kThin64) return (const void*)&dma_kernel<IN, OUT, 64, 64, 128, 4, 2, 2, 2, 4, 0, 16, 0, 0, 1>;
    if (variant == kThin32) return (const void*)&dma_kernel<IN, OUT, 32, 64, 128, 4, 2, 2, 2, 2, 0, 16, 0, 0, 1>;
    return nullptr;  // no split form of this tile
}
template <int IN>
static const void* sk_fn_out(int out, int variant) {
    if (out == GEMM_BT_F32) return sk_fn_t<IN, GEMM_BT_F32>(variant);
    if (out == GEMM_BT_BF16) return sk_fn_t<IN, GEMM_BT_BF16>(variant);
    return sk_fn_t<IN, GEMM_BT_F16>(variant);
}
static const void* sk_fn(int variant, int in_dtype, int out_dtype) {
    return in_dtype == GEMM_BT_BF16 ? sk_fn_out<GEMM_BT_BF16>(out_dtype, variant)
                                    : sk_fn_out<GEMM_BT_F16>(out_dtype, variant);
}

// Workspace of the split kernels: a fixed area of arrival counters (one per
// split tile), then one slot of one fp32 tile per workgroup.
constexpr int64_t kSkCounterBytes = 16384;
constexpr int64_t kSkMaxTiles = kSkCounterBytes / 4;

// Scratch of gemm_bt_noalloc: the workspace of the largest split plan on a
// device of up to 256 CUs (counters, then one 128 x 128 fp32 slot per
// workgroup of a grid of at most 256), as a device array of the library's own.
// Every GPU the library runs on holds one copy (16.02 MiB) until the process
// ends.  It is zero when the code object is loaded, and every call leaves its
// counter area zero again.  Host code must not pass `scratch` itself to a
// kernel (on the host it names a stand-in, not device memory): it uses the
// per-device address from hipGetSymbolAddress (noalloc_scratch below).
constexpr int64_t kScratchBytes = kSkCounterBytes + 256 * 128 * 128 * 4;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Skinny DMA-kernel variants [in][out]; index 0 is the default.
struct SkinnyVariant {
    const char* name;
    int bn, kb, stages, waves;
    const void* fn[5][4];  // 16-bit inputs only: [bf16, f16][f32, bf16, f16]
};

template <int BN, int KB, int S, int W, bool ALL = false, int ROT = 0>
static SkinnyVariant skinny_variant(const char* name) {
    SkinnyVariant v = {name, BN, KB, S, W, {}};
    v.fn[0][1] = (const void*)&skinny_dma_kernel<GEMM_BT_BF16, GEMM_BT_BF16, BN, KB, S, W, ROT>;
    v.fn[1][2] = (const void*)&skinny_dma_kernel<GEMM_BT_F16, GEMM_BT_F16, BN, KB, S, W, ROT>;
    if constexpr (ALL) {
        v.fn[0][0] = (const void*)&skinny_dma_kernel<GEMM_BT_BF16, GEMM_BT_F32, BN, KB, S, W, ROT>;
        v.fn[0][2] = (const void*)&skinny_dma_kernel<GEMM_BT_BF16, GEMM_BT_F16, BN, KB, S, W, ROT>;
        v.fn[1][0] = (const void*)&skinny_dma_kernel<GEMM_BT_F16, GEMM_BT_F32, BN, KB, S, W, ROT>;
        v.fn[1][1] = (const void*)&skinny_dma_kernel<GEMM_BT_F16, GEMM_BT_BF16, BN, KB, S, W, ROT>;
    }
    return v;
}

static const SkinnyVariant* skinny_variants(int* count) {
    static const SkinnyVariant v[] = {
        skinny_variant<8, 256, 3, 1, true>("S8K256x3w1"),
#ifdef GEMM_BT_TUNING
        skinny_variant<16, 256, 4, 4>("S16K256x4"),
        skinny_variant<8, 256, 3, 2>("S8K256x3w2"),
        skinny_variant<8, 128, 4, 1>("S8K128x4w1"),
        skinny_variant<16, 256, 3, 1>("S16K256x3w1"),
        skinny_variant<32, 256, 6, 4>("S32K256x6"),
        skinny_variant<16, 256, 3, 1, false, 1>("S16K256x3w1r1"),
#endif
    };
    *count = (int)(sizeof(v) / sizeof(v[0]));
    return v;
}

#ifdef GEMM_BT_TUNING
constexpr int kSkinnyReg = -3;  // forced_skinny(): the register-streaming kernel
static int forced_skinny() {
    // Benchmarking aid: GEMM_BT_FORCE_SKINNY=<variant name>, or REG for the
    // register-streaming kernel.
    static std::atomic<int> cached{-2};
    int v = cached.load(std::memory_order_relaxed);
    if (v == -2) {
        v = -1;
        const char* e = std::getenv("GEMM_BT_FORCE_SKINNY");
        int n = 0;
        const SkinnyVariant* vs = skinny_variants(&n);
        for (int i = 0; e && i < n; ++i)
            if (std::strcmp(e, vs[i].name) == 0) v = i;
        if (e && std::strcmp(e, "REG") == 0) v = kSkinnyReg;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}

static bool forced_staged() {
    // Benchmarking aid: GEMM_BT_FORCE_TILE=STAGED runs the register-staged
    // kernel on 16-byte aligned rows too.
    static std::atomic<int> cached{-1};
    int v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("GEMM_BT_FORCE_TILE");
        v = (e && std::strcmp(e, "STAGED") == 0) ? 1 : 0;
        cached.store(v, std::memory_order_relaxed);
    }
    return v == 1;
}

static int forced_variant() {
    // Benchmarking aid: GEMM_BT_FORCE_TILE=<variant name> pins the DMA kernel shape.
    static std::atomic<int> cached{-2};
    int v = cached.load(std::memory_order_relaxed);
    if (v == -2) {
        v = -1;
        const char* e = std::getenv("GEMM_BT_FORCE_TILE");
        int n = 0;
        const DmaVariant* vs = dma_variants(&n);
        for (int i = 0; e && i < n; ++i)
            if (std::strcmp(e, vs[i].name) == 0) v = i;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}
#else
// The production library takes no tuning overrides.
constexpr int kSkinnyReg = -3;
static int forced_skinny() { return -1; }
static bool forced_staged() { return false; }
static int forced_variant() { return -1; }
#endif

static int pick_vec(int64_t K, int a_align, int b_align) {
    if (K % 8 == 0 && a_align % 16 == 0 && b_align % 16 == 0) return 8;
    if (K % 2 == 0 && a_align % 4 == 0 && b_align % 4 == 0) return 2;
    return 1;
}

// Largest batch: the batch index is the grid's y dimension.
constexpr int64_t kMaxBatch = 65535;

// 256x256 tiles for the LDS-DMA kernels: once they fill every CU, except
// just above one wave of them, where the last, nearly empty wave costs more
// than the 128x128 tiles' smaller per-tile reuse: up to 1.2 waves for 16-bit
// inputs (128x128 faster at 272-304 such tiles on 256 CUs), up to 17/16 waves
// for 8-bit ones (faster at 272 tiles, slower from 288 on).
static bool dma_large_tier(int64_t tiles_l, int num_cu, bool eight_bit) {
    if (tiles_l == num_cu) return true;
    return eight_bit ? tiles_l * 16 > (int64_t)num_cu * 17 : tiles_l * 5 > (int64_t)num_cu * 6;
}

// Split plan (the stream-K kernel with one piece per workgroup) for 16-bit
// inputs on the LDS-DMA path, one item: when the tiles of `variant` would fill
// at most half the CUs, each of the T tiles is split along K into
// S = floor(CUs / T) pieces of at least kSkMinSteps K steps (with
// fewer_pieces, into fewer pieces when K is too short for that many), and a
// grid of T * S workgroups computes one piece each.  Every workgroup's run of
// iterations then lies inside one tile, at the same K offset as the matching
// pieces of the other tiles, so workgroups sharing an operand panel read it
// in step, as in the plain grid.  Measured on 256 CUs, 128 x 128 tiles
// against the plain plan (us): 512x1024x32768 61 vs 121, 1024x1024x16384 51
// vs 73, 1024x2048x8192 47 vs 62, 512x2048x8192 34 vs 39, 256x4096x8192 35
// vs 41, 2048x1024x4096 27 vs 29; with pieces of 16 steps it loses
// (1024x1024x4096 22 vs 18.5), and so it does in fewer pieces of 32 steps
// (1024x1024x4096 in 2 pieces 22.3 vs 18.9, 256x4096x4096 28.5 vs 23.7).
// With more tiles than half the CUs (e.g. 192 tiles of 1000x3000), pieces
// that straddle tiles and start at different K offsets lose the panel reuse
// and the split lost everywhere it was measured (1000x3000x2050 33 vs 26.5,
// 1000x3000x8192 81 vs 65), so no split is planned there.
// Fills p and returns true, or returns false and leaves p alone.
constexpr int64_t kSkMinSteps = 32;
static bool plan_split(int64_t M, int64_t N, int64_t K, int variant, int num_cu, bool fewer_pieces,
                       gemm_bt_plan_t* p) {
    int n = 0;
    const DmaVariant& v = dma_variants(&n)[variant];
    const int64_t T = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
    const int64_t nk = ((K & ~7LL) + 63) / 64;
    if (T * 2 > num_cu || T > kSkMaxTiles) return false;
    const int64_t S = fewer_pieces ? std::min<int64_t>(num_cu / T, nk / kSkMinSteps) : num_cu / T;
    if (S < 2 || nk < kSkMinSteps * S) return false;
    p->kernel = KIND_DMA;
    p->variant = variant;
    p->bm = v.bm;
    p->bn = v.bn;
    p->bk = v.bk;
    p->stages = v.stages;
    p->threads = 64 * v.wm * v.wn;
    p->lds_bytes = v.lds_bytes;
    p->tiles_m = (M + v.bm - 1) / v.bm;
    p->tiles_n = (N + v.bn - 1) / v.bn;
    p->grid = T * S;
    p->split_tiles = T;
    p->workspace_bytes = kSkCounterBytes + p->grid * (int64_t)v.bm * v.bn * 4;
    return true;
}

// Which split, if any (the measured rule; see plan_split).  plain_tiles is
// the workgroup count of the plain plan.
//  * Thin products (M <= 64): 32 x 64 tiles for M <= 32, else 64 x 64, split
//    into as many pieces of 32 or more K steps as fill the CUs.  Per FLOP the
//    small tiles re-read B once per 32 or 64 rows of A; splitting K instead
//    of narrowing the tiles keeps that at once per row block and fills the
//    CUs all the same.  Measured (us, plain plan vs split): 64x8192x8192
//    40.6 vs 35.5, 48x8192x8192 42.6 vs 36.8, 17x8192x8192 39.8 vs 33.7,
//    64x4096x16384 f16 48.3 (128 x 128 tiles split) vs 38.4, 64x3072x8192
//    35.0 vs 20.7 (4 pieces), 32x4096x4096 20.7 vs 15.3 (2 pieces),
//    64x1024x65536 244 vs 45; 32 x 64 against 64 x 64 tiles for M <= 32:
//    24x8192x8192 35.3 vs 36.2, 32x4096x8192 23.1 vs 23.9.
//  * Otherwise 128 x 128 tiles, except when the plain grid already covers
//    every CU and M fills less than 3/4 of the 128-row tiles (their rows
//    are then mostly padding): 100x4096x16384 (rows 78 % full) splits at 47.7
//    against 65.4.
static bool plan_split_rule(int64_t M, int64_t N, int64_t K, int num_cu, int64_t plain_tiles, bool ring,
                            gemm_bt_plan_t* p) {
#ifdef GEMM_BT_TUNING
    if (const char* e = std::getenv("GEMM_BT_SPLIT_TILE")) return plan_split(M, N, K, std::atoi(e), num_cu, true, p);
#endif
    if (M <= 64) return plan_split(M, N, K, M <= 32 ? kThin32 : kThin64, num_cu, true, p);
    const int64_t rows = ((M + 127) / 128) * 128;
    if (plain_tiles >= num_cu && M * 4 < rows * 3) return false;
    return plan_split(M, N, K, ring ? kRing128 : kSkVariant, num_cu, false, p);
}

static int plan_impl(int64_t batch, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align,
                     int b_align, int c_align, int num_cu, bool allow_sk, gemm_bt_plan_t* p) {
    if (!p) return GEMM_BT_ERR_INVALID_VALUE;
    std::memset(p, 0, sizeof(*p));
    if (batch < 0 || M < 0 || N < 0 || K < 0) return GEMM_BT_ERR_INVALID_VALUE;
    if (batch > kMaxBatch) return GEMM_BT_ERR_UNSUPPORTED;
    p->batch = batch;
    if (in_dtype != GEMM_BT_BF16 && in_dtype != GEMM_BT_F16 && !is_8bit(in_dtype)) return GEMM_BT_ERR_UNSUPPORTED;
    if (out_dtype != GEMM_BT_F32 && out_dtype != GEMM_BT_BF16 && out_dtype != GEMM_BT_F16 && out_dtype != GEMM_BT_INT32)
        return GEMM_BT_ERR_UNSUPPORTED;
    // integer inputs give integer outputs, float inputs float outputs
    if ((in_dtype == GEMM_BT_INT8) != (out_dtype == GEMM_BT_INT32)) return GEMM_BT_ERR_UNSUPPORTED;
    // int8: every partial sum within int32 (|product| <= 2^14, K * 2^14 < 2^31)
    if (in_dtype == GEMM_BT_INT8 && K > 131071) return GEMM_BT_ERR_UNSUPPORTED;
    const int osz = out_size(out_dtype);
    // 32-bit buffer offsets inside one 256-row panel of A, B and C.
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF) return GEMM_BT_ERR_UNSUPPORTED;
    const int isz = is_8bit(in_dtype) ? 1 : 2;
    if (256 * K * isz >= 0x7FFFFFFFLL || 256 * N * (int64_t)osz >= 0x7FFFFFFFLL) return GEMM_BT_ERR_UNSUPPORTED;
    if (batch == 0 || M == 0 || N == 0) {
        p->kernel = KIND_NONE;
        return GEMM_BT_OK;
    }
    // the tile tiers count the workgroups of all batch items
    const int64_t tiles_l = ((M + 255) / 256) * ((N + 255) / 256) * batch;
    const int64_t tiles_m128 = ((M + 127) / 128) * ((N + 127) / 128) * batch;
    if (K == 0) {
        p->kernel = KIND_FILL;
        p->threads = 256;
        const int64_t n16 = M * N * osz / 2;
        int64_t g = (n16 + 255) / 256;
        p->grid = g < 4096 ? g : 4096;
        return GEMM_BT_OK;
    }
    // Row split: a single product with just over one wave of 256 x 256 tiles
    // (up to 1.375 waves; W waves up to W + 0.375) runs as two launches on the stream, the first
    // R * 256 rows as one wave of 256 x 256 tiles (R tile rows, at least 7/8
    // of the CUs) and the remaining rows on their own plan, split along K
    // where that plan allows.  Every tier that covers the whole product in
    // one grid leaves most CUs idle in its last wave.  Same box, us (the
    // 128 x 256 plan vs the sum of the two launches): 4352x4096x4096 147.7 vs
    // 97.8 + 23.7, 4160x4096x4096 145.6 vs 97.8 + 17.5, 4608x4096x4096 146.1
    // vs 97.8 + 30.0, 4352^2x4096 148.9 vs 97.8 + 34.4, 5120x4096x4096 152.4
    // vs 97.8 + 41.1, 4352x4096x2048 79.3 vs 55.2 + 12.1; 8-bit inputs alike
    // (E4M3 -> bf16: 4352x4096x4096 84.1 vs 55.6 + 12.4, 4608x4096x4096 86.1
    // vs 55.6 + 19.1, 5120x4096x4096 85.9 vs 55.6 + 23.6).  Past 1.375 waves
    // the second launch costs more than the last wave saves (6144x4096x4096
    // 163.2 vs 97.8 + 62.6, 5120^2x4096 166.4 vs 131.1 + 57.5).  Likewise
    // just past W >= 2 whole waves: the first launch is W waves (8448x4096x4096
    // 253.1 vs 191.3 + 23.6, 8704x4096x4096 251.3 vs 191.3 + 29.9,
    // 9216x4096x4096 251.6 vs 191.3 + 40.7, 8448x4096x2048 134.7 vs 102.8 +
    // 11.8, 12544x4096x4096 340.1 vs 280.3 + 23.6).
    const int64_t waves_l = tiles_l / num_cu;  // whole waves of 256 x 256 tiles
    const bool split_band = waves_l >= 1 && tiles_l % num_cu != 0 &&
                            (tiles_l - waves_l * num_cu) * 8 <= (int64_t)num_cu * 3;
    if (batch == 1 && !forced_staged() && forced_variant() < 0 && split_band) {
        const int64_t tn = (N + 255) / 256;
        const int64_t r1 = waves_l * num_cu / tn;  // tile rows of the first launch
        const int64_t m1 = r1 * 256;
        if (r1 * tn * 8 >= waves_l * num_cu * 7 && m1 < M) {
            gemm_bt_plan_t rest;
            int st = plan_impl(1, M - m1, N, K, in_dtype, out_dtype, a_align, b_align, c_align, num_cu, allow_sk,
                               &rest);
            if (st != GEMM_BT_OK) return st;
            st = plan_impl(1, m1, N, K, in_dtype, out_dtype, a_align, b_align, c_align, num_cu, allow_sk, p);
            if (st != GEMM_BT_OK) return st;
            p->split_rows = m1;
            if (rest.workspace_bytes > p->workspace_bytes) p->workspace_bytes = rest.workspace_bytes;
            return GEMM_BT_OK;
        }
    }
    // Item split: stacked items in the same bands run the first
    // floor(W * CUs / tiles per item) items as W waves of 256 x 256 tiles (at
    // least 7/8 of the CUs), then the remaining items (us, one launch on
    // 128 x 256 tiles vs the sum of the two launches): 17 items of
    // 256x4096x4096 192.1 vs 138.9 + 21.2, 9 of 512x4096x4096 171.2 vs 108.9 +
    // 33.8, 5 of 1024x4096x2048 85.6 vs 55.2 + 19.1.
    if (batch > 1 && !forced_staged() && forced_variant() < 0 && split_band) {
        const int64_t ti = tiles_l / batch;  // 256 x 256 tiles per item
        const int64_t z1 = waves_l * num_cu / ti;
        if (z1 >= 1 && z1 < batch && z1 * ti * 8 >= waves_l * num_cu * 7) {
            gemm_bt_plan_t rest;
            int st = plan_impl(batch - z1, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, num_cu, allow_sk,
                               &rest);
            if (st != GEMM_BT_OK) return st;
            st = plan_impl(z1, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, num_cu, allow_sk, p);
            if (st != GEMM_BT_OK) return st;
            p->split_items = z1;
            if (rest.workspace_bytes > p->workspace_bytes) p->workspace_bytes = rest.workspace_bytes;
            return GEMM_BT_OK;
        }
    }
    if (is_8bit(in_dtype)) {
        // 8-bit inputs: whole 16-byte chunks only (K a multiple of 16, A and B
        // 16-byte aligned), always the LDS-DMA kernel
        if (K % 16 != 0 || a_align % 16 != 0 || b_align % 16 != 0) return GEMM_BT_ERR_UNSUPPORTED;
        int n = 0;
        const DmaVariant* vs = dma_variants(&n);
        int use = kFp8Variants + (dma_large_tier(tiles_l, num_cu, true) ? 0 : (tiles_m128 * 2 > num_cu ? 1 : 2));
        // 256 x 256 tiles that fill at least half the CUs but not all, where
        // 128 x 128 ones need more than one wave (as for 16-bit inputs; us,
        // 128 x 128 vs 256 x 256, E4M3 -> bf16 and int8 -> int32):
        // 2048x4352x4096 (136 tiles) 50.6 vs 39.5, 3072^3 (144) 42.8 vs 34.0
        // and 46.1 vs 34.8, 2560x4096x4096 (160) 52.8 vs 43.3 and 55.5 vs
        // 43.2, 2000x6000x3008 (192) 48.9 vs 39.4, 3072x4096x4096 (192) 56.2 vs
        // 48.3 and 58.4 vs 47.7; at 100 tiles no better (2560^2x4096 36.2 vs
        // 37.1).
        if (use == kFp8Variants + 1 && tiles_l < num_cu && tiles_l * 2 >= num_cu && tiles_m128 > num_cu)
            use = kFp8Variants;
        const int f = forced_variant();
        if (f >= 0 && vs[f].fn[in_index(in_dtype)][out_index(out_dtype)]) use = f;
        const DmaVariant& v = vs[use];
        p->kernel = KIND_DMA;
        p->variant = use;
        p->vec = 16;
        p->bm = v.bm;
        p->bn = v.bn;
        p->bk = v.bk;
        p->stages = v.stages;
        p->threads = 64 * v.wm * v.wn;
        p->lds_bytes = v.lds_bytes;
        p->group_m = kGroupM;
        p->ksplit = 1;
        p->tiles_m = (M + p->bm - 1) / p->bm;
        p->tiles_n = (N + p->bn - 1) / p->bn;
        p->grid = p->tiles_m * p->tiles_n;
        if (p->grid * batch > 0x7FFFFFFF) return GEMM_BT_ERR_UNSUPPORTED;
        return GEMM_BT_OK;
    }
    p->vec = pick_vec(K, a_align, b_align);
    p->bk = 64;
    if (M <= 16) {
        p->kernel = KIND_SKINNY;
        p->bm = 16;
        p->tiles_m = 1;
        // the streaming DMA kernel takes rows of any (2-byte) alignment; the
        // register-streaming kernel is a tuning-build alternative
        const int f = forced_skinny();
        if (f != kSkinnyReg) {
            int n = 0;
            const SkinnyVariant* vs = skinny_variants(&n);
            int use = 0;
            if (f >= 0 && vs[f].fn[in_index(in_dtype)][out_index(out_dtype)]) use = f;
            const SkinnyVariant& v = vs[use];
            p->variant = 1 + use;
            p->bn = v.bn;
            p->bk = v.kb;
            p->stages = v.stages;
            p->ksplit = v.waves;
            p->threads = 64 * v.waves;
            const int nblk = v.bn < 16 ? 1 : v.bn / 16;
            p->lds_bytes = v.stages * (16 + v.bn) * v.kb * 2 + v.waves * nblk * 64 * 16;
        } else {
            p->variant = 0;
            p->bn = 16 * kSkinnyNB;
            p->bk = 32;
            p->stages = 2;
            p->ksplit = kSkinnyKS;
            p->threads = 64 * kSkinnyKS;
            p->lds_bytes = kSkinnyKS * kSkinnyNB * 64 * 16;
        }
        p->tiles_n = (N + p->bn - 1) / p->bn;
        p->grid = p->tiles_n;
        return GEMM_BT_OK;
    }
    const bool big = tiles_l >= num_cu;
    p->group_m = kGroupM;
#ifdef GEMM_BT_TUNING
    // tile-row band height of the banded order (GEMM_BT_GROUP_M=1 walks each die's run row by row)
    if (const char* e = std::getenv("GEMM_BT_GROUP_M")) p->group_m = std::atoi(e) > 0 ? std::atoi(e) : kGroupM;
#endif
    p->ksplit = 1;
    // the DMA kernel takes rows of any (2-byte) alignment; a K tail that is
    // not a whole 16-byte chunk is added after its loop
    if (!forced_staged()) {
        int n = 0;
        const DmaVariant* vs = dma_variants(&n);
        // 256x256 when that fills every CU (dma_large_tier); else 128x128
        // when its tiles fill more than half the CUs, else 64x64 (more
        // workgroups for what is then a thin or small, memory-bound product),
        // and 32x64 when even 64x64 tiles fill at most half the CUs
        int use = dma_large_tier(tiles_l, num_cu, false) ? 0 : (tiles_m128 * 2 > num_cu ? 1 : 2);
        const int64_t tiles_q64 = ((M + 63) / 64) * ((N + 63) / 64) * batch;
        if (use == 2 && tiles_q64 * 2 <= num_cu) use = kTiny16;
        // 128 x 256 tiles (8 waves, two per SIMD, each 64 x 64) instead of
        // 128 x 128 ones (4 waves, one per SIMD) once they make whole waves
        // or more than 1.375 waves: per FLOP they load 3/4 of the bytes, and
        // one wave's MFMAs cover the other's loads.  Measured (us, 128 x 128
        // vs 128 x 256 tiles): 2048x4096x4096 76.4 vs 61.3, 2048x4096x8192 f16
        // 140 vs 119, 2048x4096x2048 37.6 vs 33.4, 4608x4096x4096 153.5 vs
        // 148.0, 4352x4096x8192 305 vs 281; just above one wave no better
        // (3000x3000x4096, 1.125 waves, 95.3 vs 95.2).
        // Rows that are 16-byte but not 128-byte aligned: the 128-row tiers
        // below run their line-ring twins, and the 128 x 256 tier, whose
        // three stages leave no room for the ring's extra one, gives way to
        // 128 x 128 ring tiles (us, same box: 2048x4096x4104 84.5 vs 81.9,
        // 4100x4100x1000 87.2 vs 80.6).
        const bool ring = K % 8 == 0 && a_align % 16 == 0 && b_align % 16 == 0 && (K * 2) % 128 != 0;
        const int64_t tiles_h = ((M + 127) / 128) * ((N + 255) / 256) * batch;
        // Less than one wave of 256 x 256 tiles where 128-row tiles of either
        // width need more than one: the larger tiles win.  Per CU they load
        // half the bytes per FLOP of 128 x 128 ones, and a partly filled wave
        // runs each tile faster than a full one (the full chip is
        // power-bound).  Since a 128 x 256 grid has at most twice the tiles,
        // the 256 x 256 ones then fill more than half the CUs.  Measured (us,
        // the 128-row plan vs 256 x 256): 2048x4352x4096 (136 tiles) 92.6 vs
        // 75.5, 3000x3000x3072 (144) 68.9 vs 61.1, 2176x4224x4096 (153) 90.3
        // vs 73.9, 2560x4096x4096 (160) 96.2 vs 77.4, 3072x4096x4096 (192;
        // 128 x 256 tiles) 100.5 vs 85.4, 3584^3 (196) 87.4 vs 75.6.  Rows
        // that take the line ring have no 256 x 256 twin of it: there the
        // ring's 128-row tiles hold on to about 0.6 of the CUs (3000^3, 144
        // tiles, 71.5 vs 76.2; 2100x4300x3000, 153, 81.0 vs 87.8;
        // 4000x3000x5000, 192, 141.5 vs 124.3; 3072x4096x4104, 192, 108.7 vs
        // 100.6; 2000x6000x3000, 192, 108.6 vs 76.3).  Stacked items alike
        // (items x M x N x K): 9x1024x1024x4096 (144) 109.5 vs 78.7,
        // 10x1024x1024x2048 (160) 57.9 vs 44.7, 3x2048x2048x4096 (192) 102.6
        // vs 85.3, 2x2048x3072x4096 (192) 106.3 vs 83.9, 6x1024x2048x3000
        // (192, line ring) 89.6 vs 88.1.
        if (use == 1 && tiles_l < num_cu && tiles_h > num_cu &&
            (!ring || tiles_l * 5 >= (int64_t)num_cu * 3))
            use = 0;
        if (use == 1 && !ring && tiles_h >= num_cu && (tiles_h % num_cu == 0 || tiles_h * 8 > (int64_t)num_cu * 11))
            use = kWide16;
        // From 1.2 up to 1.375 waves of 256 x 256 tiles, 128 x 256 ones (more
        // than 2.4 waves) lose less to the last wave (us, 256 x 256 vs 128 x
        // 256, same box): 4608^2x4096 (324 tiles) 159.2 vs 146.9, x2048 86.3
        // vs 80.3, x8192 307.3 vs 304.5; 5120x4608x4096 (360) 158.5 vs 159.2;
        // 5120^2x4096 (400) 163.2 vs 194.2, 5376^2x4096 (441) 172.7 vs 197.2.
        if (use == 0 && !ring && tiles_l > num_cu && tiles_l * 8 <= (int64_t)num_cu * 11 &&
            tiles_h * 8 > (int64_t)num_cu * 11)
            use = kWide16;
        // One wave of 128 x 256 tiles where 128 x 128 ones need two (us, 128
        // x 128 vs 128 x 256): 2500^3 (400 vs 200 tiles) 66.2 vs 55.4,
        // 1500x4500x3500 (432 vs 216) 94.2 vs 87.5, 2500x2500x2496 51.3 vs 44.6,
        // 4 items of 1024x1536x4096 (384 vs 192) 73.3 vs 55.4, 8 of
        // 640x1024x4096 (320 vs 160) 69.9 vs 58.8.
        if (use == 1 && !ring && tiles_h <= num_cu && tiles_m128 > num_cu) use = kWide16;
        // 96 x 128 or 128 x 96 tiles instead of 128 x 128 ones for a single
        // product when they still make at most one wave and keep more CUs
        // busy: the CUs that would idle in the one wave then work.  Of the two,
        // the one with more tiles within the wave (96 x 128 on a tie).
        // Measured (us, 128 x 128 vs the narrower tile, bf16 unless noted):
        // 96 x 128: 768x4096x4096 37.1 vs 33.6, 3000x1000x4096 37.0 vs 32.1,
        // 1536x2048x4096 29.2 vs 26.4, 700x3200x4096 (150 vs 200 tiles) 33.2 vs
        // 29.6, 1152x2048x4096 26.6 vs 23.6, 768x4096x2048 16.9 vs 15.9,
        // 768x4096x8192 f16 69.4 vs 62.1, 760x4000x4104 48.3 vs 45.8;
        // 128 x 96: 1024x3072x4096 36.4 vs 33.3, 2048x1536x2048 17.3 vs 16.1,
        // 1000x3000x2048 -> f32 18.8 vs 17.7, 1000x3000x2050 -> f32 24.6 vs
        // 24.0.  With more tiles than CUs either loses (1000x3000x2050 on 264
        // tiles of 96 x 128: 24.3 vs 41.3).
        const int64_t tiles_s = ((M + 95) / 96) * ((N + 127) / 128);
        const int64_t tiles_n96 = ((M + 127) / 128) * ((N + 95) / 96);
        if (use == 1 && batch == 1) {
            const int64_t best = tiles_s <= num_cu ? tiles_s : 0, alt = tiles_n96 <= num_cu ? tiles_n96 : 0;
            if (alt > best && alt > tiles_m128) use = kNarrow16;
            else if (best > tiles_m128) use = kShort16;
        }
        // Several waves of 128 x 128 tiles: every wave costs a full one, the
        // last too, so 128 x 96 (or 96 x 128) tiles, whose waves take about
        // 0.9 of the time, win when they need no more waves, i.e. when 0.9 *
        // their waves < the 128 x 128 waves.  Measured (us, 128 x 128 vs
        // 128 x 96): 3000^3 (576 vs 768 tiles, 3 waves each) 79.0 vs 70.9,
        // 3072^3 75.5 vs 68.8; not where the narrower tiles need another wave
        // (2000x7000x3000 107.6 vs 113.9, 5000x2000x2000 57.5 vs 65.0,
        // 3000x4000x2048 54.3 vs 56.5).  Of the two, 128 x 96 (3000^3 70.9 vs
        // 76.7 for 96 x 128).
        if (use == 1 && batch == 1 && tiles_m128 > num_cu) {
            const int64_t w128 = (tiles_m128 + num_cu - 1) / num_cu;
            const int64_t wn = (tiles_n96 + num_cu - 1) / num_cu, ws = (tiles_s + num_cu - 1) / num_cu;
            if (9 * wn < 10 * w128) use = kNarrow16;
            else if (9 * ws < 10 * w128) use = kShort16;
        }
        // Rows that are 16-byte aligned but not 128-byte aligned: the 128-row
        // tiers load whole cache lines through the line ring (each 128-byte
        // K segment of such a row spans two lines).  Measured (us, same box,
        // plain vs line ring): 1024x4096x4104 f16 58.7 vs 44.5 (128 x 128),
        // 768x4096x4104 50.3 vs 39.0 (96 x 128), 1000x3000x3000 -> f32 32.4 vs
        // 28.7 and 1000x3000x2056 25.0 vs 22.8 (128 x 96).  It costs a stage of
        // prefetch depth, so aligned rows keep the plain ring (1000x3000x2048
        // 20.4 vs 22.2), and so does the 64 x 64 tier while its tiles fit one
        // workgroup per CU (1000x1000xK, 256 tiles: K = 1000 10.5 vs 11.1,
        // 4000 20.0 vs 24.0); with more tiles than CUs two workgroups share a
        // CU and the ring wins (1000x1500x3000 29.1 vs 23.2, 700x2000x3000
        // 31.0 vs 22.6, 1000x2000x1000 14.5 vs 13.2).  The 32 x 64 tier, used
        // only when even 64 x 64 tiles fill half the CUs, keeps its plain ring
        // (500x500x1000 8.5 vs 10.0).
        if (ring) {
            if (use == 1) use = kRing128;
            else if (use == kShort16) use = kRingShort;
            else if (use == kNarrow16) use = kRingNarrow;
            else if (use == 2 && tiles_q64 > num_cu) use = kRing64;
        }
        const int f = forced_variant();
        if (f >= 0 && vs[f].fn[in_index(in_dtype)][out_index(out_dtype)]) use = f;
        const DmaVariant& v = vs[use];
        p->kernel = KIND_DMA;
        p->variant = use;
        p->bm = v.bm;
        p->bn = v.bn;
        p->bk = v.bk;
        p->stages = v.stages;
        p->threads = 64 * v.wm * v.wn;
        p->lds_bytes = v.lds_bytes;
        const int64_t plain_tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn) * batch;
        if (allow_sk && f < 0 && batch == 1 && plan_split_rule(M, N, K, num_cu, plain_tiles, ring, p))
            return GEMM_BT_OK;
    } else {
        // tuning build only (GEMM_BT_FORCE_TILE=STAGED): the register-staged kernel
        const TileCfg c = big ? kCfgL : kCfgM;
        p->kernel = KIND_TILED;
        p->variant = big ? 0 : 1;
        p->bm = c.bm;
        p->bn = c.bn;
        p->stages = 2;
        p->threads = 64 * c.wm * c.wn;
        p->lds_bytes = 2 * (c.bm + c.bn) * 64 * 2;
    }
    p->tiles_m = (M + p->bm - 1) / p->bm;
    p->tiles_n = (N + p->bn - 1) / p->bn;
    p->grid = p->tiles_m * p->tiles_n;
    // the tiled kernels launch all items' tiles in one grid row
    if (p->grid * batch > 0x7FFFFFFF) return GEMM_BT_ERR_UNSUPPORTED;
    (void)c_align;
    return GEMM_BT_OK;
}

// Plan for operands stored K-outer (A as K x M and/or B as K x N): the
// 128 x 128 transpose-read kernel; 16-bit inputs with every operand row in
// whole, aligned 16-byte chunks.
static int plan_layout_impl(int64_t batch, int64_t M, int64_t N, int64_t K, int a_layout, int b_layout, int in_dtype,
                            int out_dtype, int a_align, int b_align, int c_align, int num_cu, gemm_bt_plan_t* p) {
    if (!p) return GEMM_BT_ERR_INVALID_VALUE;
    if ((a_layout != GEMM_BT_K_INNER && a_layout != GEMM_BT_K_OUTER) ||
        (b_layout != GEMM_BT_K_INNER && b_layout != GEMM_BT_K_OUTER)) {
        std::memset(p, 0, sizeof(*p));
        return GEMM_BT_ERR_INVALID_VALUE;
    }
    if (a_layout == GEMM_BT_K_INNER && b_layout == GEMM_BT_K_INNER)
        return plan_impl(batch, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, num_cu, false, p);
    std::memset(p, 0, sizeof(*p));
    if (batch < 0 || M < 0 || N < 0 || K < 0) return GEMM_BT_ERR_INVALID_VALUE;
    if (batch > kMaxBatch) return GEMM_BT_ERR_UNSUPPORTED;
    p->batch = batch;
    if (in_dtype != GEMM_BT_BF16 && in_dtype != GEMM_BT_F16) return GEMM_BT_ERR_UNSUPPORTED;
    if (out_dtype != GEMM_BT_F32 && out_dtype != GEMM_BT_BF16 && out_dtype != GEMM_BT_F16)
        return GEMM_BT_ERR_UNSUPPORTED;
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF) return GEMM_BT_ERR_UNSUPPORTED;
    const int osz = out_size(out_dtype);
    // 32-bit buffer offsets: a K-outer operand as a whole, a K-inner one per
    // 128-row panel, C per 128-row panel
    auto fits = [&](int layout, int64_t ext) {
        return layout == GEMM_BT_K_OUTER ? K * ext * 2 < 0x7FFFFFFFLL : 128 * K * 2 < 0x7FFFFFFFLL;
    };
    if (!fits(a_layout, M) || !fits(b_layout, N) || 128 * N * (int64_t)osz >= 0x7FFFFFFFLL)
        return GEMM_BT_ERR_UNSUPPORTED;
    if (batch == 0 || M == 0 || N == 0) {
        p->kernel = KIND_NONE;
        return GEMM_BT_OK;
    }
    if (K == 0) {
        p->kernel = KIND_FILL;
        p->threads = 256;
        const int64_t g = (M * N * osz / 2 + 255) / 256;
        p->grid = g < 4096 ? g : 4096;
        return GEMM_BT_OK;
    }
    // whole 16-byte chunks along every operand row, 16-byte aligned operands
    auto rows_ok = [&](int layout, int64_t ext, int align) {
        return align % 16 == 0 && (layout == GEMM_BT_K_OUTER ? ext % 8 == 0 : K % 8 == 0);
    };
    if (!rows_ok(a_layout, M, a_align) || !rows_ok(b_layout, N, b_align)) return GEMM_BT_ERR_UNSUPPORTED;
    // 256 x 256 tiles (8 waves) when the tiles of all items make exactly one
    // wave over the CUs or more than 1.375 waves, else 128 x 128 (4 waves):
    // just above one wave the nearly empty last wave costs more than the
    // smaller tiles' lower reuse (B stored K x N, 4096 x 4096 per item x M rows:
    // 128 x 128 tiles 8-17 % faster at 272-320 such tiles on 256 CUs, even at
    // 352, 4 % slower at 384)
    const int64_t tiles_l = ((M + 255) / 256) * ((N + 255) / 256) * batch;
    bool big = tiles_l == num_cu || tiles_l * 8 > (int64_t)num_cu * 11;
    // and when fewer 256 x 256 tiles than CUs fill at least half of them where
    // 128 x 128 ones need more than one wave (us, 128 vs 256, bf16, B stored
    // K x N unless noted): 2048x4352x4096 (136 tiles) 124.8 vs 98.3, 3072^3
    // (144) 82.2 vs 75.4, A stored K x M 84.0 vs 75.9, 2560x4096x4096 (160)
    // 106.3 vs 96.1, 3072x4096x4096 (192) 112.4 vs 98.6, both stored K-outer
    // 115.8 vs 108.0, 3 items of 2048x2048x4096 (192) 119.7 vs 103.3; at 100
    // tiles no better (2560^2x4096 63.9 vs 97.2)
    const int64_t tiles_128 = ((M + 127) / 128) * ((N + 127) / 128) * batch;
    if (tiles_l < num_cu && tiles_l * 2 >= num_cu && tiles_128 > num_cu) big = true;
#ifdef GEMM_BT_TUNING
    // GEMM_BT_LAYOUT_TILE=128 or 256 forces the tile size
    if (const char* e = std::getenv("GEMM_BT_LAYOUT_TILE")) big = std::atoi(e) == 256;
#endif
    const int bt = big ? 256 : 128;
    p->kernel = KIND_TRANS;
    p->variant = (a_layout == GEMM_BT_K_OUTER ? 1 : 0) + (b_layout == GEMM_BT_K_OUTER ? 2 : 0) - 1 + (big ? 3 : 0);
    p->bm = p->bn = bt;
    p->bk = 64;
    p->threads = big ? 512 : 256;
    p->vec = 8;
    p->group_m = kGroupM;
    p->ksplit = 1;
    p->stages = 2;
    p->lds_bytes = 2 * 2 * bt * 64 * 2;
    p->tiles_m = (M + bt - 1) / bt;
    p->tiles_n = (N + bt - 1) / bt;
    p->grid = p->tiles_m * p->tiles_n;
    if (p->grid * batch > 0x7FFFFFFF) return GEMM_BT_ERR_UNSUPPORTED;
    (void)c_align;
    return GEMM_BT_OK;
}

// transpose-read kernels [in: bf16, f16][out: f32, bf16, f16][variant: A K-outer, B K-outer, both; + 3 for the
// 256 x 256 tile]
template <int IN, int OUT, int BT, int W2>
static const void* trans_fn_t(int layouts) {
    if (layouts == 0) return (const void*)&trans_kernel<IN, OUT, true, false, BT, BT, 2, W2>;
    if (layouts == 1) return (const void*)&trans_kernel<IN, OUT, false, true, BT, BT, 2, W2>;
    return (const void*)&trans_kernel<IN, OUT, true, true, BT, BT, 2, W2>;
}
template <int IN, int OUT>
static const void* trans_fn_v(int variant) {
    return variant >= 3 ? trans_fn_t<IN, OUT, 256, 4>(variant - 3) : trans_fn_t<IN, OUT, 128, 2>(variant);
}
template <int IN>
static const void* trans_fn_out(int out, int variant) {
    if (out == GEMM_BT_F32) return trans_fn_v<IN, GEMM_BT_F32>(variant);
    if (out == GEMM_BT_BF16) return trans_fn_v<IN, GEMM_BT_BF16>(variant);
    return trans_fn_v<IN, GEMM_BT_F16>(variant);
}

// ---- kernel selection --------------------------------------------------------


#ifdef GEMM_BT_TUNING
constexpr int kSwz = 2;  // LDS swizzle of the register-staged kernel
template <int IN, int OUT, int VEC>
static const void* tiled_fn(int cfg) {
    if (cfg == 0)
        return (const void*)&staged_kernel<IN, OUT, kCfgL.bm, kCfgL.bn, kCfgL.wm, kCfgL.wn, VEC, kSwz>;
    return (const void*)&staged_kernel<IN, OUT, kCfgM.bm, kCfgM.bn, kCfgM.wm, kCfgM.wn, VEC, kSwz>;
}

template <int IN, int OUT>
static const void* tiled_fn_vec(int cfg, int vec) {
    if (vec == 8) return tiled_fn<IN, OUT, 8>(cfg);
    if (vec == 2) return tiled_fn<IN, OUT, 2>(cfg);
    return tiled_fn<IN, OUT, 1>(cfg);
}

template <int IN>
static const void* tiled_fn_out(int out, int cfg, int vec) {
    if (out == GEMM_BT_F32) return tiled_fn_vec<IN, GEMM_BT_F32>(cfg, vec);
    if (out == GEMM_BT_BF16) return tiled_fn_vec<IN, GEMM_BT_BF16>(cfg, vec);
    return tiled_fn_vec<IN, GEMM_BT_F16>(cfg, vec);
}

template <int IN, int OUT>
static const void* skinny_fn_vec(int vec) {
    if (vec == 2) return (const void*)&skinny_kernel<IN, OUT, kSkinnyNB, kSkinnyKS, 2>;
    return (const void*)&skinny_kernel<IN, OUT, kSkinnyNB, kSkinnyKS, 1>;
}

template <int IN>
static const void* skinny_fn_out(int out, int vec) {
    if (out == GEMM_BT_F32) return skinny_fn_vec<IN, GEMM_BT_F32>(vec);
    if (out == GEMM_BT_BF16) return skinny_fn_vec<IN, GEMM_BT_BF16>(vec);
    return skinny_fn_vec<IN, GEMM_BT_F16>(vec);
}
#endif

// ---- device checks -------------------------------------------------------------

constexpr int kMaxDev = 64;
static std::atomic<int> g_dev_state[kMaxDev];  // 0 unknown, 1 gfx950, 2 other
static std::atomic<int> g_dev_cus[kMaxDev];

static int check_device(int* num_cu) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return GEMM_BT_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDev) return GEMM_BT_ERR_NO_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_BT_ERR_NO_DEVICE;
        }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    if (st != 1) return GEMM_BT_ERR_NO_DEVICE;
    *num_cu = g_dev_cus[dev].load(std::memory_order_relaxed);
    return GEMM_BT_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU has its own copy at its own
// address).  NULL when the lookup fails.
static std::atomic<void*> g_scratch_ptr[kMaxDev];
static void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

static int align_of(const void* p) {
    const uintptr_t v = (uintptr_t)p;
    if (v % 16 == 0) return 16;
    if (v % 8 == 0) return 8;
    if (v % 4 == 0) return 4;
    if (v % 2 == 0) return 2;
    return 1;
}

// Alignment of every item's pointer in a batched call: the base pointer's,
// lowered by that of the byte stride between items.
static int item_align(const void* base, int64_t batch, int64_t stride, int esz) {
    const int a = align_of(base);
    if (batch <= 1 || stride == 0) return a;
    const int s = align_of((const void*)(uintptr_t)((uint64_t)stride * (uint64_t)esz));
    return a < s ? a : s;
}

// Checks shared by the batched entry points once the plan is known: items of
// C must not overlap, byte strides must fit 63 bits, pointers must be present
// and hold whole elements.
static int check_items(const void* A, const void* B, const void* C, int kind, int64_t batch, int64_t M, int64_t N,
                       int64_t stride_a, int64_t stride_b, int64_t stride_c, int isz, int osz) {
    if (batch > 1 && stride_c < M * N) return GEMM_BT_ERR_INVALID_VALUE;
    if (stride_a > (INT64_MAX >> 2) || stride_b > (INT64_MAX >> 2) || stride_c > (INT64_MAX >> 3))
        return GEMM_BT_ERR_INVALID_VALUE;
    if (!C) return GEMM_BT_ERR_INVALID_VALUE;
    if (kind != KIND_FILL && (!A || !B)) return GEMM_BT_ERR_INVALID_VALUE;
    if ((uintptr_t)A % isz || (uintptr_t)B % isz || (uintptr_t)C % osz) return GEMM_BT_ERR_INVALID_VALUE;
    return GEMM_BT_OK;
}

// CU count the plans are made for: the current device's when it is a
// gfx950, else 256 (an MI355X), so that a plan taken on the host describes the
// launch on the device that is present.
static int plan_cus() {
    int n = 256;
    return check_device(&n) == GEMM_BT_OK ? n : 256;
}

// Stream-K arguments of a plan: the counters at the start of the workspace,
// the partial-sum slots after them.  Zero for a data-parallel plan.
static SkArgs sk_args(const gemm_bt_plan_t& p, int64_t K, void* ws) {
    SkArgs a = {0, 0, 0, nullptr, nullptr};
    if (p.split_tiles > 0) {
        a.tiles = (int)p.split_tiles;
        a.pieces = (int)(p.grid / p.split_tiles);
        a.nk = (int)(((K & ~7LL) + p.bk - 1) / p.bk);
        a.counters = (unsigned*)ws;
        a.partials = (float*)((char*)ws + kSkCounterBytes);
    }
    return a;
}

// Every K-inner call: argument checks, the plan for the current device and
// the launch.  `ws` (with `ws_bytes`) enables the stream-K plan; NULL plans
// the data-parallel grid as gemm_bt does.
static int launch_inner(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                        int64_t stride_a, int64_t stride_b, int64_t stride_c, int in_dtype, int out_dtype, void* ws,
                        size_t ws_bytes, void* stream) {
    gemm_bt_plan_t p;
    if (stride_a < 0 || stride_b < 0 || stride_c < 0) return GEMM_BT_ERR_INVALID_VALUE;
    const bool multi = batch > 1;
    const int isz = is_8bit(in_dtype) ? 1 : 2;
    const int osz = out_size(out_dtype);
    const int a_al = item_align(A, batch, stride_a, isz), b_al = item_align(B, batch, stride_b, isz),
              c_al = item_align(C, batch, stride_c, osz);
    const bool allow_sk = ws != nullptr;
    // Plan against the default CU count first: it validates the arguments
    // without touching the device.
    int st = plan_impl(batch, M, N, K, in_dtype, out_dtype, a_al, b_al, c_al, 256, allow_sk, &p);
    if (st != GEMM_BT_OK) return st;
    if (p.kernel == KIND_NONE) return GEMM_BT_OK;
    st = check_items(A, B, C, p.kernel, batch, M, N, stride_a, stride_b, stride_c, isz, osz);
    if (st != GEMM_BT_OK) return st;

    int num_cu = 256;
    st = check_device(&num_cu);
    if (st != GEMM_BT_OK) return st;
    if (num_cu != 256) {
        st = plan_impl(batch, M, N, K, in_dtype, out_dtype, a_al, b_al, c_al, num_cu, allow_sk, &p);
        if (st != GEMM_BT_OK) return st;
    }
    if ((p.split_tiles > 0 || p.split_rows > 0 || p.split_items > 0) && p.workspace_bytes > 0 &&
        ((uintptr_t)ws % 16 != 0 || ws_bytes < (size_t)p.workspace_bytes))
        return GEMM_BT_ERR_INVALID_VALUE;
    if (p.split_rows > 0) {
        // two launches in stream order: rows [0, m1), then the rest (each
        // with its own plan; the second may use the workspace)
        const int64_t m1 = p.split_rows;
        st = launch_inner(A, B, C, 1, m1, N, K, 0, 0, 0, in_dtype, out_dtype, ws, ws_bytes, stream);
        if (st != GEMM_BT_OK) return st;
        return launch_inner((const char*)A + m1 * K * isz, B, (char*)C + m1 * N * osz, 1, M - m1, N, K, 0, 0, 0,
                            in_dtype, out_dtype, ws, ws_bytes, stream);
    }
    if (p.split_items > 0) {
        // items [0, z1), then the rest, in stream order (a stride of 0
        // shares that operand among the items of both launches)
        const int64_t z1 = p.split_items;
        st = launch_inner(A, B, C, z1, M, N, K, stride_a, stride_b, stride_c, in_dtype, out_dtype, ws, ws_bytes,
                          stream);
        if (st != GEMM_BT_OK) return st;
        return launch_inner((const char*)A + z1 * stride_a * isz, (const char*)B + z1 * stride_b * isz,
                            (char*)C + z1 * stride_c * osz, batch - z1, M, N, K, stride_a, stride_b, stride_c,
                            in_dtype, out_dtype, ws, ws_bytes, stream);
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    int Mi = (int)M, Ni = (int)N, Ki = (int)K;
    long long sa = multi ? (long long)stride_a * isz : 0, sb = multi ? (long long)stride_b * isz : 0,
              sc = multi ? (long long)stride_c * osz : 0;
    const unsigned gy = (unsigned)batch;

    if (p.kernel == KIND_FILL) {
        u16* c16 = (u16*)C;
        size_t n16 = (size_t)M * (size_t)N * osz / 2;
        void* args[] = {&c16, &n16, &sc};
        e = hipLaunchKernel((const void*)&zero_fill_kernel, dim3((unsigned)p.grid, gy), dim3(p.threads), args, 0, s);
    } else {
        const u16* a = (const u16*)A;
        const u16* b = (const u16*)B;
        // Vector stores need 4 consecutive outputs inside one row, aligned;
        // 2 = rows of C are also whole 16-byte chunks (the DMA kernel then
        // stores through LDS, whole rows per instruction).
        int vec_store = (N % 4 == 0) && c_al >= 4 * osz ? 1 : 0;
        if (vec_store && (N * osz) % 16 == 0 && c_al >= 16) vec_store = 2;
        if (p.kernel == KIND_DMA) {
            int n = 0;
            const void* fn = p.split_tiles > 0 ? sk_fn(p.variant, in_dtype, out_dtype)
                                               : dma_variants(&n)[p.variant].fn[in_index(in_dtype)][out_index(out_dtype)];
            if (!fn) return GEMM_BT_ERR_UNSUPPORTED;  // no kernel of this plan in this build
            SkArgs ska = sk_args(p, K, ws);
            // one grid row: the items stacked along the tile rows (stream-K: the persistent grid)
            int tm = (int)(p.tiles_m * batch), tn = (int)p.tiles_n, gm = p.group_m, itm = (int)p.tiles_m;
            const unsigned gx = (unsigned)(p.split_tiles > 0 ? p.grid : p.grid * batch);
            void* args[] = {&a, &b, &C, &Mi, &Ni, &Ki, &tm, &tn, &gm, &vec_store, &itm, &sa, &sb, &sc, &ska};
            e = hipLaunchKernel(fn, dim3(gx), dim3(p.threads), args, 0, s);
#ifdef GEMM_BT_TUNING
        } else if (p.kernel == KIND_TILED) {
            const void* fn = in_dtype == GEMM_BT_BF16 ? tiled_fn_out<GEMM_BT_BF16>(out_dtype, p.variant, p.vec)
                                                      : tiled_fn_out<GEMM_BT_F16>(out_dtype, p.variant, p.vec);
            int tm = (int)(p.tiles_m * batch), tn = (int)p.tiles_n, gm = p.group_m, itm = (int)p.tiles_m;
            void* args[] = {&a, &b, &C, &Mi, &Ni, &Ki, &tm, &tn, &gm, &vec_store, &itm, &sa, &sb, &sc};
            e = hipLaunchKernel(fn, dim3((unsigned)(p.grid * batch)), dim3(p.threads), args, 0, s);
#endif
        } else {
            const void* fn = nullptr;
            if (p.variant >= 1) {
                int n = 0;
                fn = skinny_variants(&n)[p.variant - 1].fn[in_index(in_dtype)][out_index(out_dtype)];
            } else {
#ifdef GEMM_BT_TUNING
                fn = in_dtype == GEMM_BT_BF16 ? skinny_fn_out<GEMM_BT_BF16>(out_dtype, p.vec)
                                              : skinny_fn_out<GEMM_BT_F16>(out_dtype, p.vec);
#endif
            }
            if (!fn) return GEMM_BT_ERR_UNSUPPORTED;  // no kernel of this plan in this build
            void* args[] = {&a, &b, &C, &Mi, &Ni, &Ki, &vec_store, &sa, &sb, &sc};
            e = hipLaunchKernel(fn, dim3((unsigned)p.grid, gy), dim3(p.threads), args, 0, s);
        }
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_BT_ERR_LAUNCH;
    }
    return GEMM_BT_OK;
}

}  // namespace gbt

using namespace gbt;

extern "C" {

int gemm_bt_version(void) { return 20000; }

const char* gemm_bt_status_string(int status) {
    switch (status) {
        case GEMM_BT_OK: return "ok";
        case GEMM_BT_ERR_INVALID_VALUE: return "invalid value";
        case GEMM_BT_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case GEMM_BT_ERR_NO_DEVICE: return "no gfx950 HIP device";
        case GEMM_BT_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int gemm_bt_plan(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align, int b_align,
                 int c_align, gemm_bt_plan_t* plan) {
    return plan_impl(1, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, plan_cus(), false, plan);
}

int gemm_bt_plan_ws(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align, int b_align,
                    int c_align, gemm_bt_plan_t* plan) {
    return plan_impl(1, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, plan_cus(), true, plan);
}

int gemm_bt_workspace_size(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, size_t* bytes) {
    if (!bytes) return GEMM_BT_ERR_INVALID_VALUE;
    *bytes = 0;
    gemm_bt_plan_t p;
    const int st = plan_impl(1, M, N, K, in_dtype, out_dtype, 256, 256, 256, plan_cus(), true, &p);
    if (st == GEMM_BT_OK) *bytes = (size_t)p.workspace_bytes;
    return st;
}

int gemm_bt_plan_batched(int64_t batch, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align,
                         int b_align, int c_align, gemm_bt_plan_t* plan) {
    return plan_impl(batch, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, plan_cus(), false, plan);
}

int gemm_bt_plan_layout(int64_t M, int64_t N, int64_t K, int a_layout, int b_layout, int in_dtype, int out_dtype,
                        int a_align, int b_align, int c_align, gemm_bt_plan_t* plan) {
    return plan_layout_impl(1, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align, c_align,
                            plan_cus(), plan);
}
int gemm_bt_layout(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int a_layout, int b_layout,
                   int in_dtype, int out_dtype, void* stream) {
    return gemm_bt_batched_layout(A, B, C, 1, M, N, K, 0, 0, 0, a_layout, b_layout, in_dtype, out_dtype, stream);
}

int gemm_bt_batched_layout(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                           int64_t stride_a, int64_t stride_b, int64_t stride_c, int a_layout, int b_layout,
                           int in_dtype, int out_dtype, void* stream) {
    if (a_layout == GEMM_BT_K_INNER && b_layout == GEMM_BT_K_INNER)
        return gemm_bt_batched(A, B, C, batch, M, N, K, stride_a, stride_b, stride_c, in_dtype, out_dtype, stream);
    gemm_bt_plan_t p;
    if (stride_a < 0 || stride_b < 0 || stride_c < 0) return GEMM_BT_ERR_INVALID_VALUE;
    const bool multi = batch > 1;
    const int osz = out_size(out_dtype);
    const int a_al = item_align(A, batch, stride_a, 2), b_al = item_align(B, batch, stride_b, 2),
              c_al = item_align(C, batch, stride_c, osz);
    int st = plan_layout_impl(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_al, b_al, c_al, 256, &p);
    if (st != GEMM_BT_OK) return st;
    if (p.kernel == KIND_NONE) return GEMM_BT_OK;
    st = check_items(A, B, C, p.kernel, batch, M, N, stride_a, stride_b, stride_c, 2, osz);
    if (st != GEMM_BT_OK) return st;
    int num_cu = 256;
    st = check_device(&num_cu);
    if (st != GEMM_BT_OK) return st;
    if (num_cu != 256) {
        st = plan_layout_impl(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_al, b_al, c_al, num_cu, &p);
        if (st != GEMM_BT_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    long long sa = multi ? (long long)stride_a * 2 : 0, sb = multi ? (long long)stride_b * 2 : 0,
              sc = multi ? (long long)stride_c * osz : 0;
    if (p.kernel == KIND_FILL) {
        u16* c16 = (u16*)C;
        size_t n16 = (size_t)M * (size_t)N * osz / 2;
        void* args[] = {&c16, &n16, &sc};
        e = hipLaunchKernel((const void*)&zero_fill_kernel, dim3((unsigned)p.grid, (unsigned)batch), dim3(p.threads),
                            args, 0, s);
    } else {
        const u16* a = (const u16*)A;
        const u16* b = (const u16*)B;
        int vec_store = (N % 4 == 0) && c_al >= 4 * osz ? 1 : 0;
        if (vec_store && (N * osz) % 16 == 0 && c_al >= 16) vec_store = 2;
        const void* fn = in_dtype == GEMM_BT_BF16 ? trans_fn_out<GEMM_BT_BF16>(out_dtype, p.variant)
                                                  : trans_fn_out<GEMM_BT_F16>(out_dtype, p.variant);
        // one grid row: the items stacked along the tile rows
        int Mi = (int)M, Ni = (int)N, Ki = (int)K, tm = (int)(p.tiles_m * batch), tn = (int)p.tiles_n, gm = p.group_m,
            itm = (int)p.tiles_m;
        void* args[] = {&a, &b, &C, &Mi, &Ni, &Ki, &tm, &tn, &gm, &vec_store, &itm, &sa, &sb, &sc};
        e = hipLaunchKernel(fn, dim3((unsigned)(p.grid * batch)), dim3(p.threads), args, 0, s);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_BT_ERR_LAUNCH;
    }
    return GEMM_BT_OK;
}

int gemm_bt_plan_batched_layout(int64_t batch, int64_t M, int64_t N, int64_t K, int a_layout, int b_layout,
                                int in_dtype, int out_dtype, int a_align, int b_align, int c_align,
                                gemm_bt_plan_t* plan) {
    return plan_layout_impl(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align, c_align,
                            plan_cus(), plan);
}

int gemm_bt_tile_coord(int64_t pid, int64_t tiles_m, int64_t tiles_n, int group_m, int64_t* tm, int64_t* tn) {
    if (!tm || !tn || tiles_m <= 0 || tiles_n <= 0 || group_m <= 0) return GEMM_BT_ERR_INVALID_VALUE;
    if (pid < 0 || pid >= tiles_m * tiles_n) return GEMM_BT_ERR_INVALID_VALUE;
    tile_coord(pid, tiles_m, tiles_n, group_m, tm, tn);
    return GEMM_BT_OK;
}

int gemm_bt(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
            void* stream) {
    return launch_inner(A, B, C, 1, M, N, K, 0, 0, 0, in_dtype, out_dtype, nullptr, 0, stream);
}

int gemm_bt_batched(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                    int64_t stride_a, int64_t stride_b, int64_t stride_c, int in_dtype, int out_dtype, void* stream) {
    return launch_inner(A, B, C, batch, M, N, K, stride_a, stride_b, stride_c, in_dtype, out_dtype, nullptr, 0, stream);
}

int gemm_bt_ws(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
    return launch_inner(A, B, C, 1, M, N, K, 0, 0, 0, in_dtype, out_dtype, workspace, workspace_bytes, stream);
}

int gemm_bt_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype,
                    int out_dtype, void* stream) {
    gemm_bt_plan_t p;
    int st = plan_impl(1, M, N, K, in_dtype, out_dtype, 256, 256, 256, plan_cus(), true, &p);
    if (st != GEMM_BT_OK) return st;
    if (p.workspace_bytes > kScratchBytes) return GEMM_BT_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (p.workspace_bytes > 0) {
        int num_cu = 0;
        st = check_device(&num_cu);  // a gfx950 must be current before its scratch is looked up
        if (st != GEMM_BT_OK) return st;
        ws = noalloc_scratch();
        if (!ws) return GEMM_BT_ERR_NO_DEVICE;
    }
    return launch_inner(A, B, C, 1, M, N, K, 0, 0, 0, in_dtype, out_dtype, ws, ws ? (size_t)kScratchBytes : 0,
                        stream);
}

}  // extern "C"
