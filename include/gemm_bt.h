/*
 * gemm_bt.h -- C = A * B^T on one AMD Instinct MI355X (gfx950).
 *
 * The operation.  C[i][j] = sum_k A[i][k] * B[j][k] for 0 <= i < M, 0 <= j < N,
 * with A stored M x K row-major and B stored N x K row-major, i.e. B is kept
 * transposed so both operands are read along K ("Optimizing Blackwell matrix
 * multiplication in Mojo (part 2)", sections "Starting from the 4-line kernel"
 * and "Kernel 2: TMA and Tensor Core", where B is laid out row_major(N, K) so
 * its loads coalesce).  Inputs are bf16, f16 or one of the OCP 8-bit float
 * formats E4M3 / E5M2 (both operands the same type, as the MMA contract of
 * "Writing Mosaic GPU kernels with Pallas", section "MMA (TensorCore)",
 * requires; the pages list 8-bit floats among the supported MMA element
 * types); products are accumulated in fp32 and the
 * result is rounded once, to nearest even, into the output type ("Chapter 7:
 * Writing custom kernels with Pallas", section 4.1': fp32 accumulator, cast
 * only after the last K step).  8-bit integer inputs (two's complement) are
 * the integer MMA operand type of the same Mosaic GPU section, with an int32
 * accumulator: there C is the exact int32 sum, and int8 in requires int32
 * out (and int32 out requires int8 in).  C is overwritten: there is no
 * alpha/beta.
 *
 * Layout.  Dense and contiguous: lda = ldb = K elements, ldc = N elements.
 * For 16-bit inputs pointers need only element alignment (2 bytes, 4 bytes for
 * fp32 output); 16-byte alignment together with K % 8 == 0 selects the
 * widest loads and is a performance matter only.  8-bit inputs (float or
 * integer) need whole 16-byte rows: K % 16 == 0 and A, B 16-byte aligned
 * (else UNSUPPORTED).  int8 inputs also need K <= 131071, so that no sum can
 * leave the int32 range (|A[i][k] * B[j][k]| <= 2^14).
 *
 * Ownership.  The caller owns A, B and C (device memory, e.g. from PyTorch),
 * and the workspace of gemm_bt_ws.  The library allocates nothing per call,
 * keeps no pointer after it returns and holds no state beyond a per-device
 * cache of device attributes.
 *
 * Asynchrony and errors.  gemm_bt enqueues its kernel on `stream` (two
 * kernels in stream order for a plan with split_rows or split_items) and
 * returns without waiting.  Argument errors are reported before anything is
 * enqueued.  A launch failure is reported as GEMM_BT_ERR_LAUNCH; a fault
 * inside the kernel shows at the caller's next synchronisation.  No call
 * throws, exits or aborts.  Calls are thread-safe.  C must not overlap A or B.
 */
#ifndef GEMM_BT_H
#define GEMM_BT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
    GEMM_BT_F32 = 0,      /* IEEE binary32 (output only) */
    GEMM_BT_F16 = 1,      /* IEEE binary16 */
    GEMM_BT_BF16 = 2,     /* bfloat16: the upper 16 bits of a binary32 */
    GEMM_BT_FP8_E4M3 = 3, /* OCP 8-bit E4M3 (input only): bias 7, no infinities, max 448 */
    GEMM_BT_FP8_E5M2 = 4, /* OCP 8-bit E5M2 (input only): bias 15, IEEE-style infinities */
    GEMM_BT_INT8 = 5,     /* two's-complement 8-bit integer (input only; output GEMM_BT_INT32) */
    GEMM_BT_INT32 = 6     /* two's-complement 32-bit integer (output only; input GEMM_BT_INT8) */
} gemm_bt_dtype;

/* Operand layouts for gemm_bt_layout. */
typedef enum {
    GEMM_BT_K_INNER = 0, /* A stored M x K, B stored N x K (K contiguous): the gemm_bt layout */
    GEMM_BT_K_OUTER = 1  /* A stored K x M (M contiguous), B stored K x N (N contiguous) */
} gemm_bt_layout_t;

/* Status codes returned by every entry point. */
typedef enum {
    GEMM_BT_OK = 0,
    GEMM_BT_ERR_INVALID_VALUE = 1, /* negative size, null pointer with data, bad plan pointer */
    GEMM_BT_ERR_UNSUPPORTED = 2,   /* dtype combination or size outside the supported range */
    GEMM_BT_ERR_NO_DEVICE = 3,     /* no HIP device, or it is not a gfx950 */
    GEMM_BT_ERR_LAUNCH = 4         /* the kernel launch failed */
} gemm_bt_status;

/*
 * C = A * B^T.
 *   A          device pointer, M x K elements of in_dtype, row-major
 *   B          device pointer, N x K elements of in_dtype, row-major (B^T stored)
 *   C          device pointer, M x N elements of out_dtype, row-major; overwritten
 *   M, N, K    sizes, each in [0, 2^31 - 1]; M*K, N*K and M*N elements must each
 *              fit below 2^31 bytes per 256-row panel (checked: UNSUPPORTED);
 *              8-bit inputs: K % 16 == 0 and A, B 16-byte aligned (UNSUPPORTED);
 *              int8 inputs: K <= 131071 (UNSUPPORTED)
 *   in_dtype   GEMM_BT_BF16, GEMM_BT_F16, GEMM_BT_FP8_E4M3, GEMM_BT_FP8_E5M2 or GEMM_BT_INT8
 *   out_dtype  GEMM_BT_F32, GEMM_BT_BF16 or GEMM_BT_F16 for float inputs; GEMM_BT_INT32
 *              for GEMM_BT_INT8 inputs (any other pairing: UNSUPPORTED)
 *   stream     hipStream_t to enqueue on; NULL means the default stream
 * M == 0 or N == 0: nothing is enqueued, returns GEMM_BT_OK.
 * K == 0: C is filled with zeros (the empty sum) on `stream`.
 * The device is the caller's current HIP device.
 */
int gemm_bt(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
            int in_dtype, int out_dtype, void* stream);

/*
 * Batched product: C_z = A_z * B_z^T for z = 0 .. batch-1, every item with
 * the same sizes and types ("Chapter 7: Writing custom kernels with Pallas",
 * section 5.2: batching a kernel adds a leading grid dimension and runs the
 * unchanged kernel once per item; an operand mapped with in_axes=None is
 * shared by all items rather than copied).  One launch covers all items.
 *   A, B, C    base device pointers; item z uses A + z*stride_a, B + z*stride_b
 *              and C + z*stride_c (strides in elements of the operand's type)
 *   batch      number of items, 0 .. 65535 (0: nothing enqueued; more: UNSUPPORTED)
 *   stride_a   >= 0; 0 shares one A between all items (likewise stride_b for B)
 *   stride_c   >= M*N when batch > 1, so items of C never overlap (INVALID_VALUE)
 * Strides are ignored when batch == 1.  Alignment rules apply to every item's
 * pointers (the base pointers and the strides in bytes): e.g. 8-bit inputs
 * need 16-byte aligned A and B items.  Everything else is as for gemm_bt,
 * which is the batch == 1 case of this call.  Negative sizes or strides:
 * INVALID_VALUE.
 */
int gemm_bt_batched(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                    int64_t stride_a, int64_t stride_b, int64_t stride_c, int in_dtype, int out_dtype,
                    void* stream);

/*
 * C = op(A) * op(B)^T with either operand stored K-outer ("Writing Mosaic GPU
 * kernels with Pallas", section "MMA (TensorCore)", transposed operands: for
 * 16-bit operands an A of shape (K, M), and likewise a B of shape (K, N), is
 * accepted and transposed by the hardware).  a_layout = GEMM_BT_K_OUTER: A is
 * K x M row-major; b_layout = GEMM_BT_K_OUTER: B is K x N row-major, so
 * (K_INNER, K_OUTER) is the plain C = A * B.  Both K_INNER is exactly gemm_bt.
 * Operands stored K-outer are transposed inside the kernel (LDS transpose
 * reads); nothing is copied.  Requirements (else UNSUPPORTED): bf16 or f16
 * inputs; every operand row in whole 16-byte chunks (M % 8 == 0 for a K-outer
 * A, N % 8 == 0 for a K-outer B, K % 8 == 0 for a K-inner operand) and A, B
 * 16-byte aligned; a K-outer operand below 2 GiB.  An unknown layout value is
 * INVALID_VALUE.  Everything else (C, sizes, K == 0, streams, errors) is as
 * for gemm_bt.
 */
int gemm_bt_layout(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int a_layout,
                   int b_layout, int in_dtype, int out_dtype, void* stream);

/*
 * Batched products with operand layouts: gemm_bt_batched's items (item z at
 * A + z*stride_a, B + z*stride_b, C + z*stride_c elements; a stride of 0
 * shares an operand; stride_c >= M*N when batch > 1) with each operand stored
 * as gemm_bt_layout's a_layout / b_layout say.  An item of a K-outer A is a
 * K x M matrix, of a K-outer B a K x N one.  The rules of both calls apply, to
 * every item's pointers; gemm_bt_layout is the batch == 1 case and
 * gemm_bt_batched the (K_INNER, K_INNER) one.
 */
int gemm_bt_batched_layout(const void* A, const void* B, void* C, int64_t batch, int64_t M, int64_t N, int64_t K,
                           int64_t stride_a, int64_t stride_b, int64_t stride_c, int a_layout, int b_layout,
                           int in_dtype, int out_dtype, void* stream);

/*
 * C = A * B^T with a caller-provided workspace that lets the library split
 * the K range of output tiles over workgroups (the work split of stream-K:
 * "Writing Mosaic GPU kernels with Pallas", section "Cluster launch
 * control", a grid that keeps every core busy to the end).  Where a 16-bit
 * product would leave at least half the compute units without an output
 * tile and K is long, each of its T tiles is split into S pieces of
 * consecutive K steps (at least 32 steps of 64 each), one piece per
 * workgroup.  The tiles: 32 x 64 for M <= 32, 64 x 64 for M <= 64 (thin
 * products, in K steps of 128, e.g. 64 x 8192 x 8192: 128 tiles, S = 2),
 * else 128 x 128 (e.g.
 * 1024 x 1024 x 16384: 64 tiles, S = 4); S = floor(CUs / T), for thin
 * products at most K / 2048 (then S >= 2 is required), and for 128 x 128 tiles
 * no split when M fills less than 3/4 of their rows while narrower tiles
 * already give every compute unit a workgroup.  The last of a tile's
 * workgroups to finish adds the pieces in K
 * order (piece 0 + 1 + ...), whatever the order of arrival, so the result
 * is the same bits on every run with the same sizes on the same device.
 * The sum of each output is then formed in a different order than gemm_bt's
 * (pieces summed in fp32, then added), with the same accuracy bound.  Where
 * no split is planned (every other shape, batches, 8-bit inputs, operands
 * stored K-outer) the call is exactly gemm_bt.
 *   A, B, C, M, N, K, in_dtype, out_dtype, stream: as for gemm_bt
 *   workspace        device memory of at least workspace_bytes, 16-byte
 *                    aligned, owned by the caller, or NULL (then the call is
 *                    gemm_bt).  Its first 16 KiB must hold zeros before the
 *                    first call that uses it (e.g. hipMemset once after
 *                    allocation); every call leaves them zero again, so one
 *                    workspace serves any number of later calls with no
 *                    clearing.  Calls that share a workspace must not run
 *                    concurrently (one stream, or ordered by events).
 *   workspace_bytes  its size; smaller than gemm_bt_workspace_size reports for
 *                    these sizes: INVALID_VALUE (nothing enqueued)
 * Everything else (sizes, dtypes, K == 0, alignment, errors) is as for gemm_bt.
 */
int gemm_bt_ws(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype,
               int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_bt_ws without a workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the split plan's counters and partial sums live in a scratch
 * array of the library's own in device memory, 16 KiB + 16 MiB (the largest
 * split plan on a GPU of up to 256 compute units), one copy per GPU, held
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  Same arguments, plan, kernels and results as
 * gemm_bt_ws with a large enough workspace (bit for bit); where no split is
 * planned it is gemm_bt.  A plan that would need more scratch than that
 * (more than 256 compute units): UNSUPPORTED, nothing enqueued.  All calls on
 * one GPU share its scratch, whose counters are zero when the library is
 * loaded and are left zero by every call: calls that overlap in time on one
 * GPU (different streams, or concurrent host threads without ordering) race
 * on it and must not be issued.
 */
int gemm_bt_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype,
                    int out_dtype, void* stream);

/* Workspace gemm_bt_ws needs for these sizes and types (0 when it runs the
   plain grid), for the current device (256 compute units without one).  At
   most 16 KiB + 256 * 64 KiB (16.02 MiB) on an MI355X, whatever the
   sizes.  Returns gemm_bt's status for invalid arguments. */
int gemm_bt_workspace_size(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, size_t* bytes);

/* Human-readable text for a status code (static storage; never NULL). */
const char* gemm_bt_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gemm_bt_version(void);

/*
 * Launch plan: which kernel and tile shape gemm_bt would use for a problem;
 * lets callers and tests see the tiling and the grid.  No kernel runs.  The
 * plan is made for the current device's compute-unit count when it is a
 * gfx950 (one cached device query), else for 256 (an MI355X).  `a_align`,
 * `b_align`, `c_align` are the byte alignments of the pointers that would be
 * passed (e.g. 256 for fresh allocations).
 */
typedef struct {
    int kernel;       /* 0 = none (empty), 1 = zero fill (K == 0), 2 = LDS-tiled MFMA with register-staged
                         loads (no longer planned: kind 4 takes every row alignment), 3 = skinny streaming
                         (M <= 16), 4 = LDS-tiled MFMA with direct global->LDS loads, 5 = LDS-tiled MFMA
                         with LDS transpose reads (an operand stored K-outer) */
    int variant;      /* tile-shape variant index within the kernel family */
    int bm, bn, bk;   /* workgroup tile (rows of C, columns of C, K step) */
    int threads;      /* threads per workgroup */
    int vec;          /* elements per global load: 16 (16 bytes of 8-bit data), 8 (16 bytes), 2 or 1 */
    int group_m;      /* tile-rows per group in the grouped tile order */
    int ksplit;       /* waves that split K inside a workgroup (skinny kernel) */
    int stages;       /* LDS pipeline depth: A+B stages (tiled kernels), or for the 256x256 tile the 5 slots of
                         its ring of single-operand tiles */
    int lds_bytes;    /* LDS per workgroup */
    int64_t tiles_m, tiles_n;
    int64_t grid;     /* workgroups per batch item (grid * batch are launched); for a split plan the
                         workgroups of the one launch (split_tiles * pieces per tile) */
    int64_t batch;    /* batch items (1 for gemm_bt) */
    int64_t split_tiles;     /* split plan: tiles whose K range is split over several workgroups (0: one
                                workgroup per tile) */
    int64_t workspace_bytes; /* workspace the plan needs (0 unless a launch of it splits tiles along K) */
    int64_t split_rows;      /* > 0: the product runs as two launches in stream order, rows [0, split_rows)
                                of C first, planned as the fields above describe (one wave of 256 x 256
                                tiles), then the remaining rows on their own plan; 0: one launch */
    int64_t split_items;     /* > 0: stacked items run as two launches in stream order, items
                                [0, split_items) first, planned as the fields above describe (one wave of
                                256 x 256 tiles), then the remaining items on their own plan; 0: one launch */
} gemm_bt_plan_t;

int gemm_bt_plan(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align,
                 int b_align, int c_align, gemm_bt_plan_t* plan);

/* The plan of gemm_bt_ws given a large enough workspace (the plan gemm_bt_ws
   runs when its workspace is not NULL). */
int gemm_bt_plan_ws(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, int a_align,
                    int b_align, int c_align, gemm_bt_plan_t* plan);

/* The plan of gemm_bt_layout (for kernel 5 the variant is 0: A K-outer, 1: B
   K-outer, 2: both, on 128 x 128 tiles; 3, 4, 5 the same on 256 x 256 tiles). */
int gemm_bt_plan_layout(int64_t M, int64_t N, int64_t K, int a_layout, int b_layout, int in_dtype, int out_dtype,
                        int a_align, int b_align, int c_align, gemm_bt_plan_t* plan);

/* The plan of gemm_bt_batched_layout. */
int gemm_bt_plan_batched_layout(int64_t batch, int64_t M, int64_t N, int64_t K, int a_layout, int b_layout,
                                int in_dtype, int out_dtype, int a_align, int b_align, int c_align,
                                gemm_bt_plan_t* plan);

/* The plan of gemm_bt_batched: the tile tier counts the workgroups of all
   items; the alignments are those of every item's pointers. */
int gemm_bt_plan_batched(int64_t batch, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                         int a_align, int b_align, int c_align, gemm_bt_plan_t* plan);

/*
 * Tile order used by the tiled kernel: workgroup `pid` (0 <= pid < tiles_m *
 * tiles_n) computes output tile (tm, tn).  Workgroups are first regrouped by
 * the XCD (accelerator die, 8 on MI355X, each with its own L2) that the
 * hardware dispatches them to, round-robin, so that each die receives a
 * contiguous run of tiles; that run is then walked in bands of `group_m`
 * tile-rows, column by column inside a band, so that tiles running at the
 * same time share A-row and B-row panels in L2 ("Writing Mosaic GPU kernels
 * with Pallas", section "Using the L2 cache": reorder the grid into bands of
 * mt rows so that concurrently scheduled blocks touch less data).  A batched
 * call stacks its items along the tile rows (tiles_m = batch * tile rows per
 * item), so each die receives whole items and their panels stay in its L2.
 * Host-callable copy of the device function; returns INVALID_VALUE for a pid
 * outside the grid.
 */
int gemm_bt_tile_coord(int64_t pid, int64_t tiles_m, int64_t tiles_n, int group_m, int64_t* tm,
                       int64_t* tn);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BT_H */
