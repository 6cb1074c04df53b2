/*
 * moe.h -- C ABI of the MI355X (gfx950) fused MoE expert-FFN forward.
 *
 * The library computes, on one GPU's local experts, the expert FFN of a
 * mixture-of-experts layer: a planner that groups the top-k routes by expert
 * (moe_align), then for every routed token row the gate/up GEMM, SwiGLU, an
 * on-chip requantization of the intermediate, the down GEMM and the top-k
 * weighted combine (fused_moe_*).
 *
 * Sources (web pages on fused MoE kernels):
 *   [hpc-ops RFC]  "[RFC] Fused W8A8 MoE megakernel on H20", sections
 *                  "Background" (the five stages) and "Design" (planner +
 *                  compute kernel).
 *   [prime-flash]  "Prime Flash MoE: Fused MoE Kernels for Blackwell",
 *                  sections "API", "Shapes", "Scale layout (mxfp8)",
 *                  "Constraints" and the introduction (split / fused modes).
 *   [DeepGEMM #88] "[SM90] Ring-buffered FP8 MegaMoE with a lag-ordered L1/L2
 *                  schedule", section "Before you merge" (per-128 FP8
 *                  requantization expression of the intermediate).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers are DEVICE pointers unless an argument says "host".  All tensors
 *   are dense and row-major (C order), and must be 16-byte aligned.
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Every call only enqueues work on `stream`: it never synchronizes with the
 *   device and never copies between host and device.
 * - The caller allocates and owns every buffer, including the workspace.  The
 *   library allocates no device memory and keeps no state between calls.
 * - So a planner + forward sequence can be captured into a HIP graph on a
 *   capturing stream and replayed: every clear the library does is a kernel,
 *   not a memset node.  A replay reads whatever the captured buffers hold at
 *   that time (new routing, new tokens); it keeps the captured sizes
 *   (T, block_m, mode) and pointers.
 * - Return value: MOE_OK (0) or a negative moe_status.  All argument checks
 *   run on the host BEFORE anything is enqueued, so on an error nothing has
 *   been launched.  moe_last_error() returns a message for the last failing
 *   call of the calling thread (host string owned by the library).
 * - Numbers: e4m3 means OCP FP8 E4M3FN (bias 7, max 448, no infinities);
 *   e8m0 means the OCP MX power-of-two scale 2^(c-127); bf16 is bfloat16.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* negative / zero / inconsistent sizes */
  MOE_ERR_UNSUPPORTED = -3, /* a size or option this build does not cover */
  MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -6          /* a HIP launch failed; message has the text */
} moe_status;

typedef enum {
  MOE_BF16 = 0,          /* bf16 x, w1, w2; fp32 accumulate */
  MOE_FP8_BLOCKWISE = 1, /* e4m3 with fp32 scales per 1x128 (x) and 128x128 (w) */
  MOE_MXFP8 = 2,         /* e4m3 with e8m0 scales per 32 along the contraction */
  MOE_MXFP4 = 3          /* weights e2m1 + e8m0 per 32; activations as MOE_MXFP8 */
} moe_dtype;

/*
 * Overrides of the kernel schedule for tuning sweeps ([prime-flash] "Tuning"
 * and "Constraints": its block_n / warp_n / stages knobs are exposed to the
 * caller rather than chosen inside; the gfx950 kernels here have knobs of
 * their own).  Pass NULL, or leave a field 0, for the library's choice.  A
 * set field must be a value the call's kernels support, else the call
 * fails with MOE_ERR_UNSUPPORTED before anything is launched; the result
 * does not depend on the knobs beyond fp32 summation order.
 *   k_groups  streaming gate/up kernels (block_m 16 or 32, split 0 or 1): K
 *             groups per workgroup, 1 or 2 (2 needs K >= 256); each group
 *             of 4 waves walks part of K and the groups' sums are added in
 *             a fixed order.
 *   k_split   split mode, block_m 16 or 32, or 64 with an e4m3 dtype
 *             (blockwise FP8, MXFP8: the LDS-tiled kernels): gate/up
 *             workgroups per (block, 128-wide slice) tile, 1 or 4 (4 needs
 *             K / 128 a multiple of 8 and at least 16, at block_m 16 or 32
 *             two K groups, and workspace for the partial sums:
 *             moe_workspace_size with the same tune).
 *   prefetch  streaming kernels (block_m 16 or 32, split 0 or 1, k_split 1):
 *             K steps each wave keeps in flight, 1, 2 or 4.
 *   stages    LDS-tiled kernels (e4m3 dtypes, split mode, block_m 64 or
 *             128): pipeline stages, 2 or 3.
 */
typedef struct moe_tune {
  int32_t k_groups;
  int32_t k_split;
  int32_t prefetch;
  int32_t stages;
} moe_tune;

/* Message describing the last error of the calling thread ("" if none).
 * Every entry point returns a status ([prime-flash] "Constraints": the
 * shape and alignment rules a call must meet are checked, and a violation
 * is reported, before any work is done); this is its text. */
const char* moe_last_error(void);

/*
 * Capacities of the planner outputs for any routing of T tokens with top_k
 * routes each over E experts ([prime-flash] "Shapes": sorted_token_ids and
 * expert_ids are sized for the worst-case padding; "API": moe_align pads
 * each expert's rows to a multiple of block_m):
 *   *sorted_cap = T*top_k + min(E, T*top_k) * (block_m - 1)
 *   *blocks_cap = ceil(*sorted_cap / block_m)
 * (each non-empty expert pads fewer than block_m rows).  Host out-params.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (T < 0, top_k < 1, E < 1,
 * T*top_k >= 2^31), MOE_ERR_UNSUPPORTED (block_m not 16, 32, 64, 128 or 256).
 */
int moe_align_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m,
                       int64_t* sorted_cap, int64_t* blocks_cap);

/*
 * Planner ([hpc-ops RFC] "Design": expert histogram, prefix sums and the
 * row-to-token mapping; [prime-flash] "API" moe_align and "Shapes").
 *
 *   topk_ids                 (T, top_k) int32, expert id of each route.
 *   sorted_token_ids  [out]  (sorted_cap) int32: the flat pair ids
 *                            t*top_k + j grouped by expert (experts in
 *                            ascending id, ids ascending inside an expert),
 *                            each expert padded to a multiple of block_m
 *                            with -1, and -1 from num_tokens_post_padded to
 *                            the end.
 *   expert_ids        [out]  (blocks_cap) int32: expert of each block_m
 *                            block; -1 for blocks past the last used one.
 *   num_tokens_post_padded [out] int32[1]: padded row count (multiple of
 *                            block_m).
 * Routes whose expert id is outside [0, E) are not placed (they contribute
 * nothing downstream).  Experts with no route get no block.  The output is
 * unique (bit-exact, deterministic).  E must be <= 1024.
 * Errors: as moe_align_capacity, plus MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED
 * (E > 1024), MOE_ERR_HIP.  T == 0 writes the all -1 outputs and a 0 count.
 */
int moe_align(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
              int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
              int32_t* num_tokens_post_padded, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace of moe_align: *bytes (host out) = 0 at or below 16,384 routes
 * (T * top_k), else 4 * ceil(T * top_k / 512) * E.  With at least that
 * many bytes at `ws` (device, 16-byte aligned, contents undefined on
 * return; concurrent calls need separate workspaces) moe_align plans over
 * chunks of 512 route ids in three launches (per-chunk expert counts, which
 * also set the outputs to -1; one workgroup turning them into per-chunk
 * cursors and the block owners; one wave per chunk scattering its ids in
 * order: [hpc-ops RFC] "Design", histogram, prefix sums, row-to-token
 * mapping, with the grid-wide dependencies at kernel boundaries).  With no
 * workspace (ws NULL or ws_bytes smaller) one workgroup plans every call.
 * The outputs are the same bits either way.  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE.
 */
int moe_align_workspace_size(int64_t T, int32_t top_k, int32_t E, size_t* bytes);

/*
 * Router and planner in one launch.  The gate's routing arrives at the
 * planner as topk_ids and topk_weights ([prime-flash] "Usage"); the weights
 * are the normalized routing weights ([hpc-ops RFC] "Results so far"); the
 * planner is a grid-wide dependency ([hpc-ops RFC] "Design"), so the
 * workgroups route their tokens and the last one to finish runs the planner.
 *
 *   logits                   (T, E) fp32 router logits, row-major; -inf marks
 *                            an expert masked for that token.
 *   topk_ids          [out]  (T, top_k) int32: the top_k largest logits of
 *                            each token in descending order, equal logits to
 *                            the lower expert id first (bit-exact).
 *   topk_weights      [out]  (T, top_k) fp32: softmax over all E experts,
 *                            renormalized over the selection (equivalently
 *                            exp(l_j - l_max) / sum_sel exp(l_i - l_max)),
 *                            fp32 arithmetic: within a few ulp of the exact
 *                            value.
 *   sorted_token_ids, expert_ids, num_tokens_post_padded [out]:
 *                            exactly moe_align's outputs for that topk_ids.
 *   ws, ws_bytes             device workspace of at least
 *                            moe_route_align_workspace_size bytes, 16-byte
 *                            aligned, its first 256 bytes all ZERO before
 *                            the first call that uses it; every call leaves
 *                            them zero.  Calls that may overlap need
 *                            separate workspaces.  Past 16,384 routes, a
 *                            workspace of 256 + moe_align_workspace_size(T,
 *                            top_k, E) bytes or more makes the launch route
 *                            only, and moe_align's chunked planner follow
 *                            it (same outputs).
 * E <= 1024, 1 <= top_k <= min(16, E).  NaN logits are not supported.
 * Errors: as moe_align, plus MOE_ERR_UNSUPPORTED (top_k > 16 or > E),
 * MOE_ERR_WORKSPACE (ws_bytes too small).  T == 0 writes moe_align's T == 0
 * outputs.
 */
int moe_route_align_workspace_size(size_t* bytes);
int moe_route_align(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                    int32_t* expert_ids, int32_t* num_tokens_post_padded, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * The planner of moe_align / moe_align_shared (n_shared = 0 for the former)
 * for many routes.  One workgroup plans the whole call in moe_align, which
 * keeps every dependency a workgroup barrier; past 16,384 routes
 * (T * (top_k + n_shared)) moe_align_ws instead plans over chunks of 512
 * route ids in three launches: per-chunk expert counts (which also set the
 * output to -1), one workgroup turning them into per-chunk cursors and the
 * block owners, one wave per chunk
 * scattering its ids in order ([hpc-ops RFC] "Design": histogram, prefix
 * sums, row-to-token mapping).  The outputs are those of moe_align(_shared),
 * bit for bit.
 *   moe_align_ws_size: *bytes (host out) = workspace bytes the call needs:
 *     0 at or below 16,384 routes (workspace unused, may be NULL), else
 *     4 * ceil(routes / 512) * (E + n_shared).
 *   workspace: device memory, 16-byte aligned, contents undefined on return;
 *     concurrent calls need separate workspaces.
 * Errors: as moe_align / moe_align_shared, plus MOE_ERR_WORKSPACE.
 */
int moe_align_ws_size(int64_t T, int32_t top_k, int32_t E, int32_t n_shared, size_t* bytes);
int moe_align_ws(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t n_shared,
                 int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                 int32_t* num_tokens_post_padded, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Mode choice by size ([prime-flash] introduction: split=False keeps the
 * intermediate on chip and accumulates a split-K down projection into the
 * output; split=True writes the H-wide activation once and runs the down
 * projection with no split-K, trading one HBM round trip for a reduction
 * cost that grows with token count; [hpc-ops RFC] "Results so far": the
 * fused kernel helps small-token workloads).  On MI355X the split mode
 * streams the weights faster wherever they set the time; the fused mode is
 * picked only for T*top_k <= 512 with at most 32 MB of expert weights, where
 * its one launch fewer matters.
 *   *split (host out) = 1 for split mode, 0 for the fused mode.
 * Errors: MOE_ERR_NULL.
 */
int moe_select_split(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E,
                     int32_t top_k, int32_t block_m, int32_t* split);

/*
 * Suggested block_m for a call (small blocks for decode-sized batches, so
 * that padding does not dominate; larger blocks once experts hold many
 * rows; 256 only where the dtype and K allow it).  The choice follows the
 * mean routes per active expert, assuming here that the T*top_k routes
 * spread evenly over min(T*top_k, E) experts.  *block_m is a host
 * out-param.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE.
 */
int moe_select_block_m(int32_t dtype, int64_t T, int64_t K, int32_t top_k, int32_t E,
                       int32_t* block_m);

/*
 * The same, with the number of experts that hold at least one route
 * (active_experts, in [0, E]).  The count is a host value: a caller that
 * routes on the device takes it from an earlier step or from its own
 * routing statistics, since reading it back would synchronize; inside a
 * captured graph, moe_select_block_m needs no count.  A skewed routing concentrates the routes on few experts,
 * which then hold many rows each: blockwise FP8 at K=7168, I=3072, E=384,
 * T=256 under a zipf routing (59 active experts, 26 rows each) runs in
 * 961 us with 64-row tiles against 1389 us with the 16-row blocks the
 * even-spread estimate (4 rows per expert) picks.  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE.
 */
int moe_select_block_m_routed(int32_t dtype, int64_t T, int64_t K, int32_t top_k, int32_t E,
                              int32_t active_experts, int32_t* block_m);

/*
 * Workspace bytes a fused_moe_* call with these sizes and this tune (NULL:
 * none) needs (host out-param; [prime-flash] introduction: split=True writes
 * the H-wide activation to memory once, which here lives in the caller's
 * workspace with the per-route down outputs in bf16; split=False accumulates
 * into an fp32 buffer).  split = -1 means "as moe_select_split picks"; for split = 2
 * (ring mode) the size with the default ring (see moe_ring_layout).
 * Errors: as the fused calls' size and tune checks.
 */
int moe_workspace_size(int32_t dtype, int64_t T, int64_t K, int64_t N,
                       int32_t E, int32_t top_k, int32_t block_m,
                       int32_t split, const moe_tune* tune, size_t* bytes);

/*
 * Ring-mode workspace ([DeepGEMM #88] "How it works": the intermediate pool
 * becomes a ring of block slots; "What the bound moves": the ring capacity
 * is the buffer's).  A split = 2 call takes
 *   slots = min(blocks_cap, (workspace_bytes - *fixed_bytes) / *slot_bytes)
 * ring slots of block_m intermediate rows (at least one is required); with
 * one slot per planner block the ring never wraps.  Host out-params:
 *   *fixed_bytes    bytes ahead of the ring (control words, flags, per-route
 *                   rows)
 *   *slot_bytes     bytes per slot (block_m rows of values and scales)
 *   *default_slots  the slots moe_workspace_size(.., split = 2, ..) provides:
 *                   twice the lag of a 512-workgroup grid (the launch uses
 *                   one workgroup per CU), plus two, capped at blocks_cap;
 *                   the lag is 1.5 x the grid / (I/128) blocks
 * block_m must be 16 or 32.  Errors: MOE_ERR_NULL, and as moe_workspace_size.
 */
int moe_ring_layout(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E,
                    int32_t top_k, int32_t block_m, size_t* fixed_bytes,
                    size_t* slot_bytes, int64_t* default_slots);

/*
 * The ring mode's task stream, for inspection (host only, no device work;
 * [DeepGEMM #88] "How it works": a block's down tasks sit lag units after
 * its up tasks).  For n_blocks planner blocks with up_per_block = I/128
 * gate/up tasks and down_per_block = ceil(K/256) down tasks each, ticket t
 * (t = first .. first + count - 1) is described by kind[j] (1 up, 2 down,
 * 0 past the end of the stream), block[j] and index[j] (the slice of I, or
 * the 256-column tile of the output).  Rounds r = 0, 1, .. hold the up
 * tasks of block r, then the down tasks of block r - lag; tickets
 * 0 .. n_blocks * (up_per_block + down_per_block) - 1 cover every task once.
 * A call's lag is below its ring's slot count.  kind, block, index: host
 * arrays of count int32.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE.
 */
int moe_ring_schedule(int32_t n_blocks, int32_t up_per_block, int32_t down_per_block,
                      int32_t lag, int64_t first, int64_t count, int32_t* kind,
                      int32_t* block, int32_t* index);

/*
 * Byte offsets, inside the workspace of a split-mode call, of the
 * requantized intermediate: rows follow sorted_token_ids positions
 * (sorted_cap rows), I = N/2 columns.
 *   *h_offset      values: bf16 (rows, I) / e4m3 (rows, I)
 *   *hs_offset     scales: fp32 (rows, I/128) blockwise, e8m0 (rows, I/32) MX,
 *                  unused (equal to *h_offset) for bf16
 * Rows whose sorted id is -1 hold unspecified bytes.  For inspection only.
 * Errors: as moe_workspace_size.
 */
int moe_workspace_layout(int32_t dtype, int64_t T, int64_t K, int64_t N,
                         int32_t E, int32_t top_k, int32_t block_m,
                         size_t* h_offset, size_t* hs_offset);

/*
 * Fused expert FFN forward ([hpc-ops RFC] "Background" stages 1-5:
 * gather, gate/up grouped GEMM, SwiGLU + requantization, down grouped GEMM,
 * top-k weighted reduction; [prime-flash] "API" / "Shapes").
 *
 * Common arguments (all three dtypes):
 *   sorted_token_ids, expert_ids, num_tokens_post_padded
 *                    moe_align outputs for the same topk_ids, E and block_m
 *                    (read on the device; no host synchronization).
 *   topk_weights     (T, top_k) fp32 routing weights.
 *   out       [out]  (T, K) bf16.  EVERY element is written: a token whose
 *                    routes are all outside [0, E) gets zeros.  out is
 *                    sum_j topk_weights[t, j] * y_j summed in fp32 with one
 *                    rounding to bf16; in split and ring mode each route's
 *                    row y_j is first held in bf16 in the workspace (the
 *                    combine buffer of [DeepGEMM #88] "The rest of the
 *                    memory numbers": two bytes per token, route and
 *                    column).
 *   T, K, N, E, top_k, block_m
 *                    tokens, hidden size, fused gate+up width (N = 2I; rows
 *                    [0, I) of w1 are the gate, [I, N) the up projection),
 *                    experts, routes per token, planner block.
 *                    K % 128 == 0 and I % 128 == 0 are required.
 *                    block_m is 16, 32, 64 or 128, or 256 for the e4m3
 *                    dtypes when K % 256 == 0 (split mode only).
 *   split            -1: choose by size (moe_select_split); 0: fused mode
 *                    (the intermediate stays on chip, the down GEMM is
 *                    split-K over 128-wide slices of I accumulated in fp32);
 *                    1: split mode (the requantized intermediate is written
 *                    to the workspace once, the down GEMM runs with no
 *                    split-K, and the combine is deterministic: the same
 *                    inputs give bitwise the same output);
 *                    2: ring mode, block_m 16 or 32 ([DeepGEMM #88] "How it
 *                    works"): one persistent grid runs the split mode's
 *                    gate/up and down tiles from a lag-ordered task stream,
 *                    the intermediate in a ring of block slots sized by the
 *                    workspace (moe_ring_layout); bitwise equal to split
 *                    mode.  Its waits are bounded: the int at byte offset 4
 *                    of the workspace is nonzero after a call in which one
 *                    gave up (a broken invariant; the output is then
 *                    invalid).
 *   tune             NULL, or schedule overrides (moe_tune above).
 *   workspace, workspace_bytes
 *                    device scratch of at least moe_workspace_size bytes
 *                    (same sizes, split and tune);
 *                    contents undefined on return; concurrent calls need
 *                    separate workspaces.
 *   stream           hipStream_t as void*.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP.  T == 0 is a successful no-op.
 */

/* bf16 path: x (T, K), w1 (E, N, K), w2 (E, K, N/2), all bf16.  The
 * intermediate is rounded to bf16 before the down GEMM. */
int fused_moe_bf16(const void* x, const void* w1, const void* w2,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded,
                   const float* topk_weights, void* out, int64_t T, int64_t K,
                   int64_t N, int32_t E, int32_t top_k, int32_t block_m,
                   int32_t split, const moe_tune* tune, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Blockwise FP8 W8A8 path ([hpc-ops RFC] "Background": blockwise FP8 MoE;
 * [DeepGEMM #88] "Before you merge": the intermediate is requantized per
 * row and 128 columns with amax floored at 1e-10, sf = amax*(1/448),
 * sf_inv = 1/sf, q = e4m3(h*sf_inv), saturating).
 *   x (T, K) e4m3, x_scale (T, K/128) fp32;
 *   w1 (E, N, K) e4m3, w1_scale (E, N/128, K/128) fp32;
 *   w2 (E, K, N/2) e4m3, w2_scale (E, K/128, (N/2)/128) fp32. */
int fused_moe_fp8_blockwise(const void* x, const float* x_scale,
                            const void* w1, const float* w1_scale,
                            const void* w2, const float* w2_scale,
                            const int32_t* sorted_token_ids,
                            const int32_t* expert_ids,
                            const int32_t* num_tokens_post_padded,
                            const float* topk_weights, void* out, int64_t T,
                            int64_t K, int64_t N, int32_t E, int32_t top_k,
                            int32_t block_m, int32_t split, const moe_tune* tune,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * blockwise FP8 path of fused_moe_fp8_blockwise with no workspace argument
 * and no tune.  The workspace is a static array of 64 MiB that the library
 * holds on every GPU it runs on until the process ends (enough for the
 * decode sizes at K = 4096, I = 2048, e.g. T = 256 with top-6 over 256
 * experts and block_m 16, split mode).  A call whose moe_workspace_size(.., NULL)
 * exceeds 64 MiB fails with MOE_ERR_WORKSPACE before anything is launched.
 * Nothing is allocated: the array's address on the current device is looked
 * up once (hipGetSymbolAddress) on that device's first call.  Every call on
 * one GPU shares that GPU's array, so calls that may overlap on one GPU (two
 * streams, two threads) race and must be serialized by the caller; the
 * kernels clear what they count on, so the contents a previous call left do
 * not matter.  Otherwise exactly fused_moe_fp8_blockwise (same arguments,
 * results and errors). */
int fused_moe_fp8_blockwise_noalloc(const void* x, const float* x_scale,
                                    const void* w1, const float* w1_scale,
                                    const void* w2, const float* w2_scale,
                                    const int32_t* sorted_token_ids,
                                    const int32_t* expert_ids,
                                    const int32_t* num_tokens_post_padded,
                                    const float* topk_weights, void* out, int64_t T,
                                    int64_t K, int64_t N, int32_t E, int32_t top_k,
                                    int32_t block_m, int32_t split, void* stream);

/* MXFP8 path ([prime-flash] "Scale layout (mxfp8)": e4m3 values with e8m0
 * scales per 32 along K, activation scales row-major; the intermediate is
 * requantized to mxfp8 on chip before the down GEMM, shared exponent
 * floor(log2 amax) - 8 per 32 columns, elements saturating).  All scales are
 * row-major here (the page's blocked weight-scale tiles are an addressing
 * scheme of its hardware and are not used).
 *   x (T, K) e4m3, x_scale (T, K/32) e8m0;
 *   w1 (E, N, K) e4m3, w1_scale (E, N, K/32) e8m0;
 *   w2 (E, K, N/2) e4m3, w2_scale (E, K, (N/2)/32) e8m0. */
int fused_moe_mxfp8(const void* x, const uint8_t* x_scale, const void* w1,
                    const uint8_t* w1_scale, const void* w2,
                    const uint8_t* w2_scale, const int32_t* sorted_token_ids,
                    const int32_t* expert_ids,
                    const int32_t* num_tokens_post_padded,
                    const float* topk_weights, void* out, int64_t T, int64_t K,
                    int64_t N, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t split, const moe_tune* tune, void* workspace,
                    size_t workspace_bytes, void* stream);

/* MXFP4 weights x MX FP8 activations ([DeepGEMM #411] "Summary": routed
 * weights stay packed MXFP4 in memory, E2M1 elements with one UE8M0 exponent
 * per 32 along K; activations FP8).  The e2m1 elements (OCP MX FP4: 1 sign,
 * 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6) are packed two per byte, element 2j in the low nibble of byte j,
 * along the contraction dimension.  Activations and the on-chip intermediate
 * are MX FP8 exactly as in fused_moe_mxfp8 (workspace as for MOE_MXFP8).
 *   x (T, K) e4m3, x_scale (T, K/32) e8m0;
 *   w1 (E, N, K/2) bytes, w1_scale (E, N, K/32) e8m0;
 *   w2 (E, K, (N/2)/2) bytes, w2_scale (E, K, (N/2)/32) e8m0.
 * block_m 256 is not available for this dtype (MOE_ERR_UNSUPPORTED). */
int fused_moe_mxfp4(const void* x, const uint8_t* x_scale, const void* w1,
                    const uint8_t* w1_scale, const void* w2,
                    const uint8_t* w2_scale, const int32_t* sorted_token_ids,
                    const int32_t* expert_ids,
                    const int32_t* num_tokens_post_padded,
                    const float* topk_weights, void* out, int64_t T, int64_t K,
                    int64_t N, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t split, const moe_tune* tune, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Shared experts.  [DeepGEMM #411] "Summary" runs the routed and the shared
 * experts' two GEMMs in one kernel; [DeepGEMM #88] "Performance" runs the
 * shared expert as a separate GEMM.  A shared expert is an FFN of the same
 * format as the routed ones that every token adds with weight 1; here it is
 * computed by the same kernels, as one more route per token.
 *
 * Planner: moe_align with n_shared shared experts numbered E .. E+n_shared-1:
 * routes t*top_k + j keep topk_ids[t][j] (local only in [0, E)), and route
 * T*top_k + t*n_shared + s goes to expert E + s.  Capacities are
 * moe_align_capacity(T, top_k + n_shared, E + n_shared, block_m).  Errors as
 * moe_align, plus MOE_ERR_SHAPE (n_shared < 0), MOE_ERR_UNSUPPORTED
 * (E + n_shared > 1024).
 */
int moe_align_shared(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                     int32_t n_shared, int32_t block_m, int32_t* sorted_token_ids,
                     int32_t* expert_ids, int32_t* num_tokens_post_padded, void* stream);

/*
 * Forward with shared experts, any dtype (dtype: moe_dtype; operands and
 * scales as in that dtype's fused_moe_* entry point, bf16 passes NULL
 * scales).  w1, w2 and their scales hold E + n_shared experts: the E routed
 * ones, then the n_shared shared ones (concatenated once at load time).
 * sorted_token_ids / expert_ids / num_tokens_post_padded come from
 * moe_align_shared with the same n_shared.  E is the routed expert count and
 * top_k the routed top-k; the workspace is moe_workspace_size(dtype, T, K, N,
 * E + n_shared, top_k + n_shared, block_m, split).
 *   out[t] = bf16(sum_j topk_weights[t][j] * FFN_{topk_ids[t][j]}(x[t])
 *                 + sum_s FFN_{E+s}(x[t]))
 * one rounding at the end.  n_shared = 0 is exactly the fused_moe_* call.
 * Errors as the fused_moe_* entry points, plus MOE_ERR_SHAPE (n_shared < 0).
 */
int fused_moe_shared(int32_t dtype, const void* x, const void* x_scale, const void* w1,
                     const void* w1_scale, const void* w2, const void* w2_scale,
                     int32_t n_shared, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                     const float* topk_weights, void* out, int64_t T, int64_t K, int64_t N,
                     int32_t E, int32_t top_k, int32_t block_m, int32_t split,
                     const moe_tune* tune, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split mode's second half alone, for testing the down GEMM and the
 * combine apart from the gate/up GEMM and the requantization ([prime-flash]
 * "Tests and benchmarks": the comparison isolates the kernel from the
 * quantizer; [hpc-ops RFC] "Background" stages 4-5).  The caller places the
 * requantized intermediate in the workspace, rows in sorted_token_ids order
 * at moe_workspace_layout's offsets (values, then scales), and the call runs
 * the down GEMM of every planner block and the top-k weighted combine into
 * `out`, exactly as fused_moe_* in split mode (split = 1, no tune) would
 * after its gate/up GEMM.  Arguments as fused_moe_* (w2 and its scales only;
 * bf16 passes NULL scales); the workspace is moe_workspace_size(dtype, T, K,
 * N, E, top_k, block_m, 1, NULL) bytes.  Rows of -1 positions may hold any
 * bytes.  Errors as fused_moe_*.
 */
int fused_moe_down_combine(int32_t dtype, const void* w2, const void* w2_scale,
                           const int32_t* sorted_token_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, const float* topk_weights,
                           void* out, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                           int32_t block_m, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Diagnostic, not a step of the forward: one 128-wide K step of the matrix
 * instruction each dtype's kernels use, D = C + A . B^T, per 16 x 16 tile,
 * through the kernels' own operand layout and instruction wrappers.  The
 * parity tests accept outputs within an error model of these instructions
 * (their sums are not correctly rounded: an e4m3 instruction keeps a limited
 * number of bits of the products it aligns); a test measures the
 * instructions against that model with this call.
 *   a        (n_tiles, 16, 128) A rows: e4m3 bytes, or bf16 (256 bytes a row)
 *   b        (n_tiles, 16, 128) B rows as a; MOE_MXFP4: (n_tiles, 16, 64)
 *            packed e2m1 (element 2j in the low nibble of byte j)
 *   a_scale, b_scale  MOE_MXFP8 / MOE_MXFP4: (n_tiles, 16, 4) e8m0 bytes, one
 *            per 32-wide K block of each row; unused (may be NULL) otherwise
 *   c        (n_tiles, 16, 16) fp32 accumulator input, or NULL for zeros
 *   d [out]  (n_tiles, 16, 16) fp32: d[t][i][j] = c[t][i][j] + sum_k
 *            A[t][i][k] B[t][j][k] (times the rows' block scales for MX)
 * MOE_FP8_BLOCKWISE uses the unscaled e4m3 instruction (block scales are
 * applied outside it by the kernels).  Device pointers, 16-byte aligned;
 * asynchronous on `stream`.  Returns MOE_ERR_UNSUPPORTED (dtype),
 * MOE_ERR_SHAPE (n_tiles outside [0, 2^24]), MOE_ERR_NULL, MOE_ERR_ALIGN or
 * MOE_ERR_HIP; no message is recorded for this call.
 */
int moe_mfma_probe(int32_t dtype, const void* a, const void* b, const uint8_t* a_scale,
                   const uint8_t* b_scale, const float* c, float* d, int64_t n_tiles,
                   void* stream);

/*
 * Profiling hook (changes no result): the next fused_moe_* calls made by the
 * calling thread record the caller's hipEvent_t handles `before` and `after`
 * (passed as void*) on their stream immediately before and after one kernel:
 *   which = 1: the main weight-streaming kernel (the fused kernel in fused
 *              mode, the gate/up kernel in split mode);
 *   which = 2: the down kernel (split mode only; fused mode records nothing).
 * which = 0 or NULL events switch the hook off.  The handles stay owned by
 * the caller and must outlive the calls that record them.
 * Errors: MOE_ERR_UNSUPPORTED (which outside 0..2).
 */
int moe_set_timing_events(void* before, void* after, int32_t which);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
