/*
 * lora.h -- C ABI of the routed multi-tenant LoRA delta for MI355X (gfx950).
 *
 * The operation (metrale docs, module lora_delta, function apply_lora_bgmv;
 * vLLM punica_base.py, PunicaWrapperBase.add_shrink / add_expand /
 * add_lora_linear): every row i of a batch that names an adapter slot
 * s = slot[i] >= 0 gets
 *
 *     y[i, :] += scale[s] * (x[i, :] @ A_s^T) @ B_s^T
 *
 * computed as a shrink (xa = scale * x @ A^T, fp32) then an expand
 * (y += xa @ B^T).  A row with a negative slot gets no delta.  The routed-MoE
 * variant (FlashInfer docs, flashinfer.fused_moe.bgmv_moe_gemm1_lora_delta)
 * gives one gate/up delta per (token, top-k slot), and the down-projection
 * variant (vLLM punica_base.py, add_lora_w2) adds one router-weighted delta
 * to each (token, top-k slot) output row of the expert down projection.
 *
 * Conventions for every function below:
 *  - bf16 values travel as uint16_t bit patterns; float is IEEE binary32.
 *  - Every array pointer is a DEVICE pointer unless marked [host].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it: no call allocates, frees, synchronizes, prints or
 *    aborts (metrale docs, module lora_delta invariants: launchers only
 *    launch).  Pointers must stay valid until the stream reaches the call.
 *  - The caller owns every buffer, including metadata and workspaces.  The
 *    library keeps no pointer after a call returns and holds no state
 *    besides the MFMA row threshold, which is per calling thread
 *    (lora_set_mfma_min_rows).
 *  - Every check that can run on the host runs before any launch and
 *    returns an error code; nothing is enqueued then.
 *  - Workspaces must be zero-filled before their first use.  The meta
 *    workspace's counters return to zero after every call; where a fused
 *    or MoE call builds its metadata, they sit at byte 64 of that
 *    workspace, which no call of any shape uses for anything else.  The
 *    fused and MoE workspaces hold a control line (below) whose tag of the last
 *    completed call tags the partial results of the next one; they stay
 *    valid for calls of any shape that fits them, for 2^31 - 2 calls
 *    (then the tags start over: zero-fill the workspace again before that).
 *    Calls that share a workspace must be ordered (same stream).
 *  - Inside a fused call, units that wait for other units' results do so
 *    with bounded polls.  Such a wait can only run out when calls sharing a
 *    workspace overlap; the kernel then still finishes (the rows concerned
 *    get undefined values) and sets the control line's error word to 1,
 *    which the library never clears.
 *
 * Control line (int32 words, at a fixed byte offset of the workspace:
 * LORA_FUSED_CTL_OFFSET for lora_delta_fused, LORA_MOE_CTL_OFFSET for
 * moe_lora_gemm1_delta and moe_lora_w2_delta, whatever the call's shape):
 *    [0] error word: 0, or 1 once a bounded wait has given up
 *    [1] tag of the last completed call (0 before the first; tags run
 *        0x80000001, 0x80000002, ..., so the low 31 bits count the calls)
 *    [2] tiles finished by a running call: 0 between calls
 * Read it after the stream has reached the call.
 *
 * Layouts (metrale docs, LoraPair and LoraRoute; the slices follow vLLM's
 * add_shrink / add_expand, one A and one block of B rows per output slice):
 *    x       [n][ldx]                       bf16, row-major, k_in used columns
 *    a_pool  [num_slots][num_slices][max_rank][k_in]   bf16
 *    b_pool  [num_slots][N][max_rank]       bf16, N = sum(slice_sizes);
 *                                            slice l owns rows off_l .. off_l+w_l
 *    scale   [num_slots]                    float (applied to the fp32 shrink
 *                                            result, never folded into B)
 *    xa      [num_slices][n][max_rank]      float
 *    y       [n][ldy]                       bf16, slice l's window is columns
 *                                            offset_start+off_l .. +w_l
 * An adapter of true rank r < max_rank is stored zero-padded: rows r.. of A
 * and columns r.. of B are zero, and both stages contract at max_rank.
 *
 * Shape limits: k_in (H) and every slice width a multiple of 8; max_rank
 * (rank) a multiple of 8, at most 128; 1 <= num_slices <= 8; ldx, ldy,
 * offset_start multiples of 8; x, y, xa, pools 16-byte aligned;
 * num_slots <= 1<<20; n <= 1<<22.
 */
#ifndef TENANT_LORA_H
#define TENANT_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LORA_OK = 0,
    LORA_EINVAL = -1,       /* bad pointer, size, alignment or leading dimension */
    LORA_EUNSUPPORTED = -2, /* a shape outside the limits above */
    LORA_EWORKSPACE = -3,   /* workspace or metadata buffer too small */
    LORA_ELAUNCH = -4,      /* the HIP runtime refused a launch */
    LORA_ESCRATCH = -5      /* lora_delta_fused_noalloc: the call does not fit the fixed buffer */
};

/* Byte offsets of the control line in the fused and MoE workspaces. */
#define LORA_FUSED_CTL_OFFSET 0
#define LORA_MOE_CTL_OFFSET 128

/* Rows per tile of the per-segment work lists built by lora_meta_build. */
#define LORA_TILE_ROWS 16
/* int32 words per tile record. */
#define LORA_TILE_WORDS 32

/*
 * Per-step routing metadata, built once per batch by lora_meta_build and read
 * by every shrink / expand / fused call of that batch (vLLM punica_base.py,
 * PunicaWrapperBase: metadata updated once per step and reused by all LoRA
 * layers; prefill_metadata groups rows of one adapter into segments).
 * Active rows (0 <= slot < num_slots) are sorted by (slot, row); a segment is
 * a run of one slot.  Sizes in elements:
 *   sorted_rows  [n]                 active rows in (slot, row) order
 *   seg_offsets  [min(n,S) + 1]      segment starts in sorted_rows, then n_active
 *   seg_slot     [min(n,S)]          each segment's slot, strictly ascending
 *   counts       [8]                 {n_active, n_segments, n_invalid,
 *                                     n_segments_with_at_least_16_rows,
 *                                     n_tiles, 0, 0, 0}
 *   tiles        [lora_meta_max_tiles(n,S) * LORA_TILE_WORDS]
 *       Each segment is cut into tiles of 16 consecutive sorted rows, the
 *       last one ragged; when n <= 1024, a segment of 9..15 rows is cut into
 *       two tiles of ceil(rows/2) and floor(rows/2) rows (run in parallel).
 *       Record t (32 int32): [0] slot, [1] first sorted position, [2] rows in
 *       the tile (0 marks an unused record), [3] rows in the whole segment,
 *       [4] segment index, [5] the tile's index within its segment,
 *       [8..23] the tile's original row ids.
 * Entries past n_active / n_segments are left unwritten.
 */
typedef struct {
    int32_t *sorted_rows;
    int32_t *seg_offsets;
    int32_t *seg_slot;
    int32_t *counts;
    int32_t *tiles;
} lora_meta_t;

/* Number of tile records the tiles array must hold for n rows and S slots:
 * with g = min(n, S), min(n, ceil(n/16) + g) when n > 1024, else
 * min(n, ceil(n/16) + g + min(g, floor(n/9)), ceil(n/8) + g). */
int32_t lora_meta_max_tiles(int32_t n, int32_t num_slots);

/* Workspace bytes lora_meta_build needs for n rows and S slots. */
size_t lora_meta_workspace_bytes(int32_t n, int32_t num_slots);

/*
 * Build the metadata for slot[n] (int32; negative = no delta; >= num_slots =
 * invalid, excluded and counted in counts[2]).  All meta arrays are written
 * on the device; the result is unique (bit-exact).  n == 0 writes
 * counts = 0 and seg_offsets[0] = 0.  num_slots in [1, 1<<20]; when n > 1024
 * num_slots must be at most 8192 (LORA_EUNSUPPORTED otherwise).
 */
int lora_meta_build(const int32_t *slot, int32_t n, int32_t num_slots, lora_meta_t meta,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * Metadata for the expert-sorted fold (metrale source lora/expert_apply.rs:
 * expert_delta_workitems, apply_expert_lora_sorted, apply_router_lora),
 * built on the device from the expert_offsets prefix sum with no host copy.
 * expert_offsets is [num_experts + 1] uint32 (device): expert e owns sorted
 * rows expert_offsets[e] .. expert_offsets[e+1]; expert_slot is
 * [num_experts] int32 (device), the pool slot of expert e's pair, or -1 when
 * e has none.  The result is exactly lora_meta_build over n rows with
 * slot[r] = expert_slot[e] for the e whose block holds r and -1 for rows in
 * no block (and for rows >= expert_offsets[num_experts]), so
 * lora_delta_fused with it folds each adapted expert's pair over its block
 * of rows; a slot >= num_slots is counted as invalid.  The router fold is
 * the case of one block {0, n} and one slot.  Offsets that are not
 * non-decreasing are outside the contract: each row then still gets at most
 * one expert (the one a binary search for the first offset above the row
 * finds).  Workspace as for lora_meta_build.  Errors: LORA_EINVAL for bad
 * sizes or null pointers, LORA_EUNSUPPORTED as for lora_meta_build,
 * LORA_EWORKSPACE for a missing or small workspace.
 */
int lora_meta_from_offsets(const uint32_t *expert_offsets, int32_t num_experts,
                           const int32_t *expert_slot, int32_t n, int32_t num_slots,
                           lora_meta_t meta, void *ws, size_t ws_bytes, void *stream);

/*
 * Shrink (vLLM punica_base.py, add_shrink semantics; metrale lora_delta,
 * apply_lora_bgmv): for every active row i with slot s, slice l, rank r:
 *     xa[l][i][r] = scale[s] * sum_k x[i][k] * a_pool[s][l][r][k]
 * accumulated in fp32 from exact bf16 products.  Rows without an active slot
 * are not written.  xa is [num_slices][n][max_rank] float.
 */
int lora_shrink(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in,
                const uint16_t *a_pool, const float *scale, int32_t num_slots,
                int32_t num_slices, int32_t max_rank, lora_meta_t meta, float *xa,
                void *stream);

/*
 * Expand (vLLM punica_base.py, add_expand semantics): for every active row i
 * with slot s, slice l of width w_l at offset off_l, column c < w_l:
 *     y[i][offset_start + off_l + c] = (add_inputs ? y[i][...] : 0)
 *                                      + sum_r xa[l][i][r] * b_pool[s][off_l + c][r]
 * accumulated in fp32, rounded once to bf16 (nearest-even).  Every other
 * element of y is left untouched.  slice_sizes is a [host] array of
 * num_slices widths.
 */
int lora_expand(const float *xa, const uint16_t *b_pool, int32_t num_slots,
                int32_t num_slices, const int32_t *slice_sizes, int32_t max_rank, int32_t n,
                lora_meta_t meta, uint16_t *y, int64_t ldy, int32_t offset_start,
                int32_t add_inputs, void *stream);

/* Workspace bytes lora_delta_fused needs. */
size_t lora_fused_workspace_bytes(int32_t n, int32_t num_slots, int32_t num_slices,
                                  int32_t max_rank, int32_t k_in);

/*
 * Fused delta (vLLM punica_base.py, add_lora_linear semantics; metrale
 * lora_delta, apply_lora_bgmv): the shrink then the expand with
 * add_inputs = 1, in one launch; xa stays in the workspace (fp32).
 *     y[i][window] += (scale[s] * x[i] @ A_s^T) @ B_s^T
 * Rows without an active slot and columns outside the slice windows are
 * left untouched.  Segments with at least 16 rows run on bf16 MFMA with the
 * fp32 xa split into two bf16 terms; shorter ones on the vector ALU.
 */
int lora_delta_fused(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in,
                     const uint16_t *a_pool, const uint16_t *b_pool, const float *scale,
                     int32_t num_slots, int32_t num_slices, const int32_t *slice_sizes,
                     int32_t max_rank, lora_meta_t meta, uint16_t *y, int64_t ldy,
                     int32_t offset_start, void *ws, size_t ws_bytes, void *stream);

/*
 * The routing metadata and the fused delta in one call (vLLM punica_base.py:
 * the wrapper's metadata update for the step, then add_lora_linear; metrale
 * lora_delta docs, apply_lora_bgmv): meta is written exactly as
 * lora_meta_build(slot, n, num_slots, meta, ...) writes it, so that later
 * calls of the same step (the other LoRA layers) can pass it to
 * lora_delta_fused, and y is updated exactly as lora_delta_fused(..., meta,
 * ...) would update it.  Batches of at most 256 rows over at most 64 slots
 * whose call runs one 512-column batch per expand unit (decode-sized; the
 * Llama-3-8B QKV shape at rank 16 is one) do both in one launch: each
 * workgroup of the delta derives its own tile's record from slot, and one
 * more workgroup writes meta.  Other batches run the metadata kernel, then
 * the fused kernel.  ws must hold lora_fused_workspace_bytes(n, num_slots,
 * num_slices, max_rank, k_in) + lora_meta_workspace_bytes(n, num_slots)
 * bytes (the metadata build's part after the fused part); it carries the
 * fused control line at its start as for lora_delta_fused, and the same
 * workspace may be passed to either call.  Errors as for lora_meta_build and
 * lora_delta_fused (slot may be null only when n == 0).
 */
int lora_delta_fused_build(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in,
                           const uint16_t *a_pool, const uint16_t *b_pool, const float *scale,
                           int32_t num_slots, int32_t num_slices, const int32_t *slice_sizes,
                           int32_t max_rank, const int32_t *slot, lora_meta_t meta, uint16_t *y,
                           int64_t ldy, int32_t offset_start, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the fixed device buffer behind lora_delta_fused_noalloc. */
#define LORA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * lora_delta_fused without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, result and errors as
 * lora_delta_fused, whose kernels it runs; the workspace is instead a fixed
 * buffer of LORA_NOALLOC_SCRATCH_BYTES in device memory that the library
 * holds on each GPU it runs on until the process ends (zero when loaded).
 * Nothing is allocated or freed.  Calls whose workspace (as
 * lora_fused_workspace_bytes gives it) exceeds the buffer return
 * LORA_ESCRATCH before anything is enqueued; decode-sized batches fit (256
 * rows, 32 slots, three slices, rank 16, k_in 4096 need about 3 MB).  The
 * buffer used is the current device's, so `stream` must belong to the
 * current device (LORA_EINVAL otherwise); the first call on a device
 * resolves the buffer's address, so make it outside graph capture.  Every
 * call on one GPU shares that GPU's buffer, and each call finds it as the
 * last one left it (the control line's call tags keep calls apart, so
 * nothing is cleared between calls): calls on one GPU must be ordered (one
 * stream, or streams joined by events); calls that overlap race and give
 * undefined rows.
 */
int lora_delta_fused_noalloc(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in,
                             const uint16_t *a_pool, const uint16_t *b_pool, const float *scale,
                             int32_t num_slots, int32_t num_slices, const int32_t *slice_sizes,
                             int32_t max_rank, lora_meta_t meta, uint16_t *y, int64_t ldy,
                             int32_t offset_start, void *stream);

/* Workspace bytes moe_lora_gemm1_delta needs. */
size_t moe_lora_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts,
                                int32_t num_loras, int32_t rank, int32_t H);

/*
 * Routed-MoE gemm1 (gate_up) LoRA delta (FlashInfer docs,
 * flashinfer.fused_moe.bgmv_moe_gemm1_lora_delta).  For pair (t, j) with
 * expert e = topk_ids[t][j] and adapter l = lora_ids[t]:
 *   regular (shared_a == 0): w_ptr_a / w_ptr_b are [2][num_experts] int64
 *     tables of device addresses (gate row 0, up row 1); adapter l's matrices
 *     for expert e start lora_stride elements * l past the table entry;
 *     A is [rank][H], B is [inter][rank] (bf16), and
 *       out[t][j][:] = scale * concat(B_gate @ (A_gate @ x[t]), B_up @ (A_up @ x[t]))
 *   shared (shared_a != 0): the tables are [num_experts]; A is [rank][H],
 *     B is [2*inter][rank] (gate rows then up rows), and
 *       out[t][j][:] = scale * B @ (A @ x[t])
 * l < 0 gives a zero row.  l >= num_loras or e outside [0, num_experts) gives
 * a zero row and is counted: after the call the first 16 bytes of ws hold
 * counts {n_active_pairs, n_segments, n_invalid_pairs, n_long_segments}
 * (the whole pair metadata is in ws too: moe_lora_meta_layout).  The
 * control line is at byte LORA_MOE_CTL_OFFSET.
 * The delta is unweighted and kept per pair (it is added before the gated
 * activation).  out is [T][top_k][2*inter] bf16, every element written.
 * With T = 0 only the counts are written, and x, topk_ids, lora_ids and out
 * may be null.
 */
int moe_lora_gemm1_delta(const uint16_t *x, int64_t ldx, int32_t T, int32_t H,
                         const int64_t *w_ptr_a, int64_t lora_stride_a,
                         const int64_t *w_ptr_b, int64_t lora_stride_b, int32_t shared_a,
                         const int32_t *topk_ids, int32_t top_k, const int32_t *lora_ids,
                         int32_t num_experts, int32_t num_loras, int32_t rank, int32_t inter,
                         float scale, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_lora_w2_delta needs (I: the down projection's input
 * width, the intermediate size). */
size_t moe_lora_w2_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts,
                                   int32_t num_loras, int32_t rank, int32_t I);

/*
 * Routed-MoE down-projection (w2) LoRA delta, added in place to the per-pair
 * output of the expert down projection before the top-k sum (vLLM
 * punica_base.py, PunicaWrapperBase.add_lora_w2; routed as the gemm1 delta).
 * For pair p = t*top_k + j with expert e = topk_ids[t][j] and adapter
 * l = lora_ids[t]: w_ptr_a / w_ptr_b are [num_experts] int64 tables of device
 * addresses (16-byte aligned); adapter l's matrices for expert e start
 * lora_stride elements * l past the entry, A is [rank][I] and B is [H][rank]
 * (bf16); w = topk_weights[p] (fp32 [T][top_k]), or 1 when topk_weights is
 * null (the unweighted form), and
 *   y[p][:] = bf16(y[p][:] + (w * scale) * B @ (A @ x2[p]))
 * with A @ x2 and the product by B accumulated in fp32 and rounded once.
 * x2 is [T*top_k][I] bf16 with row stride ldx, y is [T*top_k][H] bf16 with
 * row stride ldy.  Pairs with l < 0, l >= num_loras or e outside
 * [0, num_experts) keep their y row; the last two are counted as invalid
 * (the counts at the start of ws as for moe_lora_gemm1_delta).  With T = 0
 * only the counts are written, and x2, topk_ids, lora_ids and y may be
 * null.  reuse_routing != 0 skips the pair metadata build and uses the one
 * already in ws (vLLM's add_lora_w2 reuses the routing add_lora_w13 built):
 * the caller guarantees that the previous MoE call on this workspace (gemm1
 * or w2) had the same T, top_k, num_experts, num_loras, topk_ids and
 * lora_ids; a workspace of the larger of moe_lora_workspace_bytes and
 * moe_lora_w2_workspace_bytes serves both calls.  Errors:
 * LORA_EINVAL for bad sizes, strides or pointers, LORA_EUNSUPPORTED for a
 * rank outside {8, 16, ..., 128}, LORA_EWORKSPACE for a missing or small
 * workspace; nothing is launched on error.
 */
int moe_lora_w2_delta(const uint16_t *x2, int64_t ldx, int32_t T, int32_t I,
                      const int64_t *w_ptr_a, int64_t lora_stride_a,
                      const int64_t *w_ptr_b, int64_t lora_stride_b,
                      const int32_t *topk_ids, int32_t top_k, const int32_t *lora_ids,
                      const float *topk_weights, int32_t num_experts, int32_t num_loras,
                      int32_t rank, int32_t H, float scale, uint16_t *y, int64_t ldy,
                      int32_t reuse_routing, void *ws, size_t ws_bytes, void *stream);

/*
 * Where a MoE call (gemm1 or w2) keeps the pair metadata it builds in ws,
 * as byte offsets into ws (offsets [host], 5 entries): counts (8 int32),
 * sorted_rows, seg_offsets, seg_slot, tiles -- the arrays of lora_meta_t for
 * n = T * top_k rows (pairs p = t * top_k + j) and S = num_loras *
 * num_experts slots, with key l * num_experts + e (vLLM punica_base.py,
 * moe_lora_align_block_size: pairs grouped by (adapter, expert); FlashInfer
 * bgmv_moe_gemm1_lora_delta: topk_ids, lora_ids).  The offsets depend on
 * (T, top_k, num_experts, num_loras) only.  LORA_EINVAL for bad sizes.
 */
int moe_lora_meta_layout(int32_t T, int32_t top_k, int32_t num_experts, int32_t num_loras,
                         size_t *offsets);

/* Segments with at least this many rows take the MFMA path, shorter ones the
 * vector-ALU path.  The default is 16 (the environment variable
 * LORA_MFMA_MIN_ROWS, read once, replaces it).  The setter overrides it for
 * the calling thread only (other threads keep theirs), for calls that
 * thread enqueues after it returns; rows <= 0 drops the override.  Both
 * paths compute the same result to within the tolerance of the fp32
 * accumulation. */
int32_t lora_mfma_min_rows(void);
void lora_set_mfma_min_rows(int32_t rows);

/* A static, human-readable name for a status code. */
const char *lora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TENANT_LORA_H */
