// kernels.h -- host-side launch interface between the C ABI (abi.cpp) and the
// HIP kernels (meta.hip, delta.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace tl {

constexpr int kKP = 512;          // k per shrink step of the fused kernel
constexpr int kEB = 512;          // output columns per expand batch of the fused kernel (128 per wave)
constexpr int kFlagWords = 64;    // 64-bit words per tile in the fused workspace: piece flags, then a count
constexpr int kMetaChunk = 1024;  // rows per workgroup (chunk) of the metadata build
constexpr int kSlotThreads = 256;       // threads (rows) of an in-launch metadata build
constexpr int kSmallBallotSlots = 64;   // slots a one-workgroup build ranks with one ballot per slot bit
constexpr int kMaxSlices = 8;
constexpr int kMaxRank = 128;
constexpr int kMetaMaxSlotsMulti = 8192;  // slot limit when n spans several 1024-row chunks
constexpr int kTileRows = 16;             // rows per tile record (the MFMA M dimension)
constexpr int kTileWords = 32;            // int32 words per tile record

// Tiles of a segment of t rows in a batch of n rows: 16-row tiles, the last
// one ragged, except that in batches of at most 1024 rows (decode-sized) a
// segment of 9..15 rows is cut into two tiles of ceil(t/2) and floor(t/2)
// rows.  Such a segment takes the vector-ALU path at the default MFMA
// threshold, whose work grows with a tile's rows, and in a small batch it is
// on the critical path; two tiles run in parallel.  (In large batches the
// extra tile would re-read the adapter for no gain.)  Tile pairing (two
// 16-row tiles in one unit) applies to segments of at least 16 rows only.
constexpr int kSplitMaxRows = 1024;
__host__ __device__ inline bool seg_is_split(int t, int n) { return n <= kSplitMaxRows && t > 8 && t < kTileRows; }
__host__ __device__ inline int seg_tiles(int t, int n) {
    return seg_is_split(t, n) ? 2 : (t + kTileRows - 1) / kTileRows;
}
__host__ __device__ inline int seg_tile_rows(int t, int n) { return seg_is_split(t, n) ? (t + 1) / 2 : kTileRows; }
// Upper bound of the tile count of n rows in at most S segments: a segment
// has at most t/16 + 1 tiles, plus one when it is split (a split segment has
// at least 9 rows), and at most t/8 + 1 tiles in any case; never more than n.
__host__ __device__ inline int tile_bound_of(int n, int S) {
    if (n <= 0) return 0;
    const long long segs = n < S ? n : S;
    long long m = (n + kTileRows - 1) / kTileRows + segs;
    if (n <= kSplitMaxRows) {
        const long long split = segs < n / 9 ? segs : n / 9;
        const long long b = (n + 7) / 8 + segs;
        m = m + split < b ? m + split : b;
    }
    return (int)(m < n ? m : n);
}

struct MetaOut {
    int32_t *sorted_rows;
    int32_t *seg_offsets;
    int32_t *seg_slot;
    int32_t *counts;
    int32_t *tiles;
    int tile_bound;
};

// Workspace of a multi-chunk meta build: ctl[0] the single assembler's
// ticket (unused when the build assembles in a second launch), ctl[1] invalid
// rows (both zero between calls), then rows / keys / offset+length per chunk
// row, then (hist, when the [chunk][slot] table fits, else null) the rows of
// each slot in each chunk, [chunk][S].
struct MetaWs {
    int32_t *ctl;
    int32_t *rows;
    int32_t *keys;
    int32_t *offlen;
    int32_t *hist;
};
constexpr int kMetaTable = 16384;    // LDS ints for an assembling workgroup's [chunk][slot] table and slot arrays
constexpr int kSplitMaxChunks = 64;  // a split build's workgroups each read every chunk's slot counts
__host__ __device__ inline bool meta_table_fits(int n_chunks, int S) {
    return (long long)(4 + n_chunks) * S <= kMetaTable;
}

int meta_chunks(int n);
size_t meta_dyn_lds(int n, int S);
hipError_t launch_meta_dense(const int32_t *slot, int n, int S, MetaOut out, MetaWs ws, hipStream_t st);
hipError_t launch_meta_moe(const int32_t *topk, const int32_t *lora, int top_k, int E, int L, int n_pairs,
                           MetaOut out, MetaWs ws, hipStream_t st);
hipError_t launch_meta_blocks(const uint32_t *offsets, const int32_t *block_slot, int n_blocks, int n, int S,
                              MetaOut out, MetaWs ws, hipStream_t st);

// Shapes of a dense call, validated by the caller.
struct DenseShape {
    const uint16_t *x;
    int64_t ldx;
    int n, k_in;
    const uint16_t *a_pool;
    const uint16_t *b_pool;
    const float *scale;
    int num_slots, num_slices, R;
    int slice_off[kMaxSlices + 1];  // prefix sums of the slice widths
    uint16_t *y;
    int64_t ldy;
    int offset_start;
};

// Fused-call workspace layout (all sizes derived from the shape).
struct FusedPlan {
    int tile_bound;  // tile records the meta build wrote
    size_t flag_bytes, part_bytes, total_bytes;
};
FusedPlan fused_plan(int n, int num_slots, int num_slices, int R, int k_in, int n_out);

hipError_t launch_shrink(const DenseShape &d, const int32_t *tiles, int tile_bound, float *xa, int mfma_min,
                         hipStream_t st);
hipError_t launch_expand(const DenseShape &d, const float *xa, const int32_t *tiles, int tile_bound,
                         int add_inputs, int mfma_min, hipStream_t st);
// slot != null (and meta_out): the launch also builds the batch's metadata
// from slot and writes it to meta_out; tiles and counts are then unused.
// Only where fused_builds_meta holds (hipErrorInvalidValue otherwise).
hipError_t launch_fused(const DenseShape &d, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                        void *ws, int mfma_min, hipStream_t st, const int32_t *slot = nullptr,
                        const MetaOut *meta_out = nullptr);
bool fused_builds_meta(const DenseShape &d, const FusedPlan &plan);
// Launch shape of the fused kernel (plan.cpp): narrow_call, the call runs in
// mode 0; chunks_of, expand units per tile at EC columns each;
// expand_width, the columns per expand unit.
bool narrow_call(int k_in, int EC);
int chunks_of(const int *off, int n_windows, int EC);
int expand_width(const int *off, int n_windows, int tile_bound);

// Address of the library's fixed device buffer (LORA_NOALLOC_SCRATCH_BYTES)
// on `device`, which must be the current device; resolved on the first call
// per device, then cached.
hipError_t noalloc_scratch(int device, void **ptr);

// MoE pairs whose (adapter, expert) is not valid get a zero output row.
struct ZeroFill {
    const int32_t *topk;
    const int32_t *lora;
    int top_k, E, L, n_pairs;
};

struct MoeShape {
    const uint16_t *x;
    int64_t ldx;
    int T, H;
    const int64_t *w_ptr_a;
    int64_t lora_stride_a;
    const int64_t *w_ptr_b;
    int64_t lora_stride_b;
    int shared_a;
    const int32_t *topk_ids;
    int top_k;
    const int32_t *lora_ids;
    int E, L, R, inter;
    float scale;
    uint16_t *out;
};
hipError_t launch_moe_delta(const MoeShape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                            int mfma_min, hipStream_t st);

// Routed-MoE down projection: x2 [n_pairs][I] (ldx), y [n_pairs][H] (ldy) added to.
struct MoeW2Shape {
    const uint16_t *x2;
    int64_t ldx;
    int T, I;
    const int64_t *w_ptr_a;
    int64_t lora_stride_a;
    const int64_t *w_ptr_b;
    int64_t lora_stride_b;
    int top_k;
    const float *topk_weights;  // or null
    int E, L, R, H;
    float scale;
    uint16_t *y;
    int64_t ldy;
};
hipError_t launch_moe_w2_delta(const MoeW2Shape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                               int mfma_min, hipStream_t st);

}  // namespace tl
