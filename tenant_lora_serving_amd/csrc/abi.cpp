// abi.cpp -- the library's C entry points (declared in include/lora.h):
// host-side validation, workspace carving and kernel launches.  Nothing here
// allocates, frees or synchronizes; every check runs before any launch.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "../../include/lora.h"
#include "kernels.h"

namespace {

using tl::kMaxRank;
using tl::kMaxSlices;

constexpr int kMaxRows = 1 << 22;
constexpr int kMaxSlots = 1 << 20;

// The metadata build's two counters (single assembler's ticket, invalid rows)
// when the build runs inside a fused or MoE call: bytes 64..71 of the fused
// workspace's 256-byte control area (control line at bytes 0..63, flags from
// byte 256) and of the MoE header (counts at bytes 0..31, control line at
// LORA_MOE_CTL_OFFSET).  Both headers stay in place whatever the shape.
constexpr size_t kFusedMetaCtl = 64;
constexpr size_t kMoeMetaCtl = 64;
static_assert(LORA_FUSED_CTL_OFFSET + 64 <= kFusedMetaCtl && kFusedMetaCtl + 8 <= 256,
              "the build's counters sit clear of the fused control line and flags");
static_assert(kMoeMetaCtl >= 8 * sizeof(int32_t) && kMoeMetaCtl + 8 <= LORA_MOE_CTL_OFFSET,
              "the build's counters sit clear of the MoE counts and control line");

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The MFMA row threshold: a process-wide default (16, or LORA_MFMA_MIN_ROWS
// read once), and a per-thread override that only the calling thread sees,
// so one caller's setting never changes another thread's arithmetic path.
int default_mfma_min() {
    static const int d = [] {
        if (const char *e = std::getenv("LORA_MFMA_MIN_ROWS")) {
            const int x = std::atoi(e);
            if (x > 0) return x;
        }
        return 16;
    }();
    return d;
}
thread_local int t_mfma_min = 0;  // 0: the default

int mfma_min_rows() { return t_mfma_min > 0 ? t_mfma_min : default_mfma_min(); }

int tile_bound(int n, int S) { return tl::tile_bound_of(n, S); }

// Multi-chunk metadata workspace: 64 bytes of counters, rows / keys /
// offset+length per chunk row, then [chunk][slot] counts when that table
// fits an assembling workgroup's LDS (the build then assembles in a second
// launch that reads them).
bool meta_hist(int n, int S) { return tl::meta_table_fits(tl::meta_chunks(n), S); }

size_t meta_ws_bytes(int n, int S) {
    const int chunks = tl::meta_chunks(n);
    if (chunks <= 1) return 0;
    return 64 + (size_t)3 * chunks * 1024 * sizeof(int32_t) +
           (meta_hist(n, S) ? (size_t)chunks * S * sizeof(int32_t) : 0);
}

// ctl: where the two counters live when the metadata workspace is carved
// from a larger one whose layout changes with the call's shape (the fused
// and MoE workspaces).  There they sit in that workspace's fixed header, so
// no region of a call of another shape ever covers them and they are still
// zero when the next build starts.  Null: the first 64 bytes of `ws`.
tl::MetaWs carve_meta_ws(void *ws, int n, int S, int32_t *ctl = nullptr) {
    tl::MetaWs w{};
    if (tl::meta_chunks(n) <= 1) return w;
    char *b = static_cast<char *>(ws);
    const size_t per = (size_t)tl::meta_chunks(n) * 1024;
    w.ctl = ctl ? ctl : reinterpret_cast<int32_t *>(b);
    w.rows = reinterpret_cast<int32_t *>(b + 64);
    w.keys = w.rows + per;
    w.offlen = w.keys + per;
    w.hist = meta_hist(n, S) ? w.offlen + per : nullptr;
    return w;
}

bool meta_ok(const lora_meta_t &m) {
    return m.sorted_rows && m.seg_offsets && m.seg_slot && m.counts && m.tiles;
}

int check_meta_shape(int n, int S) {
    if (n < 0 || n > kMaxRows || S < 1 || S > kMaxSlots) return LORA_EINVAL;
    if (tl::meta_chunks(n) > 1 && S > tl::kMetaMaxSlotsMulti) return LORA_EUNSUPPORTED;
    return LORA_OK;
}

int check_rank(int R) { return (R >= 8 && R <= kMaxRank && R % 8 == 0) ? LORA_OK : LORA_EUNSUPPORTED; }

// Validates the fields shared by shrink / expand / fused and fills `d`.
int dense_shape(tl::DenseShape &d, int32_t n, int32_t k_in, int32_t num_slots, int32_t num_slices,
                const int32_t *slice_sizes, int32_t max_rank) {
    if (n < 0 || n > kMaxRows || num_slots < 1 || num_slots > kMaxSlots) return LORA_EINVAL;
    if (num_slices < 1 || num_slices > kMaxSlices) return LORA_EINVAL;
    if (int rc = check_rank(max_rank)) return rc;
    d.n = n;
    d.k_in = k_in;
    d.num_slots = num_slots;
    d.num_slices = num_slices;
    d.R = max_rank;
    d.slice_off[0] = 0;
    for (int l = 0; l < num_slices; ++l) {
        const int w = slice_sizes ? slice_sizes[l] : -1;
        if (w <= 0 || w % 8 != 0) return LORA_EINVAL;
        if ((long long)d.slice_off[l] + w > (1 << 28)) return LORA_EINVAL;
        d.slice_off[l + 1] = d.slice_off[l] + w;
    }
    for (int l = num_slices + 1; l <= kMaxSlices; ++l) d.slice_off[l] = d.slice_off[num_slices];
    return LORA_OK;
}

int check_x(const uint16_t *x, int64_t ldx, int32_t k_in) {
    if (!x || !aligned16(x)) return LORA_EINVAL;
    if (k_in < 8 || k_in % 8 != 0 || k_in > (1 << 20)) return LORA_EINVAL;
    if (ldx < k_in || ldx % 8 != 0) return LORA_EINVAL;
    return LORA_OK;
}

int check_y(const uint16_t *y, int64_t ldy, int32_t offset_start, int n_out) {
    if (!y || !aligned16(y)) return LORA_EINVAL;
    if (offset_start < 0 || offset_start % 8 != 0) return LORA_EINVAL;
    if (ldy % 8 != 0 || ldy < (int64_t)offset_start + n_out) return LORA_EINVAL;
    return LORA_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ELAUNCH; }

// A MoE call without pairs reads and writes no rows: its row and routing
// pointers may be null (sizes and strides are still checked).
// (the placeholder is a non-null, 16-byte aligned address that is never read)
template <class T>
const T *rows_or_placeholder(const T *p, long long n_pairs) {
    constexpr uintptr_t kPlaceholder = 256;
    return n_pairs > 0 ? p : reinterpret_cast<const T *>(kPlaceholder);
}

}  // namespace

extern "C" {

int32_t lora_meta_max_tiles(int32_t n, int32_t num_slots) { return tile_bound(n, num_slots); }

size_t lora_meta_workspace_bytes(int32_t n, int32_t num_slots) {
    if (check_meta_shape(n, num_slots) != LORA_OK) return 0;
    return meta_ws_bytes(n, num_slots);
}

int lora_meta_build(const int32_t *slot, int32_t n, int32_t num_slots, lora_meta_t meta, void *ws,
                    size_t ws_bytes, void *stream) {
    if (int rc = check_meta_shape(n, num_slots)) return rc;
    if (!meta_ok(meta) || (n > 0 && !slot)) return LORA_EINVAL;
    const size_t need = meta_ws_bytes(n, num_slots);
    if (need && (!ws || ws_bytes < need)) return LORA_EWORKSPACE;
    tl::MetaOut out{meta.sorted_rows, meta.seg_offsets, meta.seg_slot, meta.counts, meta.tiles,
                    tile_bound(n, num_slots)};
    return launched(tl::launch_meta_dense(slot, n, num_slots, out, carve_meta_ws(ws, n, num_slots),
                                          static_cast<hipStream_t>(stream)));
}

int lora_meta_from_offsets(const uint32_t *expert_offsets, int32_t num_experts, const int32_t *expert_slot,
                           int32_t n, int32_t num_slots, lora_meta_t meta, void *ws, size_t ws_bytes,
                           void *stream) {
    if (int rc = check_meta_shape(n, num_slots)) return rc;
    if (num_experts < 0 || num_experts > kMaxSlots) return LORA_EINVAL;
    if (!meta_ok(meta) || !expert_offsets || (num_experts > 0 && !expert_slot)) return LORA_EINVAL;
    const size_t need = meta_ws_bytes(n, num_slots);
    if (need && (!ws || ws_bytes < need)) return LORA_EWORKSPACE;
    tl::MetaOut out{meta.sorted_rows, meta.seg_offsets, meta.seg_slot, meta.counts, meta.tiles,
                    tile_bound(n, num_slots)};
    return launched(tl::launch_meta_blocks(expert_offsets, expert_slot, num_experts, n, num_slots, out,
                                           carve_meta_ws(ws, n, num_slots), static_cast<hipStream_t>(stream)));
}

int lora_shrink(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in, const uint16_t *a_pool,
                const float *scale, int32_t num_slots, int32_t num_slices, int32_t max_rank, lora_meta_t meta,
                float *xa, void *stream) {
    tl::DenseShape d{};
    int32_t dummy[kMaxSlices];
    for (int l = 0; l < kMaxSlices; ++l) dummy[l] = 8;
    if (int rc = dense_shape(d, n, k_in, num_slots, num_slices, dummy, max_rank)) return rc;
    if (int rc = check_x(x, ldx, k_in)) return rc;
    if (!a_pool || !aligned16(a_pool) || !scale || !xa || !aligned16(xa) || !meta_ok(meta)) return LORA_EINVAL;
    if (n == 0) return LORA_OK;
    d.x = x;
    d.ldx = ldx;
    d.a_pool = a_pool;
    d.scale = scale;
    return launched(tl::launch_shrink(d, meta.tiles, tile_bound(n, num_slots), xa, mfma_min_rows(),
                                      static_cast<hipStream_t>(stream)));
}

int lora_expand(const float *xa, const uint16_t *b_pool, int32_t num_slots, int32_t num_slices,
                const int32_t *slice_sizes, int32_t max_rank, int32_t n, lora_meta_t meta, uint16_t *y,
                int64_t ldy, int32_t offset_start, int32_t add_inputs, void *stream) {
    tl::DenseShape d{};
    if (int rc = dense_shape(d, n, 8, num_slots, num_slices, slice_sizes, max_rank)) return rc;
    if (int rc = check_y(y, ldy, offset_start, d.slice_off[num_slices])) return rc;
    if (!xa || !aligned16(xa) || !b_pool || !aligned16(b_pool) || !meta_ok(meta)) return LORA_EINVAL;
    if (n == 0) return LORA_OK;
    d.b_pool = b_pool;
    d.y = y;
    d.ldy = ldy;
    d.offset_start = offset_start;
    return launched(tl::launch_expand(d, xa, meta.tiles, tile_bound(n, num_slots), add_inputs, mfma_min_rows(),
                                      static_cast<hipStream_t>(stream)));
}

size_t lora_fused_workspace_bytes(int32_t n, int32_t num_slots, int32_t num_slices, int32_t max_rank,
                                  int32_t k_in) {
    if (n < 0 || n > kMaxRows || num_slots < 1 || num_slices < 1 || num_slices > kMaxSlices ||
        check_rank(max_rank) != LORA_OK || k_in < 8)
        return 0;
    return tl::fused_plan(n, num_slots, num_slices, max_rank, k_in, 8).total_bytes;
}

}  // extern "C"

namespace {

// The fused call with its workspace given (ws != null) or, for the
// allocation-free variant (ws == null), the library's fixed device buffer.
// build (lora_delta_fused_build): the call builds meta from slot too,
// in the fused launch itself where fused_builds_meta allows, else with the
// metadata kernel first (its workspace carved after the fused workspace).
int fused_call(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in, const uint16_t *a_pool,
               const uint16_t *b_pool, const float *scale, int32_t num_slots, int32_t num_slices,
               const int32_t *slice_sizes, int32_t max_rank, lora_meta_t meta, uint16_t *y, int64_t ldy,
               int32_t offset_start, void *ws, size_t ws_bytes, bool own_scratch, bool build,
               const int32_t *slot, void *stream) {
    tl::DenseShape d{};
    if (int rc = dense_shape(d, n, k_in, num_slots, num_slices, slice_sizes, max_rank)) return rc;
    if (int rc = check_x(x, ldx, k_in)) return rc;
    if (int rc = check_y(y, ldy, offset_start, d.slice_off[num_slices])) return rc;
    if (!a_pool || !aligned16(a_pool) || !b_pool || !aligned16(b_pool) || !scale || !meta_ok(meta))
        return LORA_EINVAL;
    const tl::FusedPlan plan =
        tl::fused_plan(n, num_slots, num_slices, max_rank, k_in, d.slice_off[num_slices]);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (build) {
        if (int rc = check_meta_shape(n, num_slots)) return rc;
        if (n > 0 && !slot) return LORA_EINVAL;
        const size_t need = plan.total_bytes + meta_ws_bytes(n, num_slots);
        if (!ws || ws_bytes < need || !aligned16(ws)) return LORA_EWORKSPACE;
        tl::MetaOut mo{meta.sorted_rows, meta.seg_offsets, meta.seg_slot, meta.counts, meta.tiles,
                       tile_bound(n, num_slots)};
        const tl::MetaWs meta_ws =
            carve_meta_ws(static_cast<char *>(ws) + plan.total_bytes, n, num_slots,
                          reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kFusedMetaCtl));
        if (n == 0) return launched(tl::launch_meta_dense(slot, n, num_slots, mo, meta_ws, st));
        d.x = x;
        d.ldx = ldx;
        d.a_pool = a_pool;
        d.b_pool = b_pool;
        d.scale = scale;
        d.y = y;
        d.ldy = ldy;
        d.offset_start = offset_start;
        if (tl::fused_builds_meta(d, plan))
            return launched(tl::launch_fused(d, nullptr, nullptr, plan, ws, mfma_min_rows(), st, slot, &mo));
        const hipError_t e = tl::launch_meta_dense(slot, n, num_slots, mo, meta_ws, st);
        if (e != hipSuccess) return LORA_ELAUNCH;
        return launched(tl::launch_fused(d, meta.tiles, meta.counts, plan, ws, mfma_min_rows(), st));
    }
    if (own_scratch) {
        if (plan.total_bytes > (size_t)LORA_NOALLOC_SCRATCH_BYTES) return LORA_ESCRATCH;
        if (n == 0) return LORA_OK;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return LORA_ELAUNCH;
        if (st) {  // the buffer resolved is the current device's: the stream must run there
            hipDevice_t sd = -1;
            if (hipStreamGetDevice(st, &sd) != hipSuccess || sd != dev) return LORA_EINVAL;
        }
        if (tl::noalloc_scratch(dev, &ws) != hipSuccess) return LORA_ELAUNCH;
    } else {
        if (!ws || ws_bytes < plan.total_bytes || !aligned16(ws)) return LORA_EWORKSPACE;
        if (n == 0) return LORA_OK;
    }
    d.x = x;
    d.ldx = ldx;
    d.a_pool = a_pool;
    d.b_pool = b_pool;
    d.scale = scale;
    d.y = y;
    d.ldy = ldy;
    d.offset_start = offset_start;
    return launched(tl::launch_fused(d, meta.tiles, meta.counts, plan, ws, mfma_min_rows(), st));
}

}  // namespace

extern "C" {

int lora_delta_fused(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in, const uint16_t *a_pool,
                     const uint16_t *b_pool, const float *scale, int32_t num_slots, int32_t num_slices,
                     const int32_t *slice_sizes, int32_t max_rank, lora_meta_t meta, uint16_t *y, int64_t ldy,
                     int32_t offset_start, void *ws, size_t ws_bytes, void *stream) {
    return fused_call(x, ldx, n, k_in, a_pool, b_pool, scale, num_slots, num_slices, slice_sizes, max_rank, meta,
                      y, ldy, offset_start, ws, ws_bytes, false, false, nullptr, stream);
}

int lora_delta_fused_noalloc(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in, const uint16_t *a_pool,
                             const uint16_t *b_pool, const float *scale, int32_t num_slots, int32_t num_slices,
                             const int32_t *slice_sizes, int32_t max_rank, lora_meta_t meta, uint16_t *y,
                             int64_t ldy, int32_t offset_start, void *stream) {
    return fused_call(x, ldx, n, k_in, a_pool, b_pool, scale, num_slots, num_slices, slice_sizes, max_rank, meta,
                      y, ldy, offset_start, nullptr, 0, true, false, nullptr, stream);
}

int lora_delta_fused_build(const uint16_t *x, int64_t ldx, int32_t n, int32_t k_in, const uint16_t *a_pool,
                           const uint16_t *b_pool, const float *scale, int32_t num_slots, int32_t num_slices,
                           const int32_t *slice_sizes, int32_t max_rank, const int32_t *slot, lora_meta_t meta,
                           uint16_t *y, int64_t ldy, int32_t offset_start, void *ws, size_t ws_bytes,
                           void *stream) {
    return fused_call(x, ldx, n, k_in, a_pool, b_pool, scale, num_slots, num_slices, slice_sizes, max_rank, meta,
                      y, ldy, offset_start, ws, ws_bytes, false, true, slot, stream);
}

// MoE workspace: a fixed 256-byte header (counts, 8 int32 at byte 0; the
// pair metadata build's counters at byte kMoeMetaCtl; the fused control line
// at byte LORA_MOE_CTL_OFFSET), then [sorted_rows n |
// seg_offsets cap+1 | seg_slot cap | tiles] [meta ws] [fused flags and
// partials].  The header never moves, so the control line's call tag
// survives calls of any shape; the pair metadata's offsets depend only on
// (T, top_k, E, L), so a w2 call can reuse the routing a gemm1 call built.
namespace {
struct MoeLayout {
    size_t counts, ctl, sorted, segoff, segslot, tiles, meta_ws, fused, total;
    tl::FusedPlan plan;
};
static_assert(LORA_MOE_CTL_OFFSET >= 8 * sizeof(int32_t) && LORA_MOE_CTL_OFFSET + 64 <= 256 &&
                  LORA_MOE_CTL_OFFSET % 64 == 0,
              "the control line sits in the header, clear of the counts");
static MoeLayout moe_layout(int T, int top_k, int E, int L, int R, int k_in, int n_sh) {
    MoeLayout m{};
    const int n = T * top_k, S = L * E, cap = n < S ? n : S;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    m.counts = 0;
    m.ctl = LORA_MOE_CTL_OFFSET;
    size_t o = 256;
    m.sorted = o;
    o = up(o + (size_t)n * sizeof(int32_t));
    m.segoff = o;
    o = up(o + (size_t)(cap + 1) * sizeof(int32_t));
    m.segslot = o;
    o = up(o + (size_t)(cap > 0 ? cap : 1) * sizeof(int32_t));
    m.tiles = o;
    o = up(o + (size_t)tile_bound(n, S) * LORA_TILE_WORDS * sizeof(int32_t));
    m.meta_ws = o;
    o = up(o + meta_ws_bytes(n, S));
    m.plan = tl::fused_plan(n, S, n_sh, R, k_in, 8);
    m.fused = o;
    o = up(o + m.plan.total_bytes);
    m.total = o;
    return m;
}
}  // namespace

size_t moe_lora_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts, int32_t num_loras, int32_t rank,
                                int32_t H) {
    if (T < 0 || top_k < 1 || num_experts < 1 || num_loras < 1 || check_rank(rank) != LORA_OK || H < 8)
        return 0;
    if ((long long)T * top_k > kMaxRows || (long long)num_experts * num_loras > kMaxSlots) return 0;
    // the regular form needs the larger partial buffer (two shrink slices)
    return moe_layout(T, top_k, num_experts, num_loras, rank, H, 2).total;
}

int moe_lora_gemm1_delta(const uint16_t *x, int64_t ldx, int32_t T, int32_t H, const int64_t *w_ptr_a,
                         int64_t lora_stride_a, const int64_t *w_ptr_b, int64_t lora_stride_b, int32_t shared_a,
                         const int32_t *topk_ids, int32_t top_k, const int32_t *lora_ids, int32_t num_experts,
                         int32_t num_loras, int32_t rank, int32_t inter, float scale, uint16_t *out, void *ws,
                         size_t ws_bytes, void *stream) {
    if (T < 0 || top_k < 1 || num_experts < 1 || num_loras < 1) return LORA_EINVAL;
    if ((long long)T * top_k > kMaxRows || (long long)num_experts * num_loras > kMaxSlots) return LORA_EINVAL;
    if (int rc = check_rank(rank)) return rc;
    const long long np = (long long)T * top_k;
    if (int rc = check_x(rows_or_placeholder(x, np), ldx, H)) return rc;
    if (inter < 8 || inter % 8 != 0 || inter > (1 << 24)) return LORA_EINVAL;
    if (lora_stride_a < 0 || lora_stride_b < 0 || lora_stride_a % 8 != 0 || lora_stride_b % 8 != 0)
        return LORA_EINVAL;
    if (!w_ptr_a || !w_ptr_b) return LORA_EINVAL;
    if (np > 0 && (!topk_ids || !lora_ids || !out || !aligned16(out))) return LORA_EINVAL;
    const int n = T * top_k, S = num_experts * num_loras;
    if (int rc = check_meta_shape(n, S)) return rc;
    const MoeLayout lay = moe_layout(T, top_k, num_experts, num_loras, rank, H, shared_a ? 1 : 2);
    if (!ws || !aligned16(ws) || ws_bytes < lay.total) return LORA_EWORKSPACE;
    char *b = static_cast<char *>(ws);
    tl::MetaOut mo{reinterpret_cast<int32_t *>(b + lay.sorted), reinterpret_cast<int32_t *>(b + lay.segoff),
                   reinterpret_cast<int32_t *>(b + lay.segslot), reinterpret_cast<int32_t *>(b + lay.counts),
                   reinterpret_cast<int32_t *>(b + lay.tiles), tile_bound(n, S)};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = tl::launch_meta_moe(topk_ids, lora_ids, top_k, num_experts, num_loras, n, mo,
                                       carve_meta_ws(b + lay.meta_ws, n, S, reinterpret_cast<int32_t *>(b + kMoeMetaCtl)), st);
    if (e != hipSuccess) return LORA_ELAUNCH;
    if (n == 0) return LORA_OK;
    tl::MoeShape m{x, ldx, T, H, w_ptr_a, lora_stride_a, w_ptr_b, lora_stride_b, shared_a, topk_ids, top_k,
                   lora_ids, num_experts, num_loras, rank, inter, scale, out};
    return launched(tl::launch_moe_delta(m, mo, lay.plan, b + lay.fused, reinterpret_cast<int *>(b + lay.ctl),
                                         mfma_min_rows(), st));
}

size_t moe_lora_w2_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts, int32_t num_loras, int32_t rank,
                                   int32_t I) {
    if (T < 0 || top_k < 1 || num_experts < 1 || num_loras < 1 || check_rank(rank) != LORA_OK || I < 8)
        return 0;
    if ((long long)T * top_k > kMaxRows || (long long)num_experts * num_loras > kMaxSlots) return 0;
    return moe_layout(T, top_k, num_experts, num_loras, rank, I, 1).total;
}

int moe_lora_w2_delta(const uint16_t *x2, int64_t ldx, int32_t T, int32_t I, const int64_t *w_ptr_a,
                      int64_t lora_stride_a, const int64_t *w_ptr_b, int64_t lora_stride_b, const int32_t *topk_ids,
                      int32_t top_k, const int32_t *lora_ids, const float *topk_weights, int32_t num_experts,
                      int32_t num_loras, int32_t rank, int32_t H, float scale, uint16_t *y, int64_t ldy,
                      int32_t reuse_routing, void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || top_k < 1 || num_experts < 1 || num_loras < 1) return LORA_EINVAL;
    if ((long long)T * top_k > kMaxRows || (long long)num_experts * num_loras > kMaxSlots) return LORA_EINVAL;
    if (int rc = check_rank(rank)) return rc;
    const long long np = (long long)T * top_k;
    if (int rc = check_x(rows_or_placeholder(x2, np), ldx, I)) return rc;
    if (H < 8 || H % 8 != 0 || H > (1 << 24)) return LORA_EINVAL;
    if (int rc = check_y(rows_or_placeholder(y, np), ldy, 0, H)) return rc;
    if (lora_stride_a < 0 || lora_stride_b < 0 || lora_stride_a % 8 != 0 || lora_stride_b % 8 != 0)
        return LORA_EINVAL;
    if (!w_ptr_a || !w_ptr_b) return LORA_EINVAL;
    if (np > 0 && (!topk_ids || !lora_ids)) return LORA_EINVAL;
    if (topk_weights && (reinterpret_cast<uintptr_t>(topk_weights) & 3u)) return LORA_EINVAL;
    const int n = T * top_k, S = num_experts * num_loras;
    if (int rc = check_meta_shape(n, S)) return rc;
    const MoeLayout lay = moe_layout(T, top_k, num_experts, num_loras, rank, I, 1);
    if (!ws || !aligned16(ws) || ws_bytes < lay.total) return LORA_EWORKSPACE;
    char *b = static_cast<char *>(ws);
    tl::MetaOut mo{reinterpret_cast<int32_t *>(b + lay.sorted), reinterpret_cast<int32_t *>(b + lay.segoff),
                   reinterpret_cast<int32_t *>(b + lay.segslot), reinterpret_cast<int32_t *>(b + lay.counts),
                   reinterpret_cast<int32_t *>(b + lay.tiles), tile_bound(n, S)};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (!reuse_routing) {
        const hipError_t e = tl::launch_meta_moe(topk_ids, lora_ids, top_k, num_experts, num_loras, n, mo,
                                                 carve_meta_ws(b + lay.meta_ws, n, S, reinterpret_cast<int32_t *>(b + kMoeMetaCtl)), st);
        if (e != hipSuccess) return LORA_ELAUNCH;
    }
    if (n == 0) return LORA_OK;
    tl::MoeW2Shape m{x2, ldx, T, I, w_ptr_a, lora_stride_a, w_ptr_b, lora_stride_b, top_k, topk_weights,
                     num_experts, num_loras, rank, H, scale, y, ldy};
    return launched(
        tl::launch_moe_w2_delta(m, mo, lay.plan, b + lay.fused, reinterpret_cast<int *>(b + lay.ctl),
                                mfma_min_rows(), st));
}

int moe_lora_meta_layout(int32_t T, int32_t top_k, int32_t num_experts, int32_t num_loras, size_t *offsets) {
    if (!offsets || T < 0 || top_k < 1 || num_experts < 1 || num_loras < 1) return LORA_EINVAL;
    if ((long long)T * top_k > kMaxRows || (long long)num_experts * num_loras > kMaxSlots) return LORA_EINVAL;
    // the metadata part of the layout does not depend on rank, width or form
    const MoeLayout lay = moe_layout(T, top_k, num_experts, num_loras, 8, 8, 1);
    offsets[0] = lay.counts;
    offsets[1] = lay.sorted;
    offsets[2] = lay.segoff;
    offsets[3] = lay.segslot;
    offsets[4] = lay.tiles;
    return LORA_OK;
}

int32_t lora_mfma_min_rows(void) { return mfma_min_rows(); }

void lora_set_mfma_min_rows(int32_t rows) { t_mfma_min = rows > 0 ? rows : 0; }

const char *lora_status_string(int status) {
    switch (status) {
    case LORA_OK: return "ok";
    case LORA_EINVAL: return "invalid argument (pointer, size, alignment or leading dimension)";
    case LORA_EUNSUPPORTED: return "unsupported shape";
    case LORA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LORA_ELAUNCH: return "kernel launch failed";
    case LORA_ESCRATCH: return "the call needs more workspace than the library's fixed device buffer holds";
    default: return "unknown status";
    }
}

}  // extern "C"
