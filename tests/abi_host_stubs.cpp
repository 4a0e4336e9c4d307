// abi_host_stubs.cpp -- host stand-ins for the library's device launchers and
// for the two HIP runtime calls the C entry points make, linked with abi.cpp
// and plan.cpp into a host-only build of the C ABI that runs under
// AddressSanitizer and UndefinedBehaviorSanitizer with no GPU.  Each stub
// counts its calls and keeps the arguments a test wants to check (sizes and
// the device addresses the entry point derived from its workspace); nothing
// here dereferences a device address.
#include <string.h>

#include "../tenant_lora_serving_amd/csrc/kernels.h"

namespace {

enum Kind { kMetaDense, kMetaMoe, kMetaBlocks, kShrink, kExpand, kFused, kMoe, kMoeW2, kScratch, kKinds };
constexpr int kVals = 12;
long long g_calls[kKinds];
long long g_val[kKinds][kVals];

void rec(int k, std::initializer_list<long long> v) {
    ++g_calls[k];
    int i = 0;
    for (long long x : v) g_val[k][i++] = x;
}

long long p(const void *q) { return (long long)(const char *)q; }

// A device address that no test passes in: what the fixed buffer resolves to.
constexpr long long kScratchAddr = 0x7f0000000000LL;

}  // namespace

extern "C" {

void stub_reset(void) {
    memset(g_calls, 0, sizeof(g_calls));
    memset(g_val, 0, sizeof(g_val));
}
long long stub_calls(int kind) { return (kind >= 0 && kind < kKinds) ? g_calls[kind] : -1; }
long long stub_value(int kind, int i) { return (kind >= 0 && kind < kKinds && i >= 0 && i < kVals) ? g_val[kind][i] : 0; }
long long stub_scratch_address(void) { return kScratchAddr; }

hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *d) {
    *d = 0;
    return hipSuccess;
}

}  // extern "C"

namespace tl {

size_t meta_dyn_lds(int, int) { return 0; }

static void rec_meta(int k, const MetaOut &o, const MetaWs &w, long long a, long long b) {
    rec(k, {p(o.sorted_rows), p(o.seg_offsets), p(o.seg_slot), p(o.counts), p(o.tiles), o.tile_bound, p(w.ctl),
            p(w.rows), p(w.keys), p(w.offlen), a, b});
}

hipError_t launch_meta_dense(const int32_t *slot, int n, int S, MetaOut out, MetaWs ws, hipStream_t) {
    (void)slot;
    rec_meta(kMetaDense, out, ws, n, S);
    return hipSuccess;
}
hipError_t launch_meta_moe(const int32_t *, const int32_t *, int top_k, int, int, int n_pairs, MetaOut out,
                           MetaWs ws, hipStream_t) {
    rec_meta(kMetaMoe, out, ws, n_pairs, top_k);
    return hipSuccess;
}
hipError_t launch_meta_blocks(const uint32_t *, const int32_t *, int n_blocks, int n, int, MetaOut out, MetaWs ws,
                              hipStream_t) {
    rec_meta(kMetaBlocks, out, ws, n, n_blocks);
    return hipSuccess;
}
hipError_t launch_shrink(const DenseShape &d, const int32_t *tiles, int tile_bound, float *xa, int mfma_min,
                         hipStream_t) {
    rec(kShrink, {d.n, d.k_in, d.R, p(tiles), tile_bound, p(xa), mfma_min});
    return hipSuccess;
}
hipError_t launch_expand(const DenseShape &d, const float *xa, const int32_t *tiles, int tile_bound, int add_inputs,
                         int mfma_min, hipStream_t) {
    rec(kExpand, {d.n, d.slice_off[d.num_slices], d.R, p(tiles), tile_bound, p(xa), add_inputs, mfma_min});
    return hipSuccess;
}
hipError_t launch_fused(const DenseShape &d, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                        void *ws, int mfma_min, hipStream_t, const int32_t *slot, const MetaOut *meta_out) {
    rec(kFused, {d.n, d.k_in, d.slice_off[d.num_slices], p(tiles), p(counts), plan.tile_bound,
                 (long long)plan.total_bytes, p(ws), mfma_min, p(slot), meta_out ? p(meta_out->tiles) : 0,
                 meta_out ? meta_out->tile_bound : -1});
    return hipSuccess;
}
hipError_t noalloc_scratch(int device, void **ptr) {
    rec(kScratch, {device});
    *ptr = (void *)kScratchAddr;
    return hipSuccess;
}
hipError_t launch_moe_delta(const MoeShape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                            int mfma_min, hipStream_t) {
    rec(kMoe, {m.T, m.top_k, m.shared_a, p(meta.counts), p(meta.tiles), meta.tile_bound,
               (long long)plan.total_bytes, p(ws), p(ctl), mfma_min});
    return hipSuccess;
}
hipError_t launch_moe_w2_delta(const MoeW2Shape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                               int mfma_min, hipStream_t) {
    rec(kMoeW2, {m.T, m.top_k, m.I, p(meta.counts), p(meta.tiles), meta.tile_bound,
                 (long long)plan.total_bytes, p(ws), p(ctl), mfma_min});
    return hipSuccess;
}

}  // namespace tl
