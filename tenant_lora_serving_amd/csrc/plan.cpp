// plan.cpp -- host-side sizing shared by the C entry points and the
// launchers: how many metadata chunks a batch has, and the fused workspace's
// layout.  Plain host C++ (no device code), so the validation layer can also
// be built for the host alone.
#include <algorithm>

#include "kernels.h"

namespace tl {

int meta_chunks(int n) { return n <= 0 ? 1 : (n + kMetaChunk - 1) / kMetaChunk; }

// Fused workspace: [control line, 256 B] [per tile: kFlagWords 64-bit words, P piece
// flags .. the finished-consumer count] [tagged partials: tile_bound x P x n_rr x 16 uint64].
// Sized for the most pieces any launch of this shape can use: one per kKP k,
// at most kFlagWords - 1 (the launcher picks the actual count).
FusedPlan fused_plan(int n, int num_slots, int n_sh, int R, int k_in, int n_out) {
    (void)n_out;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    FusedPlan p{};
    p.tile_bound = tile_bound_of(n, num_slots);
    const int steps = (k_in + kKP - 1) / kKP;
    const int ks = std::max(1, (steps + kFlagWords - 2) / (kFlagWords - 1));
    const int p_max = (steps + ks - 1) / ks;
    p.flag_bytes = up(256 + (size_t)p.tile_bound * kFlagWords * sizeof(uint64_t));
    p.part_bytes = up((size_t)p.tile_bound * p_max * n_sh * R * kTileRows * sizeof(uint64_t));
    p.total_bytes = p.flag_bytes + p.part_bytes;
    return p;
}

// Mode 0 (one 512-column batch per expand unit, one 512-k step per shrink
// unit): what launch_fused_op picks for these expand units and this k_in.
bool narrow_call(int k_in, int EC) {
    const int steps = (k_in + kKP - 1) / kKP;
    return EC <= kEB && steps <= kFlagWords - 1;
}

int chunks_of(const int *off, int n_windows, int EC) {
    int c = 0;
    for (int l = 0; l < n_windows; ++l) c += (off[l + 1] - off[l] + EC - 1) / EC;
    return c;
}

// Columns per expand unit: 512 while that keeps the expand units of a call
// within about 2048 workgroups, else 1024 or 2048, so that each unit's read
// of the tile's partials and its fixed chain latency cover more columns.
// Past that, the widest chunk of 5..8 batches that cuts every window into
// equal whole-batch chunks, if one does (a ragged last chunk per window
// leaves short units at the end of the call).
int expand_width(const int *off, int n_windows, int tile_bound) {
    int ec = kEB;
    while (ec < 4 * kEB && (long long)tile_bound * chunks_of(off, n_windows, ec) > 2048) ec *= 2;
    if (ec == 4 * kEB && (long long)tile_bound * chunks_of(off, n_windows, ec) > 2048) {
        for (int e = 8; e > 4; --e) {
            bool even = true;
            for (int l = 0; l < n_windows; ++l) even = even && ((off[l + 1] - off[l] + kEB - 1) / kEB) % e == 0;
            if (even) return e * kEB;
        }
    }
    return ec;
}

// One launch builds the metadata too: a batch of at most kSlotThreads rows
// over at most kSmallBallotSlots slots whose call runs in mode 0.
bool fused_builds_meta(const DenseShape &d, const FusedPlan &plan) {
    return d.n <= kSlotThreads && d.num_slots <= kSmallBallotSlots &&
           narrow_call(d.k_in, expand_width(d.slice_off, d.num_slices, plan.tile_bound));
}

}  // namespace tl
