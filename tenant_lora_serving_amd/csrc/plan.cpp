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

}  // namespace tl
