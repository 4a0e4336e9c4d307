// fused_dense.hip -- the dense routed LoRA delta's launch (lora_delta_fused)
// and the fused workspace plan; the kernels are in fused.h.
#include "fused.h"

namespace tl {

// Workspace: [control line, 256 B] [per tile: kFlagWords 64-bit words, P piece
// flags .. the finished-consumer count] [tagged partials: tile_bound x P x n_rr x 16 uint64].
// Sized for the most pieces any launch of this shape can use: one per 512 k,
// at most kFlagWords - 1 (launch_fused_op picks the actual count).
FusedPlan fused_plan(int n, int num_slots, int n_sh, int R, int k_in, int n_out) {
    (void)n_out;
    FusedPlan p{};
    p.tile_bound = tile_bound_of(n, num_slots);
    const int steps = (k_in + kKP - 1) / kKP;
    const int ks = std::max(1, (steps + kFlagWords - 2) / (kFlagWords - 1));
    const int p_max = (steps + ks - 1) / ks;
    p.flag_bytes = align_up(256 + (size_t)p.tile_bound * kFlagWords * sizeof(uint64_t), 256);
    p.part_bytes = align_up((size_t)p.tile_bound * p_max * n_sh * R * kTileRows * sizeof(uint64_t), 256);
    p.total_bytes = p.flag_bytes + p.part_bytes;
    return p;
}

hipError_t launch_fused(const DenseShape &d, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                        void *ws, int mfma_min, hipStream_t st) {
    DenseOp op{};
    op.x = d.x;
    op.ldx = d.ldx;
    op.a_pool = d.a_pool;
    op.b_pool = d.b_pool;
    op.scale = d.scale;
    op.y = d.y;
    op.ldy = d.ldy;
    op.k_in = d.k_in;
    op.R = d.R;
    op.n_sh = d.num_slices;
    op.n_sl = d.num_slices;
    op.n_out = d.slice_off[d.num_slices];
    op.col0 = d.offset_start;
    for (int l = 0; l <= kMaxSlices; ++l) op.off[l] = d.slice_off[l < d.num_slices ? l : d.num_slices];
    const int EC = expand_width(d.slice_off, d.num_slices, plan.tile_bound);
    const int C = chunks_of(d.slice_off, d.num_slices, EC);
    const bool lean = (long long)d.n >= (long long)mfma_min * d.num_slots;
    const ZeroFill nz{nullptr, nullptr, 1, 1, 1, 0};
    // the control line is the first 256 bytes of the fused workspace
    int *ctl = static_cast<int *>(ws);
    if (d.R == 16 && narrow_call(d.k_in, EC)) {
        DenseOpR<16> o16;
        static_cast<DenseOp &>(o16) = op;
        return launch_fused_op(o16, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st);
    }
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st);
}

}  // namespace tl
