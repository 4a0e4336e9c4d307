// fused_dense.hip -- the dense routed LoRA delta's launch (lora_delta_fused,
// and lora_delta_fused_build when it can build the metadata in the same
// launch); the kernels are in fused.h.
#include "fused.h"

namespace tl {

hipError_t launch_fused(const DenseShape &d, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                        void *ws, int mfma_min, hipStream_t st, const int32_t *slot, const MetaOut *meta_out) {
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
    if (slot) {
        if (!meta_out || !fused_builds_meta(d, plan)) return hipErrorInvalidValue;
        const SlotBuild sb{slot, d.n, d.num_slots, *meta_out};
        if (d.R == 16) {
            BuildOp<DenseOpR<16>> o16;
            static_cast<DenseOp &>(o16) = op;
            return launch_fused_op(o16, nullptr, nullptr, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st, &sb);
        }
        BuildOp<DenseOp> ob;
        static_cast<DenseOp &>(ob) = op;
        return launch_fused_op(ob, nullptr, nullptr, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st, &sb);
    }
    if (d.R == 16 && narrow_call(d.k_in, EC)) {
        DenseOpR<16> o16;
        static_cast<DenseOp &>(o16) = op;
        return launch_fused_op(o16, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st);
    }
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, nz, 0, st);
}

}  // namespace tl
