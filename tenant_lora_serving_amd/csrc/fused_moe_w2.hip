// fused_moe_w2.hip -- the routed-MoE down-projection delta's launch
// (moe_lora_w2_delta); the kernels are in fused.h.
#include "fused.h"

namespace tl {

hipError_t launch_moe_w2_delta(const MoeW2Shape &m, const int32_t *tiles, const int32_t *counts,
                               const FusedPlan &plan, void *ws, int *ctl, int mfma_min, hipStream_t st) {
    MoeW2Op op{};
    op.x = m.x2;
    op.ldx = m.ldx;
    op.wa = m.w_ptr_a;
    op.lsa = m.lora_stride_a;
    op.wb = m.w_ptr_b;
    op.lsb = m.lora_stride_b;
    op.wt = m.topk_weights;
    op.y = m.y;
    op.ldy = m.ldy;
    op.sc = m.scale;
    op.k_in = m.I;
    op.R = m.R;
    op.n_sh = 1;
    op.n_out = m.H;
    op.E = m.E;
    // unrouted pairs keep their y row: nothing to zero
    const ZeroFill zf{nullptr, nullptr, m.top_k, m.E, m.L, 0};
    const int off[2] = {0, m.H};
    const int EC = expand_width(off, 1, plan.tile_bound);
    const int C = chunks_of(off, 1, EC);
    const bool lean = (long long)m.T * m.top_k >= (long long)mfma_min * m.E * m.L;
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, zf, 0, st);
}

}  // namespace tl
