// fused_moe.hip -- the routed-MoE gemm1 delta's launch (moe_lora_gemm1_delta);
// the kernels are in fused.h.
#include "fused.h"

namespace tl {

hipError_t launch_moe_delta(const MoeShape &m, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                            void *ws, int *ctl, int mfma_min, hipStream_t st) {
    MoeOp op{};
    op.x = m.x;
    op.ldx = m.ldx;
    op.top_k = m.top_k;
    op.wa = m.w_ptr_a;
    op.lsa = m.lora_stride_a;
    op.wb = m.w_ptr_b;
    op.lsb = m.lora_stride_b;
    op.out = m.out;
    op.sc = m.scale;
    op.k_in = m.H;
    op.R = m.R;
    op.n_sh = m.shared_a ? 1 : 2;
    op.n_out = 2 * m.inter;
    op.E = m.E;
    op.inter = m.inter;
    op.shared = m.shared_a ? 1 : 0;
    const int n_pairs = m.T * m.top_k;
    const ZeroFill zf{m.topk_ids, m.lora_ids, m.top_k, m.E, m.L, n_pairs};
    const int zero_units = (n_pairs + 15) / 16;
    const int off[3] = {0, m.inter, 2 * m.inter};
    const int EC = expand_width(off, 2, plan.tile_bound);
    const int C = chunks_of(off, 2, EC);
    const bool lean = (long long)n_pairs >= (long long)mfma_min * m.E * m.L;
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 0, zf, zero_units, st);
}

}  // namespace tl
