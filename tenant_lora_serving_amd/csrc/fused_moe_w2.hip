// fused_moe_w2.hip -- the routed-MoE down-projection delta's launch
// (moe_lora_w2_delta); the kernels are in fused.h.
#include "fused.h"
#include "segment.h"

namespace tl {

template <int G, int RK>
static hipError_t launch_segment_w2(const MoeW2Op &op, const SegArgs &sa, hipStream_t st) {
    const ZeroFill none{nullptr, nullptr, 1, 1, 1, 0};
    hipLaunchKernelGGL((segment_kernel<G, RK, MoeW2Op>), dim3((unsigned)(sa.n_units + sa.tile_bound)), dim3(256), 0,
                       st, op, sa, none);
    return hipGetLastError();
}

hipError_t launch_moe_w2_delta(const MoeW2Shape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                               int mfma_min, hipStream_t st) {
    const int32_t *tiles = meta.tiles, *counts = meta.counts;
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
    // ranks 8, 16 and 32 with at most 64 pairs per key on average: one
    // workgroup per segment (segment.h), as for gemm1
    const long long n_pairs = (long long)m.T * m.top_k, S = (long long)m.E * m.L, cap = n_pairs < S ? n_pairs : S;
    const bool fits = n_pairs * m.ldx * 2 < (1ll << 31) && n_pairs * m.ldy * 2 < (1ll << 31);
    if (n_pairs > 0 && fits && n_pairs <= 64 * S) {
        const SegArgs sa{tiles, plan.tile_bound, meta.sorted_rows, meta.seg_offsets, meta.seg_slot, counts, (int)cap,
                         (int)n_pairs, ctl, m.E};
        switch (m.R) {
        case 8: return launch_segment_w2<1, 8>(op, sa, st);
        case 16: return launch_segment_w2<1, 16>(op, sa, st);
        case 32: return launch_segment_w2<2, 32>(op, sa, st);
        default: break;
        }
    }
    const int off[2] = {0, m.H};
    const int EC = expand_width(off, 1, plan.tile_bound);
    const int C = chunks_of(off, 1, EC);
    const bool lean = (long long)m.T * m.top_k >= (long long)mfma_min * m.E * m.L;
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 1, zf, 0, st);
}

}  // namespace tl
