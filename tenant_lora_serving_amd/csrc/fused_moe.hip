// fused_moe.hip -- the routed-MoE gemm1 delta's launch (moe_lora_gemm1_delta);
// the kernels are in fused.h.
#include "fused.h"
#include "segment.h"

namespace tl {

template <int G, int RK>
static hipError_t launch_segment(const MoeOp &op, const SegArgs &sa, const ZeroFill &zf, int zero_units,
                                 hipStream_t st) {
    hipLaunchKernelGGL((segment_kernel<G, RK, MoeOp>), dim3((unsigned)(sa.n_units + sa.tile_bound + zero_units)),
                       dim3(256), 0, st, op, sa, zf);
    return hipGetLastError();
}

hipError_t launch_moe_delta(const MoeShape &m, const MetaOut &meta, const FusedPlan &plan, void *ws, int *ctl,
                            int mfma_min, hipStream_t st) {
    const int32_t *tiles = meta.tiles, *counts = meta.counts;
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
    // Ranks 8, 16 and 32, with segments of at most 64 pairs on average: one
    // workgroup per segment does the shrink and the expand (segment.h).
    // Other shapes take the fused kernel's hand-off between workgroups, which
    // spreads a long segment over many.  The buffer resources of the segment
    // kernel need every extent below 2^31 bytes.
    const int G = (op.n_sh * m.R + 15) / 16;
    const long long S = (long long)m.E * m.L, cap = n_pairs < S ? n_pairs : S;
    const bool fits = (long long)m.T * m.ldx * 2 < (1ll << 31) && (long long)n_pairs * op.n_out * 2 < (1ll << 31);
    if (n_pairs > 0 && fits && (long long)n_pairs <= 64 * S) {
        const SegArgs sa{tiles,  plan.tile_bound, meta.sorted_rows, meta.seg_offsets, meta.seg_slot, counts, (int)cap,
                         n_pairs, ctl, m.E};
        switch (m.R * 8 + G) {
        case 8 * 8 + 1: return launch_segment<1, 8>(op, sa, zf, zero_units, st);
        case 16 * 8 + 1: return launch_segment<1, 16>(op, sa, zf, zero_units, st);
        case 16 * 8 + 2: return launch_segment<2, 16>(op, sa, zf, zero_units, st);
        case 32 * 8 + 2: return launch_segment<2, 32>(op, sa, zf, zero_units, st);
        case 32 * 8 + 4: return launch_segment<4, 32>(op, sa, zf, zero_units, st);
        default: break;
        }
    }
    const int off[3] = {0, m.inter, 2 * m.inter};
    const int EC = expand_width(off, 2, plan.tile_bound);
    const int C = chunks_of(off, 2, EC);
    const bool lean = (long long)n_pairs >= (long long)mfma_min * m.E * m.L;
    return launch_fused_op(op, tiles, counts, plan, C, EC, ws, ctl, mfma_min, lean, 0, zf, zero_units, st);
}

}  // namespace tl
