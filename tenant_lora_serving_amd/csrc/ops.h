// ops.h -- addressing policies of the routed LoRA delta kernels: where a row's
// input, an adapter's A and B rows and a row's output live.  Internal to the
// library; the kernels are written once against this interface.
//
// Rank rows: the shrink computes n_rr = n_sh * R values per row, rank row
// rr = l * R + r belonging to shrink slice l.  Output slices: the expand
// writes n_xs column windows [xoff(l), xoff(l + 1)), each fed by the R rank
// rows of xa block xblk(l).  kRowWeights: xa of row i is also multiplied by
// row_weight(i) (a per-row router weight).
#pragma once

#include "common.h"
#include "kernels.h"

namespace tl {

// Dense delta (vLLM punica_base.py, add_shrink / add_expand: one A and one
// block of B rows per output slice; metrale lora_delta, LoraPair layout).
struct DenseOp {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *a_pool;
    const uint16_t *b_pool;
    const float *scale;
    uint16_t *y;
    int64_t ldy;
    int k_in, R, n_sh, n_out, col0, n_sl;
    int off[kMaxSlices + 1];
    static constexpr bool kRowWeights = false;
    static constexpr bool kXOnce = true;  // each x element is read by one unit
    static constexpr int kRank = 0;  // R is a runtime value
    static constexpr bool kBuild = false;  // tile records come from the metadata

    __device__ int n_rr() const { return n_sh * R; }
    __device__ int n_xs() const { return n_sl; }
    __device__ const uint16_t *xrow(int row) const { return x + (int64_t)row * ldx; }
    // rank row rr = l*R + r of slot s: a_pool[s][l][r][:]
    __device__ const uint16_t *arow(int slot, int rr) const {
        return a_pool + ((int64_t)slot * n_sh * R + rr) * k_in;
    }
    // slice of output column c; unrolled so off[] is only read at constant
    // indices (a runtime index would move the kernel argument to scratch)
    __device__ int xslice(int c) const {
        int l = 0;
#pragma unroll
        for (int i = 1; i < kMaxSlices; ++i) l += (i < n_sl && c >= off[i]) ? 1 : 0;
        return l;
    }
    // output window of slice l (l a compile-time constant at every call)
    __device__ int xoff(int l) const { return off[l]; }
    __device__ int xblk(int l) const { return l; }
    __device__ const uint16_t *brow(int slot, int c) const {
        return b_pool + ((int64_t)slot * n_out + c) * R;
    }
    __device__ uint16_t *yrow(int row) const { return y + (int64_t)row * ldy + col0; }
    __device__ float scale_of(int slot) const { return scale[slot]; }
    __device__ float row_weight(int) const { return 1.f; }
};

// The dense delta at a rank fixed at compile time (R == RK): decode-sized
// calls at a common rank, where the fixed rank lets the kernel fit four
// waves per SIMD.  Same layout and arithmetic as DenseOp.
template <int RK>
struct DenseOpR : DenseOp {
    static constexpr int kRank = RK;

    __device__ int n_rr() const { return n_sh * RK; }
    __device__ const uint16_t *arow(int slot, int rr) const {
        return a_pool + ((int64_t)slot * n_sh * RK + rr) * k_in;
    }
    __device__ const uint16_t *brow(int slot, int c) const { return b_pool + ((int64_t)slot * n_out + c) * RK; }
};

// A dense op whose launch also builds the batch's metadata: each unit derives
// its tile's record from the slot array (the fused kernel's mode 0 only).
template <class Base>
struct BuildOp : Base {
    static constexpr bool kBuild = true;
};

// Routed MoE gemm1 (FlashInfer bgmv_moe_gemm1_lora_delta): key = l*E + e,
// rows are (token, slot) pairs; output window 0 is gate, window 1 is up.
struct MoeOp {
    const uint16_t *x;
    int64_t ldx;
    int top_k;
    const int64_t *wa;
    int64_t lsa;
    const int64_t *wb;
    int64_t lsb;
    uint16_t *out;
    float sc;
    int k_in, R, n_sh, n_out, E, inter, shared;
    static constexpr bool kRowWeights = false;
    static constexpr bool kXOnce = false;  // a token's x row serves its top_k pairs
    static constexpr bool kAddInputs = false;  // out is written, not added to
    static constexpr int kRank = 0;
    static constexpr bool kBuild = false;

    __device__ int n_rr() const { return n_sh * R; }
    __device__ int n_xs() const { return 2; }
    __device__ const uint16_t *xrow(int pair) const { return x + (int64_t)(pair / top_k) * ldx; }
    __device__ const uint16_t *arow(int key, int rr) const {
        const int l = key / E, e = key - l * E;
        const int sg = rr / R, r = rr - sg * R;
        const uint16_t *base = reinterpret_cast<const uint16_t *>(wa[shared ? e : sg * E + e]);
        return base + (int64_t)l * lsa + (int64_t)r * k_in;
    }
    __device__ int xslice(int c) const { return shared ? 0 : (c >= inter ? 1 : 0); }
    __device__ int xoff(int l) const { return l * inter; }
    __device__ int xblk(int l) const { return shared ? 0 : l; }
    __device__ const uint16_t *brow(int key, int c) const {
        const int l = key / E, e = key - l * E;
        if (shared)
            return reinterpret_cast<const uint16_t *>(wb[e]) + (int64_t)l * lsb + (int64_t)c * R;
        const int sg = c >= inter ? 1 : 0;
        return reinterpret_cast<const uint16_t *>(wb[sg * E + e]) + (int64_t)l * lsb +
               (int64_t)(c - sg * inter) * R;
    }
    __device__ uint16_t *yrow(int pair) const { return out + (int64_t)pair * n_out; }
    __device__ float scale_of(int) const { return sc; }
    __device__ float row_weight(int) const { return 1.f; }

    // The (adapter, expert) matrices of one key, resolved once: table reads
    // inside a load loop would each be followed by a wait for every load in
    // flight (the next load's address depends on them).
    struct Bases {
        const uint16_t *a[2];
        const uint16_t *b[2];
    };
    __device__ Bases bases(int key) const {
        const int l = key / E, e = key - l * E;
        Bases bs;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const int ia = shared ? e : sg * E + e;
            bs.a[sg] = reinterpret_cast<const uint16_t *>(wa[ia]) + (int64_t)l * lsa;
            bs.b[sg] = reinterpret_cast<const uint16_t *>(wb[ia]) + (int64_t)l * lsb;
        }
        return bs;
    }
    // rank row rr of the resolved key (rows R.. belong to the up slice)
    __device__ const uint16_t *arow_b(const Bases &bs, int rr) const {
        const int sg = rr >= R ? 1 : 0;
        return bs.a[sg] + (int64_t)(rr - sg * R) * k_in;
    }
    // output column c of the resolved key (gate columns 0..I, up I..2I)
    __device__ const uint16_t *brow_b(const Bases &bs, int c) const {
        if (shared) return bs.b[0] + (int64_t)c * R;
        const int sg = c >= inter ? 1 : 0;
        return bs.b[sg] + (int64_t)(c - sg * inter) * R;
    }

    // Buffer resources and byte offsets (all extents below 2^31 bytes; the
    // launcher checks): x rows of n_rows pairs, slice sg of a key's A and B,
    // the output rows.
    __device__ rsrc_t x_rsrc(int n_rows) const {
        return make_rsrc(x, (uint32_t)((int64_t)(n_rows / top_k) * ldx * 2));
    }
    __device__ uint32_t x_off(int pair, int k) const {
        return (uint32_t)(((int64_t)(pair / top_k) * ldx + k) * 2);
    }
    __device__ rsrc_t a_rsrc(const Bases &bs, int sg) const {
        return make_rsrc(bs.a[shared ? 0 : sg], (uint32_t)(R * k_in * 2));
    }
    __device__ uint32_t a_off(int r, int k) const { return (uint32_t)((r * k_in + k) * 2); }
    // window l's B: its own matrix (regular) or rows l*I.. of the fused one
    __device__ rsrc_t b_rsrc(const Bases &bs, int l) const {
        return shared ? make_rsrc(bs.b[0], (uint32_t)(2 * inter * R * 2)) : make_rsrc(bs.b[l], (uint32_t)(inter * R * 2));
    }
    __device__ uint32_t b_off(int l, int cw, int rk) const {
        return (uint32_t)(((shared ? l * inter + cw : cw) * R + rk) * 2);
    }
    __device__ rsrc_t y_rsrc(int n_rows) const { return make_rsrc(out, (uint32_t)((int64_t)n_rows * n_out * 2)); }
    __device__ uint32_t y_off(int pair, int col) const { return (uint32_t)(((int64_t)pair * n_out + col) * 2); }
};

// Routed MoE down projection (vLLM punica_base.py, add_lora_w2): rows are
// (token, slot) pairs p, each with its own input row x2[p] (the activated
// gemm1 output) and output row y[p] (added to in place); key = l*E + e; one
// shrink slice and one output window [0, H); xa of pair p is scaled by the
// pair's router weight when weights are given.
struct MoeW2Op {
    const uint16_t *x;
    int64_t ldx;
    const int64_t *wa;
    int64_t lsa;
    const int64_t *wb;
    int64_t lsb;
    const float *wt;  // [n_pairs] router weights, or null
    uint16_t *y;
    int64_t ldy;
    float sc;
    int k_in, R, n_sh, n_out, E;
    static constexpr bool kRowWeights = true;
    static constexpr bool kXOnce = true;  // x rows are per pair
    static constexpr int kRank = 0;
    static constexpr bool kBuild = false;

    __device__ int n_rr() const { return R; }
    __device__ int n_xs() const { return 1; }
    __device__ const uint16_t *xrow(int pair) const { return x + (int64_t)pair * ldx; }
    __device__ const uint16_t *arow(int key, int rr) const {
        const int l = key / E, e = key - l * E;
        return reinterpret_cast<const uint16_t *>(wa[e]) + (int64_t)l * lsa + (int64_t)rr * k_in;
    }
    __device__ int xslice(int) const { return 0; }
    __device__ int xoff(int l) const { return l * n_out; }
    __device__ int xblk(int) const { return 0; }
    __device__ const uint16_t *brow(int key, int c) const {
        const int l = key / E, e = key - l * E;
        return reinterpret_cast<const uint16_t *>(wb[e]) + (int64_t)l * lsb + (int64_t)c * R;
    }
    __device__ uint16_t *yrow(int pair) const { return y + (int64_t)pair * ldy; }
    __device__ float scale_of(int) const { return sc; }
    __device__ float row_weight(int pair) const { return wt ? wt[pair] : 1.f; }

    static constexpr bool kAddInputs = true;  // y is added to in place
    // The key's matrices resolved once (see MoeOp::Bases); one slice.
    struct Bases {
        const uint16_t *a[1];
        const uint16_t *b[1];
    };
    __device__ Bases bases(int key) const {
        const int l = key / E, e = key - l * E;
        Bases bs;
        bs.a[0] = reinterpret_cast<const uint16_t *>(wa[e]) + (int64_t)l * lsa;
        bs.b[0] = reinterpret_cast<const uint16_t *>(wb[e]) + (int64_t)l * lsb;
        return bs;
    }
    // buffer resources and byte offsets (extents below 2^31 bytes, checked by the launcher)
    __device__ rsrc_t x_rsrc(int n_rows) const { return make_rsrc(x, (uint32_t)((int64_t)n_rows * ldx * 2)); }
    __device__ uint32_t x_off(int pair, int k) const { return (uint32_t)(((int64_t)pair * ldx + k) * 2); }
    __device__ rsrc_t a_rsrc(const Bases &bs, int) const { return make_rsrc(bs.a[0], (uint32_t)(R * k_in * 2)); }
    __device__ uint32_t a_off(int r, int k) const { return (uint32_t)((r * k_in + k) * 2); }
    __device__ rsrc_t b_rsrc(const Bases &bs, int) const { return make_rsrc(bs.b[0], (uint32_t)(n_out * R * 2)); }
    __device__ uint32_t b_off(int, int cw, int rk) const { return (uint32_t)((cw * R + rk) * 2); }
    __device__ rsrc_t y_rsrc(int n_rows) const { return make_rsrc(y, (uint32_t)((int64_t)n_rows * ldy * 2)); }
    __device__ uint32_t y_off(int pair, int col) const { return (uint32_t)(((int64_t)pair * ldy + col) * 2); }
};

}  // namespace tl
