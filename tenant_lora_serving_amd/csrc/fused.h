// fused.h -- the routed LoRA delta in one launch (shrink, then expand) for
// gfx950, dense and routed-MoE gemm1.
//
// Semantics (vLLM punica_base.py, add_lora_linear = add_shrink then
// add_expand; metrale lora_delta docs, apply_lora_bgmv; FlashInfer
// bgmv_moe_gemm1_lora_delta): rows of one adapter slot form a segment; the
// shrink gives xa = scale * x @ A^T in fp32, the expand adds xa @ B^T to the
// row's output window and rounds once to bf16.
//
// Work units (a workgroup of 4 waves each), all shrink units first:
//   shrink unit (tile t, k piece p): every rank row of the tile's adapter over
//     k in [512p, 512p + 512); writes an fp32 partial block part[t][p][16][rr]
//     and raises the piece's flag.
//   expand unit (tile t, column chunk): one to eight 512-column batches of
//     one output window.  It issues its B and y loads, waits for the tile's
//     P flags, sums the P partials in piece order (bitwise reproducible),
//     scales, and adds xa @ B^T to y.
// A consumer only waits on producers with lower workgroup ids, which never
// wait themselves; workgroups are dispatched in id order, so every awaited
// producer is running or done and the wait always ends.  It is still bounded
// and reports a flag instead of spinning forever.
//
// Hand-off without fences.  Every partial is a 64-bit word {fp32 value, tag}
// written and read as one agent-scope atomic, and the tag names the call
// (next_tag of the last completed call's tag on this workspace: the top bit
// set, one more per call).  A reader that sees the current tag therefore sees the
// value, so the producer needs no release (an L2 write-back) and the consumer
// no acquire (an L2 invalidate).  The piece flags carry the same tag and only
// tell the consumer when to start reading; a word that still shows an old tag
// is read again.  The last consumer of a tile counts the tile as finished,
// and the last finished tile of the call records its tag.  Tags grow until
// they start over after 2^31 - 2 calls, so data left by an earlier call, of
// any shape, is never taken for the current one.
//
// The latency chain (tile record -> A/x loads -> reduce -> publish -> poll ->
// partial loads -> expand -> y store) is what bounds a decode-sized call, so
// every wave reads its tile record itself (scalar fields through readlane),
// every unit issues all of its first-pass loads before it waits for any, and
// the x tile is staged once in LDS for all four waves.
//
// Segments with at least mfma_min rows run on v_mfma_f32_16x16x32_bf16
// (tile rows are the MFMA rows; the expand feeds xa as bf16 hi + lo terms,
// hi = bf16(xa), lo = bf16(xa - hi)).  Shorter ones run on the vector ALU:
//   shrink: a wave is 4 DPP rows of 16 lanes; the 16 lanes of a row split the
//     unit's k range (8 k each, 4 steps of 128), each row of lanes owns
//     RPL rank rows, and the 16 per-lane dot products of a (row, rank row)
//     are summed with DPP row moves.
//   expand: a lane owns two adjacent output columns (their B rows are 2R
//     consecutive bf16) and multiplies them by fp32 xa read from LDS with
//     uniform addresses; y is read and written 4 bytes per lane, so a wave's
//     access to one row is 256 contiguous bytes.
#pragma once

#include "common.h"
#include "kernels.h"
#include "ops.h"
#include "slot_meta.h"

#include <algorithm>

namespace tl {

constexpr int kFT = 256;      // threads per workgroup
constexpr int kXS = kKP + 8;  // padded LDS row stride (bf16) of the staged x tile
constexpr int kXaBytes = kTileRows * kMaxRank * 4;  // LDS for a tile's xa (fp32, or bf16 hi/lo pairs)
constexpr int kBStage = 128 * 32 + (128 * 32 / 128) * 8;  // bf16 per wave: 128 columns x 32 ranks + padding
constexpr int kBHalf = 64 * 128;  // bytes per wave: B of 64 columns at rank 64, staged in LDS (wide MFMA expand)
constexpr int kDtStride = 68;  // fp32 row stride of a wave's 16 x 64 output tile in LDS (64 + 4 pad)
constexpr int kSpinLimit = 1 << 22;
constexpr int kShrinkUnits = 1024;  // shrink units a call keeps before its units take several k steps

// ============================================================ tile record, per wave
// Lane i holds word (i mod 32) of the record; the scalar fields are read
// with readlane, so every branch on them is uniform.
struct Hdr {
    int rec;
    int slot, pos0, m, mseg;
};

__device__ __forceinline__ Hdr hdr_of_word(int word) {
    Hdr h;
    h.rec = word;
    h.slot = __builtin_amdgcn_readlane(h.rec, kRecSlot);
    h.pos0 = __builtin_amdgcn_readlane(h.rec, kRecPos);
    h.m = __builtin_amdgcn_readlane(h.rec, kRecRows);
    h.mseg = __builtin_amdgcn_readlane(h.rec, kRecSegRows);
    return h;
}
__device__ __forceinline__ Hdr load_hdr(const int32_t *tiles, int t) {
    return hdr_of_word(tiles[(int64_t)t * kTileWords + (lane_id() & 31)]);
}
// original row id of tile row j; j must be wave-uniform
__device__ __forceinline__ int hdr_row(const Hdr &h, int j) {
    return __builtin_amdgcn_readlane(h.rec, kRecRowIds + j);
}

// ============================================================ shrink units
// Piece 0's unit zeroes its tile's consumer count with an exchange issued
// before the unit's loads, and the count must be zero before the tile's first
// flag is raised.  Using the exchange's result (xo) right after the x tile is
// staged -- where the loads issued after the exchange are awaited anyway --
// makes the wave wait for that exchange there and for nothing else later; in
// particular the flag store does not wait for the unit's partial stores.
__device__ __forceinline__ void exchange_done(int xo) { asm volatile("" : : "v"(xo)); }

// x rows 0..15 (zero past m), k in [k0, k1), into xs[j * kXS + k - k0]: wave w
// loads rows w, w+4, w+8, w+12, one coalesced 1 KB row segment each.
template <class Op>
__device__ __forceinline__ void load_x(const Op &op, const Hdr &h, int k0, int k1, u32x4_t (&xv)[4]) {
    const int lane = lane_id(), w = wave_id();
    const int k = k0 + 8 * lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = w + 4 * u;
        const uint16_t *xp = j < h.m ? op.xrow(hdr_row(h, j)) : nullptr;
        xv[u] = (xp && k < k1) ? (Op::kXOnce ? ld16_stream(xp + k) : ld16(xp + k)) : zero4();
    }
}
__device__ __forceinline__ void store_x(const u32x4_t (&xv)[4], uint16_t *xs) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t *>(xs + (w + 4 * u) * kXS + 8 * lane) = xv[u];
}
__device__ __forceinline__ u32x4_t lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// Vector-ALU shrink of a one-step unit (k1 - k0 <= kKP) into pu[j * n_rr + rr]
// (rr < n_rr, j < m).
// Lane (rl = lane / 16, kl = lane % 16) of wave w holds rank rows
// rb + 4w + rl + 16i (i < RPL) at k = k0 + 128s + 8kl (s < 4).
template <int RPL, class Op>
__device__ __forceinline__ void shrink_valu_1(const Op &op, const Hdr &h, int k0, int k1, uint16_t *xs,
                                            uint64_t *pu, uint32_t tag, int xo) {
    const int lane = lane_id(), w = wave_id();
    const int rl = lane >> 4, kl = lane & 15;
    const int n_rr = op.n_rr(), m = h.m;
    u32x4_t a[RPL][4];
    auto load_a = [&](int rb) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int rr = rb + 4 * w + rl + 16 * i;
            const uint16_t *ap = rr < n_rr ? op.arow(h.slot, rr) : nullptr;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = k0 + 128 * s + 8 * kl;
                a[i][s] = (ap && k < k1) ? ld16_stream(ap + k) : zero4();
            }
        }
    };
    {
        u32x4_t xv[4];
        load_x(op, h, k0, k1, xv);  // x first: the LDS store below waits only for these
        load_a(0);
        store_x(xv, xs);
        __syncthreads();
    }
    exchange_done(xo);
    for (int rb = 0; rb < n_rr; rb += 16 * RPL) {
        if (rb > 0) load_a(rb);
        float sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (4 * b < m) {
                float acc[RPL][4];
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.f;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4_t xv[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) xv[jj] = lds16(xs + (4 * b + jj) * kXS + 128 * s + 8 * kl);
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = dot8(a[i][s], xv[jj], acc[i][jj]);
                }
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = group_sum(acc[i][jj], 4);
                // lane kl keeps value kl = 4i + jj of its row of lanes
                float v = acc[0][0];
#pragma unroll
                for (int q = 1; q < 4 * RPL; ++q) v = kl == q ? acc[q >> 2][q & 3] : v;
                sv[b] = v;
            }
        }
        const int i = kl >> 2, jj = kl & 3;
        const int rr = rb + 4 * w + rl + 16 * i;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = 4 * b + jj;
            if (kl < 4 * RPL && rr < n_rr && j < m) store_word64(pu + j * n_rr + rr, tagged(sv[b], tag));
        }
    }
}

// MFMA shrink of a one-step unit: wave w takes rank-row groups g = w, w+4, ... of 16;
// D[tile row][rank row] = x[16 x 32k] . A^T over 16 steps of 32 k.
template <class Op>
__device__ __forceinline__ void shrink_mfma_1(const Op &op, const Hdr &h, int k0, int k1, uint16_t *xs,
                                            uint64_t *pu, uint32_t tag, int xo) {
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 15, kq = lane >> 4;
    const int n_rr = op.n_rr(), G = (n_rr + 15) >> 4;
    u32x4_t av[16];
    auto load_a = [&](int g) {
        const int rr = 16 * g + col;
        const uint16_t *ap = (g < G && rr < n_rr) ? op.arow(h.slot, rr) : nullptr;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int k = k0 + 32 * s + 8 * kq;
            av[s] = (ap && k < k1) ? ld16_stream(ap + k) : zero4();
        }
    };
    {
        u32x4_t xv[4];
        load_x(op, h, k0, k1, xv);
        load_a(w);
        store_x(xv, xs);
        __syncthreads();
    }
    exchange_done(xo);
    for (int g = w; g < G; g += 4) {
        if (g != w) load_a(g);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        // x fragments read from LDS four steps at a time: with all sixteen
        // hoisted ahead of the MFMAs (64 more registers next to the 64 of A in
        // flight) the kernel would not fit four waves per SIMD
#pragma unroll
        for (int s0 = 0; s0 < 16; s0 += 4) {
            u32x4_t xf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) xf[s] = lds16(xs + col * kXS + 32 * (s0 + s) + 8 * kq);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(xf[s], av[s0 + s], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane holds D[4kq + i][col]: tile rows 4kq..4kq+3 of rank row rr
        const int rr = 16 * g + col;
        if (rr < n_rr) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kq + i < h.m) store_word64(pu + (4 * kq + i) * n_rr + rr, tagged(acc[i], tag));
        }
    }
}

// Vector-ALU shrink of a unit of several k steps: as shrink_valu_1 for each
// step of kKP, x staged once per (rank-row pass, step), and the per-row sums
// of the steps added up before they are stored.
template <int RPL, class Op>
__device__ __forceinline__ void shrink_valu_n(const Op &op, const Hdr &h, int k0, int k1, uint16_t *xs,
                                            uint64_t *pu, uint32_t tag, int xo) {
    const int lane = lane_id(), w = wave_id();
    const int rl = lane >> 4, kl = lane & 15;
    const int n_rr = op.n_rr(), m = h.m;
    u32x4_t a[RPL][4];
    auto load_a = [&](int rb, int ks, int ke) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int rr = rb + 4 * w + rl + 16 * i;
            const uint16_t *ap = rr < n_rr ? op.arow(h.slot, rr) : nullptr;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = ks + 128 * s + 8 * kl;
                a[i][s] = (ap && k < ke) ? ld16_stream(ap + k) : zero4();
            }
        }
    };
    // x of k step [ks, ke) into LDS, with the A of pass rb issued before the barrier
    auto stage = [&](int rb, int ks, int ke, bool reuse) {
        u32x4_t xv[4];
        load_x(op, h, ks, ke, xv);  // x first: the LDS store below waits only for these
        load_a(rb, ks, ke);
        if (reuse) __syncthreads();  // every wave is done with the previous x
        store_x(xv, xs);
        __syncthreads();
    };
    for (int rb = 0; rb < n_rr; rb += 16 * RPL) {
        float sv[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ks = k0; ks < k1; ks += kKP) {
            const int ke = min(k1, ks + kKP);
            stage(rb, ks, ke, rb > 0 || ks > k0);
            exchange_done(xo);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (4 * b < m) {
                    float acc[RPL][4];
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.f;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        u32x4_t xv[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) xv[jj] = lds16(xs + (4 * b + jj) * kXS + 128 * s + 8 * kl);
#pragma unroll
                        for (int i = 0; i < RPL; ++i)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = dot8(a[i][s], xv[jj], acc[i][jj]);
                    }
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = group_sum(acc[i][jj], 4);
                    // lane kl keeps value kl = 4i + jj of its row of lanes
                    float v = acc[0][0];
#pragma unroll
                    for (int q = 1; q < 4 * RPL; ++q) v = kl == q ? acc[q >> 2][q & 3] : v;
                    sv[b] += v;
                }
            }
        }
        const int i = kl >> 2, jj = kl & 3;
        const int rr = rb + 4 * w + rl + 16 * i;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = 4 * b + jj;
            if (kl < 4 * RPL && rr < n_rr && j < m) store_word64(pu + j * n_rr + rr, tagged(sv[b], tag));
        }
    }
}

// MFMA shrink of a unit of several k steps: as shrink_mfma_1 for each step,
// the accumulators kept across the steps;
// D[tile row][rank row] = x[16 x 32k] . A^T over 16 steps of 32 k.
template <class Op>
__device__ __forceinline__ void shrink_mfma_n(const Op &op, const Hdr &h, int k0, int k1, uint16_t *xs,
                                            uint64_t *pu, uint32_t tag, int xo) {
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 15, kq = lane >> 4;
    const int n_rr = op.n_rr(), G = (n_rr + 15) >> 4;
    u32x4_t av[16];
    auto load_a = [&](int g, int ks, int ke) {
        const int rr = 16 * g + col;
        const uint16_t *ap = (g < G && rr < n_rr) ? op.arow(h.slot, rr) : nullptr;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int k = ks + 32 * s + 8 * kq;
            av[s] = (ap && k < ke) ? ld16_stream(ap + k) : zero4();
        }
    };
    auto stage = [&](int g, int ks, int ke, bool reuse) {
        u32x4_t xv[4];
        load_x(op, h, ks, ke, xv);
        load_a(g, ks, ke);
        if (reuse) __syncthreads();  // every wave is done with the previous x
        store_x(xv, xs);
        __syncthreads();
    };
    auto store = [&](int g, const f32x4_t &acc) {
        // lane holds D[4kq + i][col]: tile rows 4kq..4kq+3 of rank row rr
        const int rr = 16 * g + col;
        if (g < G && rr < n_rr) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kq + i < h.m) store_word64(pu + (4 * kq + i) * n_rr + rr, tagged(acc[i], tag));
        }
    };
    // passes of 8 groups of 16 rank rows (two per wave, the same number of
    // passes for every wave); the accumulators live across the steps, and x
    // is staged once per step of a pass
    const int passes = (G + 7) >> 3;
    for (int ps = 0; ps < passes; ++ps) {
        const int g0 = w + 8 * ps, g1 = g0 + 4;
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int ks = k0; ks < k1; ks += kKP) {
            const int ke = min(k1, ks + kKP);
            stage(g0, ks, ke, ps > 0 || ks > k0);
            exchange_done(xo);
            if (g0 < G) {
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc0 = mfma_16x16x32(lds16(xs + col * kXS + 32 * s + 8 * kq), av[s], acc0);
            }
            if (g1 < G) {
                load_a(g1, ks, ke);
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc1 = mfma_16x16x32(lds16(xs + col * kXS + 32 * s + 8 * kq), av[s], acc1);
            }
        }
        store(g0, acc0);
        store(g1, acc1);
    }
}

// MFMA shrink of two consecutive tiles of one segment (tile rows of h0, then
// of h1, staged together), several k steps: each A fragment feeds both
// tiles' MFMAs, so the segment's A is read once for the pair.  Wave w owns
// rank-row groups w and w + 4 (at most 8 groups); the second group's A is
// loaded once the first group's MFMAs have consumed theirs.
template <class Op>
__device__ __forceinline__ void shrink_mfma_pair(const Op &op, const Hdr &h0, const Hdr &h1, int k0, int k1,
                                                 uint16_t *xs, uint64_t *pu0, uint64_t *pu1, uint32_t tag,
                                                 int xo) {
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 15, kq = lane >> 4;
    const int n_rr = op.n_rr(), G = (n_rr + 15) >> 4;
    const int rr0 = 16 * w + col, rr1 = rr0 + 64;
    const uint16_t *ap0 = (w < G && rr0 < n_rr) ? op.arow(h0.slot, rr0) : nullptr;
    const uint16_t *ap1 = (w + 4 < G && rr1 < n_rr) ? op.arow(h0.slot, rr1) : nullptr;
    u32x4_t av[16];
    f32x4_t acc[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
    uint16_t *xs1 = xs + kTileRows * kXS;
    auto load_a = [&](const uint16_t *ap, int ks, int ke) {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            const int k = ks + 32 * s2 + 8 * kq;
            av[s2] = (ap && k < ke) ? ld16_stream(ap + k) : zero4();
        }
    };
    auto mma = [&](f32x4_t (&a)[2]) {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            a[0] = mfma_16x16x32(lds16(xs + col * kXS + 32 * s2 + 8 * kq), av[s2], a[0]);
            a[1] = mfma_16x16x32(lds16(xs1 + col * kXS + 32 * s2 + 8 * kq), av[s2], a[1]);
        }
    };
    for (int ks = k0; ks < k1; ks += kKP) {
        const int ke = min(k1, ks + kKP);
        u32x4_t xv0[4], xv1[4];
        load_x(op, h0, ks, ke, xv0);
        load_x(op, h1, ks, ke, xv1);
        load_a(ap0, ks, ke);
        if (ks > k0) __syncthreads();  // every wave is done with the previous x
        store_x(xv0, xs);
        store_x(xv1, xs1);
        __syncthreads();
        exchange_done(xo);
        if (w < G) mma(acc[0]);
        if (w + 4 < G) {
            load_a(ap1, ks, ke);
            mma(acc[1]);
        }
    }
    // lane holds D[4kq + i][col]: tile rows 4kq..4kq+3 of rank row rr
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int rr = g ? rr1 : rr0;
        if (w + 4 * g < G && rr < n_rr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (4 * kq + i < h0.m) store_word64(pu0 + (4 * kq + i) * n_rr + rr, tagged(acc[g][0][i], tag));
                if (4 * kq + i < h1.m) store_word64(pu1 + (4 * kq + i) * n_rr + rr, tagged(acc[g][1][i], tag));
            }
        }
    }
}

// ============================================================ expand units
// Wait until all but at most one of pieces [0, P) of the tile carry this
// call's tag (wave 0 polls the P <= 63 flags, lane p flag p, with relaxed
// loads); false if a bounded wait gave up.  The staging that follows reads
// every piece's partial words and re-reads a word until it shows the tag, so
// the last piece to finish is awaited on its data: one round trip after it
// lands instead of two (its flag, then its words).  A flag is the word
// {tag, tag}: whatever an earlier call of another layout left at its address
// (a flag, or a partial word {value, older tag}) has an older tag in its
// upper half.
__device__ __forceinline__ bool wait_pieces(const uint64_t *flags, int P, uint32_t tag, int *ctl, int *ok_lds) {
    if (threadIdx.x == 0) *ok_lds = 1;
    if (wave_id() == 0) {
        const int lane = lane_id(), need = P > 1 ? P - 1 : P;
        int spins = 0;
        while (true) {
            const bool done = lane < P && (uint32_t)(load_word64(flags + lane) >> 32) == tag;
            if (__popcll(__ballot(done)) >= need) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                if (lane == 0) {
                    atomicExch(ctl + kCtlError, 1);
                    *ok_lds = 0;
                }
                break;
            }
        }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*ok_lds) != 0;
}

// xa of tile rows j < 16 for the R rank rows of block xb: the P partials
// summed in piece order, times the slot's scale and, with RW, the row's
// weight rw[j] (rows j >= m are zero).
// MF: bf16 hi/lo pairs xl[j][0..R) = hi, xl[j][R..2R) = lo; else fp32 xf[j][R].
// Thread -> (row j, rank r) with r fastest, in Q = 16R / 256 <= QM passes; the
// loads of every pass are issued together, 16 words per thread in flight
// (QM passes x 16/QM pieces per round trip).
template <bool MF, bool RW, int QM>
__device__ __forceinline__ void stage_xa(const uint64_t *pt, int P, int n_rr, int xb, int R, int m, float sc,
                                         const float *rw, uint32_t tag, int *ctl, char *lds) {
    constexpr int PB = 16 / QM;
    const int64_t pstride = (int64_t)n_rr * 16;
    const int n_ent = R * kTileRows;
    const uint64_t *qp[QM];
    bool ok[QM];
    float s[QM];
#pragma unroll
    for (int q = 0; q < QM; ++q) {
        const int idx = threadIdx.x + kFT * q, j = idx / R, r = idx - j * R;
        ok[q] = idx < n_ent && j < m;
        qp[q] = pt + (int64_t)j * n_rr + xb * R + r;
        s[q] = 0.f;
    }
    for (int p0 = 0; p0 < P; p0 += PB) {
        uint64_t v[QM][PB];
#pragma unroll
        for (int q = 0; q < QM; ++q)
#pragma unroll
            for (int u = 0; u < PB; ++u)
                v[q][u] = (ok[q] && p0 + u < P) ? load_word64(qp[q] + (p0 + u) * pstride) : 0;
#pragma unroll
        for (int q = 0; q < QM; ++q)
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                if (ok[q] && p0 + u < P) {
                    // a flag can become visible before the data it announces
                    int spins = 0;
                    while ((uint32_t)(v[q][u] >> 32) != tag && spins++ < kSpinLimit)
                        v[q][u] = load_word64(qp[q] + (p0 + u) * pstride);
                    if ((uint32_t)(v[q][u] >> 32) != tag) atomicExch(ctl + kCtlError, 1);
                    s[q] += __uint_as_float((uint32_t)v[q][u]);
                }
            }
    }
#pragma unroll
    for (int q = 0; q < QM; ++q) {
        const int idx = threadIdx.x + kFT * q, j = idx / R, r = idx - j * R;
        if (idx >= n_ent) continue;
        float x = 0.f;
        if (ok[q]) {
            x = s[q] * sc;
            if (RW) x *= rw[j];
        }
        if (MF) {
            uint16_t *xl = reinterpret_cast<uint16_t *>(lds);
            const float hi = bf16_round(x);
            xl[j * 2 * R + r] = __builtin_bit_cast(uint16_t, (__bf16)hi);
            xl[j * 2 * R + R + r] = __builtin_bit_cast(uint16_t, (__bf16)(x - hi));
        } else {
            reinterpret_cast<float *>(lds)[j * R + r] = x;
        }
    }
}

// stage_xa pass by pass (each pass's pieces in flight together): fewer live
// registers, for the vector-ALU expand, whose prefetch registers are live here.
template <bool MF, bool RW>
__device__ __forceinline__ void stage_xa_passes(const uint64_t *pt, int P, int n_rr, int xb, int R, int m, float sc,
                                         const float *rw, uint32_t tag, int *ctl, char *lds) {
    const int64_t pstride = (int64_t)n_rr * 16;
    // thread -> (row j, rank r) with r fastest: one pass covers 256 / R rows,
    // and a wave's loads of one piece are contiguous words
    for (int idx = threadIdx.x; idx < R * 16; idx += kFT) {
        const int j = idx / R, r = idx - j * R;
        float s = 0.f;
        if (j < m) {
            const uint64_t *q = pt + (int64_t)j * n_rr + xb * R + r;
            for (int p0 = 0; p0 < P; p0 += 8) {
                // eight loads in flight (indices past P repeat piece P - 1 and are not summed)
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = load_word64(q + min(p0 + u, P - 1) * pstride);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (p0 + u < P) {
                        // a flag can become visible before the data it announces
                        int spins = 0;
                        while ((uint32_t)(v[u] >> 32) != tag && spins++ < kSpinLimit)
                            v[u] = load_word64(q + (p0 + u) * pstride);
                        if ((uint32_t)(v[u] >> 32) != tag) atomicExch(ctl + kCtlError, 1);
                        s += __uint_as_float((uint32_t)v[u]);
                    }
                }
            }
            s *= sc;
            if (RW) s *= rw[j];
        }
        if (MF) {
            uint16_t *xl = reinterpret_cast<uint16_t *>(lds);
            const float hi = bf16_round(s);
            xl[j * 2 * R + r] = __builtin_bit_cast(uint16_t, (__bf16)hi);
            xl[j * 2 * R + R + r] = __builtin_bit_cast(uint16_t, (__bf16)(s - hi));
        } else {
            reinterpret_cast<float *>(lds)[j * R + r] = s;
        }
    }
}

// wait_pieces for two tiles at once (threads p < P poll the first tile's
// flags, threads P <= p < 2P the second's).
__device__ __forceinline__ bool wait_pieces2(const uint64_t *f0, const uint64_t *f1, int P, uint32_t tag, int *ctl,
                                             int *ok_lds) {
    if (threadIdx.x == 0) *ok_lds = 1;
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * P; i += kFT) {
        const uint64_t *f = i < P ? f0 + i : f1 + (i - P);
        int spins = 0;
        while ((uint32_t)(load_word64(f) >> 32) != tag) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                atomicExch(ctl + kCtlError, 1);
                *ok_lds = 0;
                break;
            }
        }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*ok_lds) != 0;
}

// What an expand unit needs to find its xa.
struct XaSrc {
    const uint64_t *pt;  // the tile's partial blocks
    const uint64_t *flags;  // the tile's piece flags
    int P, xb;
    bool coalesce_b;     // VALU expand: stage B through LDS with coalesced loads
    float sc;
    uint32_t tag;
    int *ctl;
    int *ok;    // LDS
    float *rw;  // LDS: the tile rows' weights (ops with row weights)
    int *count;  // the tile's finished-consumer count, or null (counted by the caller)
};

// A consumer counts itself at its tile as soon as it holds the tile's xa
// (every unit of the call has read the call's tag by then: see finish), so
// the count's round trip overlaps the unit's expand; the caller takes the
// returned old value at the end.  -1: nothing counted.
__device__ __forceinline__ int count_consumer(const XaSrc &xs) {
    return (xs.count && threadIdx.x == 0) ? atomic_add_relaxed(xs.count, 1) : -1;
}

// Row weights of the tile into xs.rw (wave 0, lanes 0..15); called after the
// unit's B and y loads are issued and before wait_pieces, whose barriers
// publish them to the other waves.
template <class Op>
__device__ __forceinline__ void load_row_weights(const Op &op, const Hdr &h, const XaSrc &xs) {
    if constexpr (Op::kRowWeights) {
        if (wave_id() == 0) {
            const int lane = lane_id();
            const int rid = __shfl(h.rec, kRecRowIds + (lane & 15), kWave);
            if (lane < kTileRows) xs.rw[lane] = lane < h.m ? op.row_weight(rid) : 0.f;
        }
    }
}

// Rows jb .. jb+3 of a vector-ALU expand (jb a compile-time multiple of 4;
// rows past m are computed from row m - 1's xa and not stored): both of the
// lane's columns over all R ranks.  Ranks 0..31 are already in bq; later
// blocks are loaded here, as are ranks 0..31 again for jb > 0 when R > 32.
template <int JB, bool BS, class Op>
__device__ __forceinline__ void valu_rows4(const Op &op, const Hdr &h, int m, int c, bool cok, bool add_inputs,
                                           const uint16_t *bp, int R, u32x4_t (&bq)[2][4],
                                           const uint32_t (&yv)[kTileRows], const float *xf) {
    float o0[4] = {0.f, 0.f, 0.f, 0.f}, o1[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < R; r0 += 32) {
        if (r0 > 0 || (JB > 0 && R > 32)) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bq[cc][q] = (bp && r0 + 8 * q < R) ? ld16_b<BS>(bp + cc * R + r0 + 8 * q) : zero4();
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int rh = r0 + 16 * half;
            if (rh < R) {
                float b0[16], b1[16];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u32x4_t u0 = bq[0][2 * half + q], u1 = bq[1][2 * half + q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b0[8 * q + 2 * e] = bf_lo(u0[e]);
                        b0[8 * q + 2 * e + 1] = bf_hi(u0[e]);
                        b1[8 * q + 2 * e] = bf_lo(u1[e]);
                        b1[8 * q + 2 * e + 1] = bf_hi(u1[e]);
                    }
                }
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    if (rh + 4 * q4 >= R) break;  // R is a multiple of 8, not always of 16
                    f32x4_t xa4[4];              // one batch of uniform-address LDS reads
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xa4[j] = *reinterpret_cast<const f32x4_t *>(xf + min(JB + j, m - 1) * R + rh + 4 * q4);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            o0[j] = __builtin_fmaf(xa4[j][e], b0[4 * q4 + e], o0[j]);
                            o1[j] = __builtin_fmaf(xa4[j][e], b1[4 * q4 + e], o1[j]);
                        }
                }
            }
        }
    }
    if (!cok) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (JB + j < m) {
            float v0 = o0[j], v1 = o1[j];
            if (add_inputs) {
                v0 += bf_lo(yv[JB + j]);
                v1 += bf_hi(yv[JB + j]);
            }
            st4_stream(op.yrow(hdr_row(h, JB + j)) + c, pack_bf16x2(v0, v1));
        }
    }
}

// valu_rows4 for one-batch units at rank 16: the lane's two B rows arrive
// converted to fp32 (once per unit rather than once per block of rows) and
// the block's 16 xa reads (uniform-address LDS reads of 4 ranks of one row)
// are all issued before its FMAs.  The FMAs are those of valu_rows4, in the
// same order, so the two give the same bits.
template <int JB, class Op>
__device__ __forceinline__ void valu_rows4_r16(const Op &op, const Hdr &h, int m, int c, bool cok, bool add_inputs,
                                               const float (&b0)[16], const float (&b1)[16],
                                               const uint32_t (&yv)[kTileRows], const float *xf) {
    float o0[4] = {0.f, 0.f, 0.f, 0.f}, o1[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4_t xa[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[q][j] = *reinterpret_cast<const f32x4_t *>(xf + min(JB + j, m - 1) * 16 + 4 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o0[j] = __builtin_fmaf(xa[q][j][e], b0[4 * q + e], o0[j]);
                o1[j] = __builtin_fmaf(xa[q][j][e], b1[4 * q + e], o1[j]);
            }
    if (!cok) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (JB + j < m) {
            float v0 = o0[j], v1 = o1[j];
            if (add_inputs) {
                v0 += bf_lo(yv[JB + j]);
                v1 += bf_hi(yv[JB + j]);
            }
            st4_stream(op.yrow(hdr_row(h, JB + j)) + c, pack_bf16x2(v0, v1));
        }
    }
}

// Vector-ALU expand of columns [c0, c1) in batches of kEB: in a batch, lane
// owns columns c, c+1 (c = batch start + 128w + 2 lane).  The first batch's B
// and y are loaded before the wait; each later batch's are loaded while the
// previous batch computes.
//
// B in large calls (R <= 32): a wave's 128 columns are 128 * R consecutive
// bf16, read with R / 4 fully coalesced 1 KB instructions (chunk i = lane +
// 64u) and handed to the owning lanes through the wave's LDS stage (16 bytes
// of padding per 256 keep both the writes and the reads free of bank
// conflicts).  Otherwise each lane reads its two B rows directly: 64 lines of
// 16 bytes per instruction cost more L2 requests but no LDS round trip, which
// is what a decode-sized call is short of.
__device__ __forceinline__ int bstage_off(int i) { return i * 8 + (i >> 4) * 8; }  // chunk i -> bf16 offset

template <bool BS, class Op>
__device__ __forceinline__ void valu_load_raw(const Op &op, const Hdr &h, int cw, int c1, int R,
                                              u32x4_t (&raw)[8]) {
    const int lane = lane_id();
    const uint16_t *base = cw < c1 ? op.brow(h.slot, cw) : nullptr;
    const int nl = R >> 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = lane + 64 * u;
        const bool ok = base && u < nl && cw + (i * 8) / R < c1;
        raw[u] = ok ? ld16_b<BS>(base + i * 8) : zero4();
    }
}

__device__ __forceinline__ void valu_transpose(const u32x4_t (&raw)[8], int R, uint16_t *bst,
                                               u32x4_t (&bq)[2][4]) {
    const int lane = lane_id();
    const int nl = R >> 2, cpr = R >> 3;  // loads per wave, 16-byte chunks per B row
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (u < nl) *reinterpret_cast<u32x4_t *>(bst + bstage_off(lane + 64 * u)) = raw[u];
    // the wave reads what its own lanes wrote: LDS operations of a wave complete
    // in order, and the wave barrier keeps the compiler from reordering them
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bq[cc][q] = q < cpr ? *reinterpret_cast<const u32x4_t *>(bst + bstage_off((2 * lane + cc) * cpr + q))
                                : zero4();
    __builtin_amdgcn_wave_barrier();
}

template <bool BS, class Op>
__device__ __forceinline__ void valu_load_b(const Op &op, const Hdr &h, int c, int c1, int R, const uint16_t *&bp,
                                            u32x4_t (&bq)[2][4]) {
    bp = c < c1 ? op.brow(h.slot, c) : nullptr;  // rows c and c+1 are adjacent
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int q = 0; q < 4; ++q) bq[cc][q] = (bp && 8 * q < R) ? ld16_b<BS>(bp + cc * R + 8 * q) : zero4();
}

template <class Op>
__device__ __forceinline__ void valu_load_y(const Op &op, const Hdr &h, int c, int c1, bool add_inputs,
                                            uint32_t (&yv)[kTileRows]) {
#pragma unroll
    for (int j = 0; j < kTileRows; ++j)
        yv[j] = (add_inputs && c < c1 && j < h.m)
                    ? ld4_stream(op.yrow(hdr_row(h, j)) + c)
                    : 0u;
}

// Expand modes (WM): 0, a unit is one batch, and none of the next-batch
// registers exist; 1, units may span several batches, and the vector-ALU
// path loads batch b + 1 while it computes batch b (B coalesced through LDS
// when R <= 32); 2, as 1 but the vector-ALU path loads each batch when it
// starts, which frees the registers (and LDS) of the prefetch for calls
// whose tiles are mostly on the MFMA path.
template <int WM, int NRS, class Op>
__device__ __forceinline__ int expand_valu(const Op &op, const Hdr &h, int c0, int c1, bool add_inputs,
                                           const XaSrc &xs, char *lds) {
    constexpr bool WIDE = WM != 0, PREFETCH = WM == 1;
    constexpr bool BS = WM != 2;  // B streamed unless the call's slots average many rows
    const int lane = lane_id(), w = wave_id();
    const int R = Op::kRank ? Op::kRank : op.R, m = h.m;
    const int nb = WIDE ? (c1 - c0 + kEB - 1) / kEB : 1;
    const bool tr = PREFETCH && xs.coalesce_b && R <= 32;
    const uint16_t *bp = nullptr;
    u32x4_t raw[8], bq[2][4];  // B: coalesced chunks, then ranks 0..31 of the lane's two columns
    uint32_t yv[kTileRows];
    const int cl = 128 * w + 2 * lane;
    if (tr)
        valu_load_raw<BS>(op, h, c0 + 128 * w, c1, R, raw);
    else
        valu_load_b<BS>(op, h, c0 + cl, c1, R, bp, bq);
    valu_load_y(op, h, c0 + cl, c1, add_inputs, yv);
    // the first batch's B reaches its lanes while the producers still run
    uint16_t *bst = reinterpret_cast<uint16_t *>(lds + kXaBytes) + w * kBStage;
    if (tr) valu_transpose(raw, R, bst, bq);
    load_row_weights(op, h, xs);
    if (!wait_pieces(xs.flags, xs.P, xs.tag, xs.ctl, xs.ok)) return count_consumer(xs);
    stage_xa_passes<false, Op::kRowWeights>(xs.pt, xs.P, op.n_rr(), xs.xb, R, m, xs.sc, xs.rw, xs.tag, xs.ctl,
                                            lds);
    __syncthreads();
    const int counted = count_consumer(xs);
    const float *xf = reinterpret_cast<const float *>(lds);
    for (int b = 0; b < nb; ++b) {
        const int c = c0 + kEB * b + cl;
        const bool cok = c < c1;
        if (tr && b > 0) valu_transpose(raw, R, bst, bq);
        if (WIDE && !PREFETCH && b > 0) {
            valu_load_b<BS>(op, h, c, c1, R, bp, bq);
            valu_load_y(op, h, c, c1, add_inputs, yv);
        }
        const uint16_t *bp_n = nullptr;
        u32x4_t bq_n[2][4];
        uint32_t yv_n[kTileRows];
        if (PREFETCH && b + 1 < nb) {
            if (tr)
                valu_load_raw<BS>(op, h, c0 + kEB * (b + 1) + 128 * w, c1, R, raw);
            else
                valu_load_b<BS>(op, h, c + kEB, c1, R, bp_n, bq_n);
            valu_load_y(op, h, c + kEB, c1, add_inputs, yv_n);
        }
        if constexpr (!WIDE) {
            if (R == 16) {
                float b0[16], b1[16];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b0[8 * q + 2 * e] = bf_lo(bq[0][q][e]);
                        b0[8 * q + 2 * e + 1] = bf_hi(bq[0][q][e]);
                        b1[8 * q + 2 * e] = bf_lo(bq[1][q][e]);
                        b1[8 * q + 2 * e + 1] = bf_hi(bq[1][q][e]);
                    }
                if (m > 0) valu_rows4_r16<0>(op, h, m, c, cok, add_inputs, b0, b1, yv, xf);
                if (m > 4) valu_rows4_r16<4>(op, h, m, c, cok, add_inputs, b0, b1, yv, xf);
                if (m > 8) valu_rows4_r16<8>(op, h, m, c, cok, add_inputs, b0, b1, yv, xf);
                if (m > 12) valu_rows4_r16<12>(op, h, m, c, cok, add_inputs, b0, b1, yv, xf);
                continue;  // one batch
            }
        }
        // rows in blocks of 4, no per-row branch inside a block
        if (m > 0) valu_rows4<0, BS>(op, h, m, c, cok, add_inputs, bp, R, bq, yv, xf);
        if (m > 4) valu_rows4<4, BS>(op, h, m, c, cok, add_inputs, bp, R, bq, yv, xf);
        if (m > 8) valu_rows4<8, BS>(op, h, m, c, cok, add_inputs, bp, R, bq, yv, xf);
        if (m > 12) valu_rows4<12, BS>(op, h, m, c, cok, add_inputs, bp, R, bq, yv, xf);
        if (PREFETCH && b + 1 < nb) {
            if (!tr) {
                bp = bp_n;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int q = 0; q < 4; ++q) bq[cc][q] = bq_n[cc][q];
            }
#pragma unroll
            for (int j = 0; j < kTileRows; ++j) yv[j] = yv_n[j];
        }
    }
    return counted;
}

// MFMA expand of columns [c0, c1) in batches of kEB: in a batch, wave w owns
// columns start + 128w .. +128 as 8 tiles of 16;
// D[column][tile row] = B[column][ranks] . (xa_hi + xa_lo)[tile row][ranks]
// as two bf16 MFMAs per 32 ranks (NRS rank steps).  A later batch's B and y
// are loaded once the MFMAs have consumed the previous batch's B.
template <int NRS, bool BS, class Op>
__device__ __forceinline__ void mfma_load_b(const Op &op, const Hdr &h, int cw0, int c1, int R,
                                            u32x4_t (&bo)[8][NRS]) {
    const int lane = lane_id();
    const int col = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        const int cc = cw0 + 16 * ct + col;
        const uint16_t *bp = cc < c1 ? op.brow(h.slot, cc) : nullptr;
#pragma unroll
        for (int s = 0; s < NRS; ++s) {
            const int rk = 32 * s + 8 * kq;
            bo[ct][s] = (bp && rk < R) ? ld16_b<BS>(bp + rk) : zero4();
        }
    }
}
// y of a wave's 16 rows x 128 columns in the row-major order of its stores:
// yv[4hf + j] holds row 4j + lane/16, columns cw0 + 64hf + 4(lane%16) .. +4
// (a row's 64 columns are 16 lanes x 8 contiguous bytes).
__device__ __forceinline__ void mfma_load_y(uint16_t *const (&yr)[4], int cw0, int c1, bool add_inputs,
                                            uint2 (&yv)[8]) {
    const int cl = 4 * (lane_id() & 15);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cy = cw0 + 64 * hf + cl;
            yv[4 * hf + j] = (add_inputs && yr[j] && cy < c1) ? ld8_stream(yr[j] + cy)
                                                              : make_uint2(0u, 0u);
        }
}

// Wide MFMA expand at ranks 33..64 (B rows of up to 128 bytes): B is loaded
// with whole rows per load -- eight lanes per row, so each instruction reads
// eight full cache lines instead of half of sixteen -- and handed to the
// MFMA operand layout through the wave's LDS region, half a batch (64
// columns) at a time.  Row rl of a half keeps its 16-byte chunk c at
// position c ^ ((rl >> 1) & 7), so the operand reads (16 rows, one chunk
// each) spread over the banks.  raw[u]: rows 8 (u mod 8) .. + 8 of half u / 8.
__device__ __forceinline__ int bstage_swz(int rl) { return (rl >> 1) & 7; }
template <bool BS, class Op>
__device__ __forceinline__ void staged_load_b(const Op &op, const Hdr &h, int cb, int c1, int R,
                                              u32x4_t (&raw)[16]) {
    const int lane = lane_id();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int rl = 8 * (u & 7) + (lane >> 3), cc = cb + 64 * (u >> 3) + rl;
        const int j = (lane & 7) ^ bstage_swz(rl);
        const uint16_t *bp = cc < c1 ? op.brow(h.slot, cc) : nullptr;
        raw[u] = (bp && 8 * j < R) ? ld16_b<BS>(bp + 8 * j) : zero4();
    }
}
// half hf of raw into the wave's region: instruction u writes 1 KB in order
__device__ __forceinline__ void staged_put_b(const u32x4_t (&raw)[16], int hf, char *breg) {
    const int lane = lane_id();
#pragma unroll
    for (int u = 0; u < 8; ++u) st16(breg + 1024 * u + 16 * lane, raw[8 * hf + u]);
}
// operand (column tile t, rank step s): lane (kq, col) takes row 16t + col,
// chunk 4s + kq
__device__ __forceinline__ u32x4_t staged_op(const char *breg, int t, int s) {
    const int lane = lane_id(), col = lane & 15, kq = lane >> 4;
    const int rl = 16 * t + col;
    return *reinterpret_cast<const u32x4_t *>(breg + rl * 128 + 16 * ((4 * s + kq) ^ bstage_swz(rl)));
}

template <int NRS, bool WIDE, bool BS, class Op>
__device__ __forceinline__ int expand_mfma(const Op &op, const Hdr &h, int c0, int c1, bool add_inputs,
                                           const XaSrc &xs, char *lds) {
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 15, kq = lane >> 4;
    const int R = Op::kRank ? Op::kRank : op.R;
    const int nb = WIDE ? (c1 - c0 + kEB - 1) / kEB : 1;
    // D comes out as row = col, columns 16ct + 4kq .. +4; y is read and
    // written row-major (rows 4j + lane/16, 8 bytes per lane) and the two
    // meet through a per-wave fp32 tile in LDS
    uint16_t *yr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * j + (lane >> 4);
        const int rid = __shfl(h.rec, kRecRowIds + row, kWave);
        yr[j] = row < h.m ? op.yrow(rid) : nullptr;
    }
    // LB: B staged through LDS (wide calls at ranks 33..64); the wave's
    // region then also holds its output tile, each in turn
    constexpr bool LB = WIDE && NRS == 2;
    char *breg = lds + kXaBytes + w * kBHalf;
    float *dt = LB ? reinterpret_cast<float *>(breg)
                   : reinterpret_cast<float *>(lds + kXaBytes) + w * kTileRows * kDtStride;
    u32x4_t bo[8][NRS];
    u32x4_t raw[LB ? 16 : 1];
    uint2 yv[8];
    if constexpr (LB)
        staged_load_b<BS>(op, h, c0 + 128 * w, c1, R, raw);
    else
        mfma_load_b<NRS, BS>(op, h, c0 + 128 * w, c1, R, bo);
    mfma_load_y(yr, c0 + 128 * w, c1, add_inputs, yv);
    load_row_weights(op, h, xs);
    if (!wait_pieces(xs.flags, xs.P, xs.tag, xs.ctl, xs.ok)) return count_consumer(xs);
    stage_xa<true, Op::kRowWeights, 2 * NRS>(xs.pt, xs.P, op.n_rr(), xs.xb, R, h.m, xs.sc, xs.rw, xs.tag, xs.ctl,
                                             lds);
    __syncthreads();
    const int counted = count_consumer(xs);
    const uint16_t *xl = reinterpret_cast<const uint16_t *>(lds) + col * 2 * R;
    u32x4_t hv[NRS], lv[NRS];
#pragma unroll
    for (int s = 0; s < NRS; ++s) {
        const int rk = 32 * s + 8 * kq;
        hv[s] = rk < R ? lds16(xl + rk) : zero4();
        lv[s] = rk < R ? lds16(xl + R + rk) : zero4();
    }
    for (int b = 0; b < nb; ++b) {
        const int cw0 = c0 + kEB * b + 128 * w;
        uint2 yv_n[8];
        // two halves of four column tiles: each half's MFMAs are issued
        // together, and the second half's overlap the first half's stores
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if constexpr (LB) {
                // this half's B rows into the region (the previous half's
                // output tile has been read back: in-order LDS), its operands
                // out in MFMA layout
                staged_put_b(raw, hf, breg);
                __builtin_amdgcn_wave_barrier();
                if (hf == 1 && b + 1 < nb) staged_load_b<BS>(op, h, cw0 + kEB, c1, R, raw);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int s = 0; s < NRS; ++s) bo[4 * hf + i][s] = staged_op(breg, i, s);
            }
            f32x4_t d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NRS; ++s) {
                    d[i] = mfma_16x16x32(bo[4 * hf + i][s], hv[s], d[i]);
                    d[i] = mfma_16x16x32(bo[4 * hf + i][s], lv[s], d[i]);
                }
            }
            __builtin_amdgcn_wave_barrier();
            if (WIDE && hf == 1 && b + 1 < nb) {
                // the MFMAs above were the last readers of this batch's B
                if constexpr (!LB) mfma_load_b<NRS, BS>(op, h, cw0 + kEB, c1, R, bo);
                mfma_load_y(yr, cw0 + kEB, c1, add_inputs, yv_n);
            }
            // the half's 16 x 64 block through the wave's LDS tile: written in
            // the MFMA layout, read back row-major, added to y, stored
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4_t *>(dt + col * kDtStride + 16 * i + 4 * kq) = d[i];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4_t o = *reinterpret_cast<const f32x4_t *>(dt + (4 * j + (lane >> 4)) * kDtStride +
                                                                    4 * (lane & 15));
                const int cy = cw0 + 64 * hf + 4 * (lane & 15);
                if (yr[j] && cy < c1) {
                    float v[4] = {o[0], o[1], o[2], o[3]};
                    if (add_inputs) {
                        const uint2 yy = yv[4 * hf + j];
                        v[0] += bf_lo(yy.x);
                        v[1] += bf_hi(yy.x);
                        v[2] += bf_lo(yy.y);
                        v[3] += bf_hi(yy.y);
                    }
                    st8_stream(yr[j] + cy, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (WIDE && b + 1 < nb) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) yv[ct] = yv_n[ct];
        }
    }
    return counted;
}

// MFMA expand of two consecutive tiles of one segment (wide calls, ranks up
// to 32): each batch's B feeds the MFMAs of both tiles, so it is read once per
// pair.  xa of the two tiles is staged side by side in LDS and both tiles' y
// of a batch is loaded when the batch starts (the first batch's before the
// wait); each half-batch goes through the wave's LDS tile once per tile.
template <int NRS, class Op>
__device__ __forceinline__ void expand_mfma_pair(const Op &op, const Hdr &h0, const Hdr &h1, int c0, int c1,
                                                 bool add_inputs, const XaSrc &xs0, const XaSrc &xs1, char *lds) {
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 15, kq = lane >> 4;
    const int R = op.R;
    const int nb = (c1 - c0 + kEB - 1) / kEB;
    uint16_t *yr[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * j + (lane >> 4);
        const int rid0 = __shfl(h0.rec, kRecRowIds + row, kWave);
        const int rid1 = __shfl(h1.rec, kRecRowIds + row, kWave);
        yr[0][j] = row < h0.m ? op.yrow(rid0) : nullptr;
        yr[1][j] = row < h1.m ? op.yrow(rid1) : nullptr;
    }
    float *dt = reinterpret_cast<float *>(lds + 2 * kXaBytes) + w * kTileRows * kDtStride;
    u32x4_t bo[8][NRS];
    uint2 yv[2][8];
    mfma_load_b<NRS, false>(op, h0, c0 + 128 * w, c1, R, bo);
    mfma_load_y(yr[0], c0 + 128 * w, c1, add_inputs, yv[0]);
    mfma_load_y(yr[1], c0 + 128 * w, c1, add_inputs, yv[1]);
    load_row_weights(op, h0, xs0);
    load_row_weights(op, h1, xs1);
    if (!wait_pieces2(xs0.flags, xs1.flags, xs0.P, xs0.tag, xs0.ctl, xs0.ok)) return;
    stage_xa<true, Op::kRowWeights, 2 * NRS>(xs0.pt, xs0.P, op.n_rr(), xs0.xb, R, h0.m, xs0.sc, xs0.rw, xs0.tag,
                                             xs0.ctl, lds);
    stage_xa<true, Op::kRowWeights, 2 * NRS>(xs1.pt, xs1.P, op.n_rr(), xs1.xb, R, h1.m, xs1.sc, xs1.rw, xs1.tag,
                                             xs1.ctl, lds + kXaBytes);
    __syncthreads();
    u32x4_t hv[2][NRS], lv[2][NRS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const uint16_t *xl = reinterpret_cast<const uint16_t *>(lds + rt * kXaBytes) + col * 2 * R;
#pragma unroll
        for (int s = 0; s < NRS; ++s) {
            const int rk = 32 * s + 8 * kq;
            hv[rt][s] = rk < R ? lds16(xl + rk) : zero4();
            lv[rt][s] = rk < R ? lds16(xl + R + rk) : zero4();
        }
    }
    for (int b = 0; b < nb; ++b) {
        const int cw0 = c0 + kEB * b + 128 * w;
        if (b > 0) {
            mfma_load_y(yr[0], cw0, c1, add_inputs, yv[0]);
            mfma_load_y(yr[1], cw0, c1, add_inputs, yv[1]);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4_t d[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    d[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NRS; ++s) {
                        d[i] = mfma_16x16x32(bo[4 * hf + i][s], hv[rt][s], d[i]);
                        d[i] = mfma_16x16x32(bo[4 * hf + i][s], lv[rt][s], d[i]);
                    }
                }
                if (hf == 1 && rt == 1 && b + 1 < nb) mfma_load_b<NRS, false>(op, h0, cw0 + kEB, c1, R, bo);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<f32x4_t *>(dt + col * kDtStride + 16 * i + 4 * kq) = d[i];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4_t o = *reinterpret_cast<const f32x4_t *>(dt + (4 * j + (lane >> 4)) * kDtStride +
                                                                        4 * (lane & 15));
                    const int cy = cw0 + 64 * hf + 4 * (lane & 15);
                    if (yr[rt][j] && cy < c1) {
                        float v[4] = {o[0], o[1], o[2], o[3]};
                        if (add_inputs) {
                            const uint2 yy = yv[rt][4 * hf + j];
                            v[0] += bf_lo(yy.x);
                            v[1] += bf_hi(yy.x);
                            v[2] += bf_lo(yy.y);
                            v[3] += bf_hi(yy.y);
                        }
                        st8_stream(yr[rt][j] + cy, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
}

// Expand chunk cc -> output window l and columns [c0, c1) (chunks of EC
// columns, window by window); slice offsets are read at constant indices.
template <class Op>
__device__ __forceinline__ void chunk_of(const Op &op, int cc, int EC, int &l, int &c0, int &c1) {
    int base = 0;
    l = -1;
    c0 = c1 = 0;
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
        if (s < op.n_xs() && l < 0) {
            const int a = op.xoff(s), b = op.xoff(s + 1);
            const int n = (b - a + EC - 1) / EC;
            if (cc < base + n) {
                l = s;
                c0 = a + (cc - base) * EC;
                c1 = min(b, c0 + EC);
            }
            base += n;
        }
    }
}

// ============================================================ unit order
// Workgroup ids: the shrink units first (padded to a multiple of 8), then
// the expand units, then the MoE zero-row units, so every consumer has a
// higher id than the producers it waits on.  Workgroups go to the 8 XCDs
// round robin (id mod 8), and each XCD has its own L2.  Shrink units
// (tile t, piece p), u = t*P + p: with P a multiple of 8, unit u sits at id u,
// so XCD p runs piece p of every tile and each A piece is fetched by one XCD;
// otherwise XCD x runs the contiguous run of units x*U/8 .. (x+1)*U/8 in order
// (U the padded count), so the tiles of one segment, which read the same A,
// run one after another on the same XCD.  Expand units come in blocks of 8 tiles x C chunks; in
// a full block, XCD x runs the C units k = x*C .. x*C + C - 1 of the
// chunk-major order (chunk k / 8 of tile k mod 8), so a chunk's B rows, which
// the 8 tiles of a long segment share, reach at most two L2s instead of all
// eight.
constexpr int kUnitShrink = 0, kUnitExpand = 1, kUnitZero = 2;
constexpr int kXcds = 8;
struct Unit {
    int kind, t, sub;
};
__device__ __forceinline__ int shrink_span(int tile_bound, int P) {
    return (tile_bound * P + kXcds - 1) / kXcds * kXcds;
}
__device__ __forceinline__ Unit unit_of(int bid, int tile_bound, int P, int C) {
    const int nS = shrink_span(tile_bound, P), nE = tile_bound * C;
    if (bid < nS) {
        const int u = (P & (kXcds - 1)) == 0 ? bid : (bid & (kXcds - 1)) * (nS / kXcds) + bid / kXcds;
        return Unit{kUnitShrink, u / P, u - (u / P) * P};
    }
    if (bid >= nS + nE) return Unit{kUnitZero, 0, bid - nS - nE};
    const int e = bid - nS, blk = kXcds * C;
    const int g = e / blk, q = e - g * blk;
    if ((g + 1) * kXcds > tile_bound)  // last, partial block: tile-major
        return Unit{kUnitExpand, g * kXcds + q / C, q % C};
    const int k = (q & (kXcds - 1)) * C + q / kXcds;
    return Unit{kUnitExpand, g * kXcds + (k & (kXcds - 1)), k / kXcds};
}

// ============================================================ kernel
struct FusedArgs {
    const int32_t *tiles;
    const int32_t *counts;  // counts[4] = tiles in use
    int tile_bound, P, C;
    int KS;          // k steps of kKP per shrink unit
    int EC;          // output columns per expand unit (a multiple of kEB)
    uint64_t *part;  // [tile_bound][P][n_rr][16] tagged partials
    int *ctl;        // control line
    uint64_t *flags;  // [tile_bound][kFlagWords]: piece flags, then the tile's finished consumers
    int mfma_min, add_inputs;
    // metadata built in the same launch (Op::kBuild: mode 0, small batches):
    // each unit derives its tile's record from the slot array, and the last
    // workgroup writes the whole metadata to meta_out
    const int32_t *slot;
    int n_rows, n_slots;
    MetaOut meta_out;
};

// Modes 0 and 2 ask for three waves per SIMD: their registers fit without
// spills up to rank 64 (mode 1 holds a second batch's B and y and gets two).
// Mode 0 at a compile-time rank fits four (at most 126 registers), so a
// decode-sized call's units are all resident from the start.
template <int WM, int NRS, class Op>
constexpr int fused_min_waves() {
    return (WM == 0 && Op::kRank != 0) ? 4 : ((WM != 1 && NRS <= 2) ? 3 : 1);
}

template <int RPL, int NRS, int WM, class Op>
__global__ __launch_bounds__(kFT, (fused_min_waves<WM, NRS, Op>())) void fused_kernel(Op op, FusedArgs fa,
                                                                                     ZeroFill zf) {
    // shrink units: the staged x tile; expand units: xa, then the waves' B stages
    constexpr int kLdsShrink = (WM != 0 ? 2 : 1) * kTileRows * kXS * 2;  // wide modes stage tile pairs
    constexpr int kLdsStage = WM == 1 ? 4 * kBStage * 2 : 0, kLdsTile = 4 * kTileRows * kDtStride * 4;
    constexpr int kLdsBStaged = (WM != 0 && NRS == 2) ? 4 * kBHalf : 0;  // B staged per wave, and its output tile
    constexpr int kLdsExpand =  // wide modes at rank <= 32 stage the xa of tile pairs
        (WM != 0 && NRS == 1 ? 2 : 1) * kXaBytes +
        (kLdsStage > kLdsTile ? (kLdsStage > kLdsBStaged ? kLdsStage : kLdsBStaged)
                              : (kLdsTile > kLdsBStaged ? kLdsTile : kLdsBStaged));
    __shared__ __align__(16) char lds[kLdsShrink > kLdsExpand ? kLdsShrink : kLdsExpand];
    static_assert(sizeof(lds) >= (kSmallBallotSlots * (kFT / kWave + 3) + kTileWords + 1) * sizeof(int) +
                                     (kFT / kWave + 1) * sizeof(Int3) + 2 * sizeof(int),
                  "the in-launch metadata build fits the unit LDS");
    __shared__ int ok;
    __shared__ float rw[Op::kRowWeights ? 2 * kTileRows : 1];
    const int P = fa.P, C = fa.C;
    const int n_rr = op.n_rr();
    if (Op::kBuild && blockIdx.x == gridDim.x - 1) {
        // the batch's metadata, as the metadata kernel writes it (no unit of
        // this launch reads it: it is for later calls that reuse it)
        int *sm = reinterpret_cast<int *>(lds);
        Int3 *scan3 = reinterpret_cast<Int3 *>(sm + fa.n_slots * (kFT / kWave + 3));
        small_meta_build<kFT>(SlotSrcDense{fa.slot}, fa.n_rows, fa.n_slots, fa.meta_out, sm, scan3,
                              reinterpret_cast<int *>(scan3 + kFT / kWave + 1));
        return;
    }
    const Unit un = unit_of(blockIdx.x, fa.tile_bound, P, C);
    if (un.kind == kUnitShrink || un.kind == kUnitExpand) {
        const int t = un.t;
        if (t >= fa.tile_bound) return;
        // The last completed call's tag, read with a plain (L2-cached) load:
        // the word changes only at the end of a call, after every unit of it
        // has read the word, and the previous call's value reaches this launch
        // through the stream's kernel boundary.  An agent-scope load here, one
        // per wave of every unit, would pass the L2 and queue thousands of
        // requests on one address ahead of the unit's own loads (no reuse:
        // 155 -> 148 us).
        const uint32_t tag = next_tag((uint32_t)fa.ctl[kCtlGen]);
        int slot_tiles = 0;
        int slot_word = 0;
        if constexpr (Op::kBuild)
            slot_word = slot_tile_record(fa.slot, fa.n_rows, fa.n_slots, t, reinterpret_cast<int *>(lds), slot_tiles);
        auto tile_hdr = [&]() { return Op::kBuild ? hdr_of_word(slot_word) : load_hdr(fa.tiles, t); };
        if (un.kind == kUnitShrink) {
            const int p = un.sub;
            const Hdr h = tile_hdr();
            if (h.m == 0) return;
            const int k0p = (p * fa.KS) * kKP, k1p = min(op.k_in, k0p + fa.KS * kKP);
            // wide calls: MFMA segments with at most 128 rank rows are shrunk two
            // tiles at a time, by the unit of the pair's first tile (the tile
            // with an even index within its segment); the second tile's unit
            // has nothing to do
            if (WM != 0 && h.mseg >= fa.mfma_min && n_rr <= 128) {
                const int jt = __builtin_amdgcn_readlane(h.rec, kRecSegTile);
                // (segments under 16 rows, cut in two tiles, are never paired)
                if ((jt & 1) && h.mseg >= kTileRows) return;
                if (!(jt & 1) && h.mseg > kTileRows * (jt + 1)) {
                    const Hdr h1 = load_hdr(fa.tiles, t + 1);
                    uint64_t *fl0 = fa.flags + (int64_t)t * kFlagWords, *fl1 = fl0 + kFlagWords;
                    int old = 0;
                    if (p == 0 && threadIdx.x < 2)
                        old = xchg_relaxed(reinterpret_cast<int *>((threadIdx.x == 0 ? fl0 : fl1) + kFlagWords - 1), 0);
                    shrink_mfma_pair(op, h, h1, k0p, k1p, reinterpret_cast<uint16_t *>(lds),
                                     fa.part + ((int64_t)t * P + p) * n_rr * 16,
                                     fa.part + ((int64_t)(t + 1) * P + p) * n_rr * 16, tag, old);
                    __syncthreads();
                    if (threadIdx.x < 2)  // (the exchanges have returned: exchange_done)
                        store_word64((threadIdx.x == 0 ? fl0 : fl1) + p, ((uint64_t)tag << 32) | tag);
                    return;
                }
            }
            uint64_t *fl = fa.flags + (int64_t)t * kFlagWords;
            // piece 0 zeroes the tile's consumer count (whatever an earlier
            // call left there); the exchange returns before its flag and its
            // partials are stored, and every consumer counts only after seeing
            // one of them
            int old = 0;
            if (p == 0 && threadIdx.x == 0) old = xchg_relaxed(reinterpret_cast<int *>(fl + kFlagWords - 1), 0);
            // (k0 written as a multiple of kKP: the loads' addressing depends on it)
            const int k0 = (p * fa.KS) * kKP, k1 = min(op.k_in, k0 + fa.KS * kKP);
            uint64_t *pu = fa.part + ((int64_t)t * P + p) * n_rr * 16;
            uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
            // units of several k steps exist only in the wide modes
            if (h.mseg >= fa.mfma_min) {
                if (WM != 0 && fa.KS > 1)
                    shrink_mfma_n(op, h, k0, k1, xs, pu, tag, old);
                else
                    shrink_mfma_1(op, h, k0, k1, xs, pu, tag, old);
            } else {
                if (WM != 0 && fa.KS > 1)
                    shrink_valu_n<RPL>(op, h, k0, k1, xs, pu, tag, old);
                else
                    shrink_valu_1<RPL>(op, h, k0, k1, xs, pu, tag, old);
            }
            // raise the flag after every wave has issued its stores (the tags,
            // not this order, are what make the hand-off correct); the stores
            // are not awaited: a consumer that sees the flag before a partial
            // word re-reads that word until its tag is the call's.  The
            // exchange has returned (exchange_done).
            __syncthreads();
            if (threadIdx.x == 0) store_word64(fl + p, ((uint64_t)tag << 32) | tag);
            return;
        }
        const int cc = un.sub;
        const int n_tiles = Op::kBuild ? slot_tiles : fa.counts[4];
        const Hdr h = tile_hdr();
        if (h.m == 0) return;
        int l, c0, c1;
        chunk_of(op, cc, fa.EC, l, c0, c1);
        // the last consumer of a tile counts the tile as finished; the last
        // finished tile of the call stores the call's tag as the last one
        // (two levels, so no single address takes one atomic per consumer).
        // A consumer counts once it holds its tile's xa: every unit of the
        // call has read the call's tag by then (each consumer at its start,
        // each producer before raising the flags its consumers waited for),
        // so the next call can take the next tag; what the unit still does
        // (its expand, its stores) is ordered before the next call by the
        // stream.
        int *tile_done = reinterpret_cast<int *>(fa.flags + (int64_t)t * kFlagWords + kFlagWords - 1);
        auto tile_finished = [&]() {
            if (atomic_add_relaxed(fa.ctl + kCtlDone, 1) == n_tiles - 1) {
                store_relaxed(fa.ctl + kCtlDone, 0);
                store_relaxed(fa.ctl + kCtlGen, (int)tag);
            }
        };
        auto finish = [&](int tt) {
            int *td = reinterpret_cast<int *>(fa.flags + (int64_t)tt * kFlagWords + kFlagWords - 1);
            if (atomic_add_relaxed(td, 1) == C - 1) tile_finished();
        };
        // wide calls: MFMA segments of rank <= 32 are expanded two tiles at a
        // time by the units of the pair's first tile, which count both tiles
        // (at rank 64 the second tile's registers would spill)
        if (WM != 0 && NRS == 1 && h.mseg >= fa.mfma_min) {
            const int jt = __builtin_amdgcn_readlane(h.rec, kRecSegTile);
            if ((jt & 1) && h.mseg >= kTileRows) return;
            if (!(jt & 1) && h.mseg > kTileRows * (jt + 1)) {
                const Hdr h1 = load_hdr(fa.tiles, t + 1);
                const float sc = op.scale_of(h.slot);
                const XaSrc xs0{fa.part + (int64_t)t * P * n_rr * 16, fa.flags + (int64_t)t * kFlagWords, P,
                                op.xblk(l), true, sc, tag, fa.ctl, &ok, rw, nullptr};
                const XaSrc xs1{fa.part + (int64_t)(t + 1) * P * n_rr * 16, fa.flags + (int64_t)(t + 1) * kFlagWords,
                                P, op.xblk(l), true, sc, tag, fa.ctl, &ok, rw + kTileRows, nullptr};
                expand_mfma_pair<NRS>(op, h, h1, c0, c1, fa.add_inputs != 0, xs0, xs1, lds);
                if (threadIdx.x == 0) {
                    finish(t);
                    finish(t + 1);
                }
                return;
            }
        }
        const XaSrc xs{fa.part + (int64_t)t * P * n_rr * 16, fa.flags + (int64_t)t * kFlagWords, P, op.xblk(l),
                       fa.EC > kEB, op.scale_of(h.slot), tag, fa.ctl, &ok, rw, tile_done};
        const int counted = h.mseg >= fa.mfma_min
                                ? expand_mfma<NRS, WM != 0, WM != 2>(op, h, c0, c1, fa.add_inputs != 0, xs, lds)
                                : expand_valu<WM, NRS>(op, h, c0, c1, fa.add_inputs != 0, xs, lds);
        if (threadIdx.x == 0 && counted == C - 1) tile_finished();
        return;
    }
    // zero rows of pairs that get no delta (MoE only)
    const int u = un.sub;
    const int tid = threadIdx.x;
    const int pair = u * 16 + (tid >> 4);
    if (pair >= zf.n_pairs) return;
    const int l = zf.lora[pair / zf.top_k], ex = zf.topk[pair];
    if (l >= 0 && l < zf.L && ex >= 0 && ex < zf.E) return;
    uint16_t *o = op.yrow(pair);
    for (int c = (tid & 15) * 8; c < op.n_out; c += 128) st16_stream(o + c, zero4());
}

// ============================================================ host side
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }


static int rpl_of(int n_rr) { return n_rr >= 64 ? 4 : (n_rr + 15) / 16; }
static int nrs_of(int R) { return R <= 32 ? 1 : (R <= 64 ? 2 : 4); }

template <int RPL, int NRS, class Op>
static hipError_t launch_fused_t(const Op &op, const FusedArgs &fa, bool mfma_lean, long long grid, ZeroFill zf,
                                 hipStream_t st) {
    const dim3 g((unsigned)grid), b(kFT);
    if constexpr (Op::kRank != 0 || Op::kBuild) {
        // compile-time ranks and in-launch metadata serve mode 0 only (the
        // callers check narrow_call)
        hipLaunchKernelGGL((fused_kernel<RPL, NRS, 0, Op>), g, b, 0, st, op, fa, zf);
    } else {
        if (fa.EC <= kEB && fa.KS == 1)
            hipLaunchKernelGGL((fused_kernel<RPL, NRS, 0, Op>), g, b, 0, st, op, fa, zf);
        else if (!mfma_lean)
            hipLaunchKernelGGL((fused_kernel<RPL, NRS, 1, Op>), g, b, 0, st, op, fa, zf);
        else
            hipLaunchKernelGGL((fused_kernel<RPL, NRS, 2, Op>), g, b, 0, st, op, fa, zf);
    }
    return hipGetLastError();
}

template <int RPL, class Op>
static hipError_t launch_fused_r(const Op &op, const FusedArgs &fa, bool mfma_lean, long long grid, ZeroFill zf,
                                 hipStream_t st) {
    if constexpr (Op::kRank != 0) {
        return launch_fused_t<RPL, (Op::kRank <= 32 ? 1 : (Op::kRank <= 64 ? 2 : 4))>(op, fa, mfma_lean, grid, zf,
                                                                                     st);
    } else {
        switch (nrs_of(op.R)) {
        case 1: return launch_fused_t<RPL, 1>(op, fa, mfma_lean, grid, zf, st);
        case 2: return launch_fused_t<RPL, 2>(op, fa, mfma_lean, grid, zf, st);
        default: return launch_fused_t<RPL, 4>(op, fa, mfma_lean, grid, zf, st);
        }
    }
}

// mfma_lean: the call averages at least mfma_min rows per slot, so most of
// its tiles are expected on the MFMA path (selects expand mode 2 over 1).
// In-launch metadata (FusedArgs::slot): the slot array, its shape and the
// caller's metadata arrays; null: the tile records come from tiles.
struct SlotBuild {
    const int32_t *slot;
    int n, S;
    MetaOut out;
};

template <class Op>
static hipError_t launch_fused_op(const Op &op, const int32_t *tiles, const int32_t *counts, const FusedPlan &plan,
                                  int C, int EC, void *ws, int *ctl, int mfma_min, bool mfma_lean,
                                  int add_inputs, ZeroFill zf, int zero_units, hipStream_t st,
                                  const SlotBuild *sb = nullptr) {
    char *w = static_cast<char *>(ws);
    FusedArgs fa{};
    fa.tiles = tiles;
    fa.counts = counts;
    fa.tile_bound = plan.tile_bound;
    // k steps per shrink unit: one while the call has few tiles (decode: its
    // latency wants every piece in flight at once); wide calls give each unit
    // several steps so that about kShrinkUnits units remain; and at most
    // kFlagWords - 1 pieces fit a tile's flag block
    const int steps = (op.k_in + kKP - 1) / kKP;
    int ks = 1;
    if (EC > kEB && plan.tile_bound > 0) {
        const int pieces = std::min(steps, std::max(1, (kShrinkUnits + plan.tile_bound - 1) / plan.tile_bound));
        ks = (steps + pieces - 1) / pieces;
    }
    ks = std::max(ks, (steps + kFlagWords - 2) / (kFlagWords - 1));
    fa.KS = ks;
    fa.P = (steps + ks - 1) / ks;
    fa.C = C;
    fa.EC = EC;
    fa.ctl = ctl;
    fa.flags = reinterpret_cast<uint64_t *>(w + 256);
    fa.part = reinterpret_cast<uint64_t *>(w + plan.flag_bytes);
    fa.mfma_min = mfma_min;
    fa.add_inputs = add_inputs;
    // every shrink unit ahead of every expand unit.  (Interleaving groups of
    // producers and consumers measured slower on the large configs: consumers
    // that start before their producers hold workgroup slots.)
    const long long n_shrink = ((long long)plan.tile_bound * fa.P + kXcds - 1) / kXcds * kXcds;
    long long grid = plan.tile_bound > 0 ? n_shrink + (long long)plan.tile_bound * C + zero_units : zero_units;
    if ((sb != nullptr) != Op::kBuild) return hipErrorInvalidValue;
    if (sb) {  // one more workgroup, the last, writes the metadata
        if (EC > kEB || fa.KS != 1) return hipErrorInvalidValue;  // mode 0 only
        fa.slot = sb->slot;
        fa.n_rows = sb->n;
        fa.n_slots = sb->S;
        fa.meta_out = sb->out;
        grid += 1;
    }
    if (grid == 0) return hipSuccess;
    switch (rpl_of(op.n_sh * op.R)) {
    case 1: return launch_fused_r<1>(op, fa, mfma_lean, grid, zf, st);
    case 2: return launch_fused_r<2>(op, fa, mfma_lean, grid, zf, st);
    case 3: return launch_fused_r<3>(op, fa, mfma_lean, grid, zf, st);
    default: return launch_fused_r<4>(op, fa, mfma_lean, grid, zf, st);
    }
}

}  // namespace tl
