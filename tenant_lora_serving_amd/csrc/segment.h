// segment.h -- the routed-MoE LoRA deltas with one workgroup per segment
// group, for gfx950: shrink and expand of up to 64 pairs of one (adapter,
// expert) segment in the same workgroup, with no hand-off between
// workgroups.
//
// Semantics: for every routed pair (t, j) with adapter l and expert e,
//  gemm1 (FlashInfer bgmv_moe_gemm1_lora_delta, description and parameters):
//   out[t][j] = scale * concat(B_gate (A_gate x[t]), B_up (A_up x[t]))
//   (shared-A form: scale * B_fused (A x[t]));
//  w2 (vLLM punica_base.py, add_lora_w2): y[p] += w[p] * scale * B (A x2[p]),
//   p = t * top_k + j, w the router weight (or 1).
// Pairs are grouped into segments of one (l, e) by the pair metadata.
//
// A segment of the MoE workloads holds a few tens of pairs, so the whole
// segment fits one workgroup: unit u takes the first 64 pairs of segment u
// of the pair metadata (sorted_rows[seg_offsets[u] ..]).  Consecutive units,
// which the hardware hands to the 8 XCDs in turn, are segments of similar
// size, so every XCD gets its share.  A longer segment's further groups of 64
// pairs are taken by the units launched after those, one per tile record: the
// unit of a tile that starts such a group (index 4, 8, ... in its segment)
// takes that group; every other tile unit returns at once.  In the unit:
//   shrink  wave w owns tile w's 16 rows (the MFMA M dimension) and every
//           rank group of 16 rank rows; k runs in stages of 256 with two
//           stages of loads in flight in registers: the stage's gathered x
//           rows and A rows, each loaded coalesced (32 threads per 512-byte
//           row slice; a load in the MFMA operand layout would touch 16 rows,
//           so 16 half-used cache lines, per 16 lanes) and handed to the
//           waves through a padded LDS stage.
//   xa      scale * the fp32 accumulators, split into bf16 hi + lo terms in
//           LDS (the bf16 MFMA sees hi + lo = xa to 2^-16 relative).
//   expand  the 2I output columns in chunks of 64 (four 16-column MFMA
//           tiles), chunk q on wave q mod 4, B rows read directly in the
//           operand layout one chunk ahead; each chunk's 16 x 64 block per
//           tile goes through the wave's LDS tile so that out rows are
//           written 128 contiguous bytes at a time (w2: y rows are read
//           the same way, their loads issued before the chunk's MFMAs).
// Ranks up to 16 fit hi and lo in one 32-wide MFMA k block (lanes of k
// quarters 0 .. R/8 - 1 carry hi, the next R/8 quarters lo, and the B
// operand repeats its R ranks); rank 32 takes two MFMAs (hi, then lo).
// Pairs without a valid (adapter, expert) get zero rows from the zero units
// after the tile units.
#pragma once

#include "common.h"
#include "kernels.h"
#include "ops.h"

namespace tl {

constexpr int kSegTiles = 4;              // tiles (of 16 pairs) per segment unit
constexpr int kSegK = 256;                // k per pipeline stage
constexpr int kSegAStride = kSegK * 2 + 16;  // bytes per staged A row (padded: conflict-free operand reads)
constexpr int kSegDt = 68;                // fp32 row stride of a wave's 16 x 64 output tile

struct SegArgs {
    const int32_t *tiles;
    int tile_bound;
    const int32_t *sorted_rows;
    const int32_t *seg_offsets;
    const int32_t *seg_slot;
    const int32_t *counts;  // counts[1]: segments
    int n_units;            // units before the zero units: the most segments the call can have
    int n_rows;             // pairs of the call (the metadata's n)
    int *ctl;               // the workspace's control line (its call tag is advanced)
    int key_div;            // > 0: segment units grouped by adapter (key / key_div) on XCDs; 0: in order
};

// Segment units by adapter.  A token's x row is read by the segments of its
// top_k experts, all of its own adapter l (keys l*E .. l*E + E-1), so when one
// XCD runs all of adapter l's segments the row is fetched from HBM once for
// that XCD's L2 instead of once per segment.  Workgroups go to the 8 XCDs
// round robin: unit u runs on XCD x = u mod 8 and takes the (u / 8)-th segment
// of class x (segments whose adapter is x mod 8, in segment order).  A class
// with more segments than its XCD has units passes the rest, in class order,
// to the units left without a segment, also in class order.  Returns the
// unit's segment (sg -1: none) with its sorted pairs [start, end) and key.
// The segment count and every segment's key and offsets are loaded at once
// (entries past the count, left by earlier calls, are read and ignored: the
// arrays hold n_units entries), so the unit knows its pairs one round trip
// after it starts.  sm: 4 * 8 * (kSegMapMax / 256) + 40 ints of LDS.
constexpr int kSegMapMax = 1024;  // most units the mapping takes (else units run in segment order)
struct SegPick {
    int sg, start, end, slot;
};
__device__ __forceinline__ SegPick unit_segment(const SegArgs &sa, int u, int *sm) {
    constexpr int Q = kSegMapMax / 256, NC = 8;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    int *cnt = sm;                   // [Q][4 waves][NC] segments of each class, then their first class rank
    int *tot = cnt + Q * 4 * NC;     // [NC] segments per class
    int *found = tot + NC;           // the unit's segment, its first and end pair, its key
    const int n_seg = __builtin_amdgcn_readfirstlane(sa.counts[1]);
    int key[Q], off0[Q], off1[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int sg = tid + 256 * q;
        const bool in = sg < sa.n_units;
        key[q] = in ? sa.seg_slot[sg] : 0;
        off0[q] = in ? sa.seg_offsets[sg] : 0;
        off1[q] = in ? sa.seg_offsets[sg + 1] : 0;
    }
    int cls[Q], rank[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) cls[q] = tid + 256 * q < n_seg ? (key[q] / sa.key_div) & (NC - 1) : -1;
    if (tid == 0) found[0] = -1;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        rank[q] = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint64_t b = __ballot(cls[q] == c);
            if (cls[q] == c) rank[q] = __popcll(b & lanemask_lt());
            if (lane == c) cnt[(q * 4 + w) * NC + c] = __popcll(b);
        }
    }
    __syncthreads();
    if (tid < NC) {  // exclusive prefix over (q, wave) blocks, in segment order, per class
        int run = 0;
        for (int i = 0; i < Q * 4; ++i) {
            const int v = cnt[i * NC + tid];
            cnt[i * NC + tid] = run;
            run += v;
        }
        tot[tid] = run;
    }
    __syncthreads();
    // the unit's (class, rank): its own class's, or an overflow one
    const int x = u & (NC - 1), i = u / NC;
    auto cap = [&](int c) { return c < sa.n_units ? (sa.n_units - c + NC - 1) / NC : 0; };
    int tc = -1, tr = -1;
    if (i < tot[x]) {
        tc = x;
        tr = i;
    } else {
        int k = i - tot[x];
        for (int c = 0; c < x; ++c) k += max(0, cap(c) - tot[c]);
        for (int c = 0; c < NC && tc < 0; ++c) {
            const int over = max(0, tot[c] - cap(c));
            if (k < over) {
                tc = c;
                tr = cap(c) + k;
            } else {
                k -= over;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (cls[q] >= 0 && cls[q] == tc && cnt[(q * 4 + w) * NC + cls[q]] + rank[q] == tr) {
            found[0] = tid + 256 * q;
            found[1] = off0[q];
            found[2] = off1[q];
            found[3] = key[q];
        }
    __syncthreads();
    SegPick pk;
    pk.sg = __builtin_amdgcn_readfirstlane(found[0]);
    pk.start = __builtin_amdgcn_readfirstlane(found[1]);
    pk.end = __builtin_amdgcn_readfirstlane(found[2]);
    pk.slot = __builtin_amdgcn_readfirstlane(found[3]);
    __syncthreads();  // (the unit's LDS stages reuse these words)
    return pk;
}

// bytes of a row of the LDS xa block: for each of nx blocks, hi[R] then lo[R] (bf16), + 16 pad
__host__ __device__ constexpr int seg_xa_stride(int nx, int R) { return nx * 4 * R + 16; }

template <int G, int RK>
constexpr int seg_lds_bytes() {
    constexpr int shrink = (64 + 16 * G) * kSegAStride;  // one stage of x rows and A rows
    constexpr int expand = kSegTiles * 16 * seg_xa_stride(2, RK) + 4 * 16 * kSegDt * 4;
    return shrink > expand ? shrink : expand;
}

// G: rank groups of 16 rank rows (n_rr <= 16 G); RK: the rank (8, 16 or 32).
template <int G, int RK, class Op>
__global__ __launch_bounds__(256, 2) void segment_kernel(Op op, SegArgs sa, ZeroFill zf) {
    static_assert(RK == 8 || RK == 16 || RK == 32, "segment units take ranks 8, 16 and 32");
    __shared__ __align__(16) char lds[seg_lds_bytes<G, RK>()];
    const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
    const int c = lane & 15, kq = lane >> 4;

    if ((int)blockIdx.x >= sa.n_units + sa.tile_bound) {
        // zero rows of pairs that get no delta
        const int pair = ((int)blockIdx.x - sa.n_units - sa.tile_bound) * 16 + (tid >> 4);
        if (pair >= zf.n_pairs) return;
        const int l = zf.lora[pair / zf.top_k], ex = zf.topk[pair];
        if (l >= 0 && l < zf.L && ex >= 0 && ex < zf.E) return;
        uint16_t *o = op.yrow(pair);
        for (int cc = (tid & 15) * 8; cc < op.n_out; cc += 128) st16_stream(o + cc, zero4());
        return;
    }
    if (blockIdx.x == 0 && tid == 0)  // the call's tag, for later calls that share the workspace
        store_relaxed(sa.ctl + kCtlGen, (int)next_tag((uint32_t)load_relaxed(sa.ctl + kCtlGen)));

    // ---- the unit's group: key, first sorted position, pairs
    const int u = blockIdx.x;
    int slot, g_start, mg;
    if (u < sa.n_units) {
        if (sa.key_div > 0 && sa.n_units <= kSegMapMax) {
            const SegPick pk = unit_segment(sa, u, reinterpret_cast<int *>(lds));
            if (pk.sg < 0) return;
            g_start = pk.start;
            mg = min(kSegTiles * 16, pk.end - pk.start);
            slot = pk.slot;
        } else {
            const int n_seg = __builtin_amdgcn_readfirstlane(sa.counts[1]);
            if (u >= n_seg) return;
            g_start = __builtin_amdgcn_readfirstlane(sa.seg_offsets[u]);
            mg = min(kSegTiles * 16, __builtin_amdgcn_readfirstlane(sa.seg_offsets[u + 1]) - g_start);
            slot = __builtin_amdgcn_readfirstlane(sa.seg_slot[u]);
        }
    } else {
        const int rec = sa.tiles[(int64_t)(u - sa.n_units) * kTileWords + (lane & 31)];
        const int jt = __builtin_amdgcn_readlane(rec, kRecSegTile);
        if (__builtin_amdgcn_readlane(rec, kRecRows) == 0 || jt == 0 || jt % kSegTiles) return;
        // (such a segment is longer than 64 pairs, so its tiles hold 16 pairs each)
        slot = __builtin_amdgcn_readlane(rec, kRecSlot);
        g_start = __builtin_amdgcn_readlane(rec, kRecPos);
        mg = min(kSegTiles * 16, __builtin_amdgcn_readlane(rec, kRecSegRows) - 16 * jt);
    }
    const int K = op.k_in, n_rr = op.n_rr();
    const auto bs = op.bases(slot);
    const rsrc_t rx = op.x_rsrc(sa.n_rows), ra0 = op.a_rsrc(bs, 0), ra1 = op.a_rsrc(bs, 1);
    const int NS = (K + kSegK - 1) / kSegK;
    const int nt = (mg + 15) / 16;  // the group's tiles of 16 pairs
    // pair ids: lane holds row (lane & 15) of each tile
    int pid[kSegTiles];
#pragma unroll
    for (int i = 0; i < kSegTiles; ++i) {
        const int j = 16 * i + c;
        pid[i] = j < mg ? sa.sorted_rows[g_start + j] : 0;
    }
    int mt[kSegTiles];
#pragma unroll
    for (int i = 0; i < kSegTiles; ++i) mt[i] = min(16, max(0, mg - 16 * i));
    // ---- shrink.  Stage s covers k in [256 s, 256 s + 256): its x rows (64
    // at most, 512 bytes each) and its 16 G A rows are loaded coalesced, 32
    // threads per row, two stages ahead into registers; each stage is written
    // to the LDS stage (padded rows: the operand reads are free of bank
    // conflicts) and every wave takes its MFMA operands from there.
    constexpr int AQ = 2 * G;  // 16-byte A chunks per thread per stage (16 G rows x 512 bytes)
    constexpr int XQ = 8;      // 16-byte x chunks per thread per stage (64 rows x 512 bytes)
    char *xbuf = lds, *abuf = lds + 64 * kSegAStride;
    // byte offset of this thread's x row of chunk i (row (tid >> 5) + 8 i), or past the buffer
    uint32_t xo[XQ];
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
        const int row = (tid >> 5) + 8 * i;
        xo[i] = row < mg ? op.x_off(sa.sorted_rows[g_start + row], 0) : kOob;
    }
    u32x4_t xr[2][XQ], ar[2][AQ];
    f32x4_t acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int s, u32x4_t (&xv)[XQ], u32x4_t (&av)[AQ]) {
        const int k = s * kSegK + 8 * (tid & 31);
        const bool kok = k < K;
#pragma unroll
        for (int i = 0; i < XQ; ++i) xv[i] = buf_ld16<Op::kXOnce ? kNt : 0>(rx, kok ? xo[i] + 2 * k : kOob);
        // thread chunk i covers rank rows 8i .. 8i + 7 (one slice: R is a multiple of 8)
#pragma unroll
        for (int i = 0; i < AQ; ++i) {
            const int row = (tid >> 5) + 8 * i;
            const int sg = (8 * i) / RK;
            av[i] = buf_ld16<kNt>(sg == 0 ? ra0 : ra1, (row < n_rr && kok) ? op.a_off(row - sg * RK, k) : kOob);
        }
    };
    auto stage = [&](const u32x4_t (&xv)[XQ], const u32x4_t (&av)[AQ]) {
        __syncthreads();  // every wave has computed the previous stage
        const int off = (tid >> 5) * kSegAStride + 16 * (tid & 31);
#pragma unroll
        for (int i = 0; i < XQ; ++i) st16(xbuf + off + 8 * i * kSegAStride, xv[i]);
#pragma unroll
        for (int i = 0; i < AQ; ++i) st16(abuf + off + 8 * i * kSegAStride, av[i]);
        __syncthreads();
    };
    auto compute = [&]() {
        if (w < nt) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4_t xf = ld16(xbuf + (16 * w + c) * kSegAStride + 64 * ks + 16 * kq);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g] = mfma_16x16x32(xf, ld16(abuf + (16 * g + c) * kSegAStride + 64 * ks + 16 * kq), acc[g]);
            }
        }
    };
    // stage s lives in register slot s % 2 until it is written to LDS; the
    // loads of stage s + 2 then refill that slot while stage s computes
    issue(0, xr[0], ar[0]);
    if (NS > 1) issue(1, xr[1], ar[1]);
    for (int s = 0; s < NS; s += 2) {
        stage(xr[0], ar[0]);
        if (s + 2 < NS) issue(s + 2, xr[0], ar[0]);
        compute();
        if (s + 1 < NS) {
            stage(xr[1], ar[1]);
            if (s + 3 < NS) issue(s + 3, xr[1], ar[1]);
            compute();
        }
    }

    // ---- xa = scale * acc as bf16 hi + lo, [row][block][hi R | lo R]
    constexpr int NX = 2;  // blocks of the LDS row (the shared form uses one)
    constexpr int XS = seg_xa_stride(NX, RK);
    __syncthreads();  // every wave is done with the A buffers, which xa and the tiles reuse
    const float sc = op.scale_of(slot);
    if (w < nt) {
        // router weights of the wave's rows 4 kq + i (w2)
        float rw[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (Op::kRowWeights) {
            int mypid = pid[0];
#pragma unroll
            for (int i = 1; i < kSegTiles; ++i) mypid = w == i ? pid[i] : mypid;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pr = __shfl(mypid, 4 * kq + i, kWave);
                rw[i] = 16 * w + 4 * kq + i < mg ? op.row_weight(pr) : 0.f;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int rr = 16 * g + c;
            if (rr < n_rr) {
                const int xb = rr / RK, r = rr - xb * RK;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * w + 4 * kq + i;
                    const float x = acc[g][i] * sc * rw[i];
                    const float hi = bf16_round(x);
                    uint16_t *xl = reinterpret_cast<uint16_t *>(lds + row * XS) + xb * 2 * RK;
                    xl[r] = __builtin_bit_cast(uint16_t, (__bf16)hi);
                    xl[RK + r] = __builtin_bit_cast(uint16_t, (__bf16)(x - hi));
                }
            }
        }
    }
    __syncthreads();

    // ---- expand: chunks of 64 columns of each window, chunk q on wave q % 4
    float *dt = reinterpret_cast<float *>(lds + kSegTiles * 16 * XS) + w * 16 * kSegDt;
    const int n_win = op.n_xs();
    const int W = op.xoff(1) - op.xoff(0);  // window width (I)
    const int cpw = (W + 63) / 64;          // chunks per window
    const int n_chunks = n_win * cpw;
    // the xa operands of every tile for each window block: RK <= 16 packs hi and lo in one k block
    constexpr int QH = RK / 8;  // k quarters of one term
    auto xa_op = [&](int rt, int xb, bool lo_term) -> u32x4_t {
        const uint16_t *xl = reinterpret_cast<const uint16_t *>(lds + (16 * rt + c) * XS) + xb * 2 * RK;
        if constexpr (RK <= 16) {
            (void)lo_term;
            if (kq < QH) return ld16(xl + 8 * kq);
            if (kq < 2 * QH) return ld16(xl + RK + 8 * (kq - QH));
            return zero4();
        } else {
            return ld16(xl + (lo_term ? RK : 0) + 8 * kq);
        }
    };
    const rsrc_t rb0 = op.b_rsrc(bs, 0), rb1 = op.b_rsrc(bs, 1), ry = op.y_rsrc(sa.n_rows);
    auto load_b = [&](int q, u32x4_t (&bv)[4]) {
        const int l = min(q, n_chunks - 1) / cpw, cw0 = 64 * (q - l * cpw);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int cw = cw0 + 16 * ct + c;  // column within window l
            const int rk = RK <= 16 ? 8 * (kq % QH) : 8 * kq;
            bv[ct] = buf_ld16<kNt>(l == 0 ? rb0 : rb1, (q < n_chunks && cw < W) ? op.b_off(l, cw, rk) : kOob);
        }
    };
    // the wave's chunks q = w + 4 j; PB chunks of B in flight (the shrink's
    // registers are free now)
    constexpr int PB = 2;
    u32x4_t bq[PB][4];
#pragma unroll
    for (int b = 0; b < PB; ++b) load_b(w + 4 * b, bq[b]);
    for (int j0 = 0; w + 4 * j0 < n_chunks; j0 += PB) {
#pragma unroll
        for (int b = 0; b < PB; ++b) {
        const int q = w + 4 * (j0 + b);
        if (q >= n_chunks) break;
        u32x4_t cur[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) cur[ct] = bq[b][ct];
        load_b(q + 4 * PB, bq[b]);  // refill the slot: the chunk PB ahead
        const int l = q / cpw, col0 = op.xoff(l) + 64 * (q - l * cpw), c1 = op.xoff(l + 1);
        const int xb = op.xblk(l);
        // row tile rt's out rows 4 j + kq, columns col0 + 4c .. + 4
        auto tile_yoff = [&](int rt, uint32_t (&yoff)[4]) {
            const int rt_pid = rt == 0 ? pid[0] : rt == 1 ? pid[1] : rt == 2 ? pid[2] : pid[3];
            const int mrt = rt == 0 ? mt[0] : rt == 1 ? mt[1] : rt == 2 ? mt[2] : mt[3];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * j + kq, col = col0 + 4 * c;
                // (the shuffle runs in every lane: a lane it reads from must be active)
                const int pr = __shfl(rt_pid, row, kWave);
                yoff[j] = (row < mrt && col < c1) ? op.y_off(pr, col) : kOob;
            }
        };
        // w2 adds to y: the y of every row tile of the chunk is loaded before
        // the chunk's first store, so its latency is paid once per chunk (the
        // compiler keeps a load of y after the stores to y before it)
        uint32_t yoff_all[Op::kAddInputs ? kSegTiles : 1][4];
        uint2 yv_all[Op::kAddInputs ? kSegTiles : 1][4];
        if constexpr (Op::kAddInputs) {
#pragma unroll
            for (int rt = 0; rt < kSegTiles; ++rt) {
                tile_yoff(rt, yoff_all[rt]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (rt >= nt) yoff_all[rt][j] = kOob;
                    yv_all[rt][j] = buf_ld8<kNt>(ry, yoff_all[rt][j]);
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < kSegTiles; ++rt) {
            if (rt >= nt) break;
            uint32_t yoff[4];
            uint2 yv[4];
            if constexpr (Op::kAddInputs) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    yoff[j] = yoff_all[rt][j];
                    yv[j] = yv_all[rt][j];
                }
            } else {
                tile_yoff(rt, yoff);
            }
            f32x4_t d[4];
            const u32x4_t h0 = xa_op(rt, xb, false);
            u32x4_t h1 = zero4();
            if constexpr (RK > 16) h1 = xa_op(rt, xb, true);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                d[ct] = mfma_16x16x32(cur[ct], h0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                if constexpr (RK > 16) d[ct] = mfma_16x16x32(cur[ct], h1, d[ct]);
            }
            // lane (c, kq) holds out row c, columns 16 ct + 4 kq .. + 4: through
            // the wave's tile to rows of 64 columns, 16 lanes x 8 bytes each
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                *reinterpret_cast<f32x4_t *>(dt + c * kSegDt + 16 * ct + 4 * kq) = d[ct];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * j + kq;
                const f32x4_t o = *reinterpret_cast<const f32x4_t *>(dt + row * kSegDt + 4 * c);
                float v[4] = {o[0], o[1], o[2], o[3]};
                if constexpr (Op::kAddInputs) {
                    v[0] += bf_lo(yv[j].x);
                    v[1] += bf_hi(yv[j].x);
                    v[2] += bf_lo(yv[j].y);
                    v[3] += bf_hi(yv[j].y);
                }
                buf_st8<kNt>(ry, yoff[j], make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
            }
            __builtin_amdgcn_wave_barrier();
        }
        }
    }
}

}  // namespace tl
