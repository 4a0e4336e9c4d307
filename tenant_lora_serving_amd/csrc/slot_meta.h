// slot_meta.h -- the routing metadata of a small batch (at most 1024 rows,
// one row per thread of one workgroup), shared by the metadata kernel and by
// the fused kernel, which can build it in the same launch as the delta.
//
// What is computed follows vLLM punica_base.py (PunicaWrapperBase: per-token
// lora indices, -1 meaning no lora) and metrale's lora_delta docs
// (apply_lora_bgmv): active rows sorted by (slot, row), segments of one slot,
// and the 16-row tile records the delta kernels run on.
#pragma once

#include "common.h"
#include "kernels.h"

namespace tl {

struct SlotSrcDense {
    const int32_t *slot;
    __device__ int32_t key(int i) const { return slot[i]; }
};

__device__ __forceinline__ void write_tile_header(int32_t *rec, int slot, int pos, int rows, int seg_rows,
                                                  int seg, int jt) {
    rec[kRecSlot] = slot;
    rec[kRecPos] = pos;
    rec[kRecRows] = rows;
    rec[kRecSegRows] = seg_rows;
    rec[kRecSeg] = seg;
    rec[kRecSegTile] = jt;
    rec[6] = 0;
    rec[7] = 0;
}

// ------------------------------------------------------------ small batches
// n <= 1024 rows and a slot table that fits LDS: one workgroup of NT >= n
// threads, one row per thread.  Each wave ranks its rows among equal slots
// with one ballot per distinct slot present in the wave and records how many
// rows of each slot it holds in a [slot][wave] table; one block scan over
// the slots turns the table into every (slot, wave)'s first sorted position
// and gives each slot its segment index and first tile.  Since waves hold
// rows in order, rows stay in ascending order within a slot.
constexpr int kSmallTable = 16384;  // slots x waves entries of the count table
constexpr int kSmallMaxSlots = 4096;

// Rank of the lane's row among the wave's active rows of the same slot, and
// (group) how many there are, for S <= kSmallBallotSlots: one ballot per bit
// of the slot number, a lane's group being the lanes that agree on every bit.
__device__ __forceinline__ int few_rank(int key, bool active, int S, int &group) {
    uint64_t same = __ballot(active);
    const int nbits = S > 1 ? 32 - __clz(S - 1) : 0;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t mb = __ballot(active && bit);
        same &= bit ? mb : ~mb;
    }
    group = __popcll(same);
    return __popcll(same & lanemask_lt());
}

template <int NT, class Src>
__device__ __forceinline__ void small_meta_build(Src src, int n, int S, const MetaOut &out, int *dyn, Int3 *scan3,
                                                 int *cnt2) {
    constexpr int W = NT / kWave;
    int *tab = dyn;                        // [S][W]: counts, then first sorted positions
    int *seg_idx = tab + (size_t)S * W;    // [S]
    int *tile_off = seg_idx + S;           // [S]
    int *start = tile_off + S;             // [S]
    int &n_long = cnt2[0], &n_invalid = cnt2[1];
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int raw = tid < n ? src.key(tid) : -1;
    const bool active = tid < n && raw >= 0 && raw < S;
    const int key = active ? raw : -1;
    for (int i = tid; i < S * W; i += NT) tab[i] = 0;
    if (tid == 0) n_long = n_invalid = 0;
    __syncthreads();
    if (tid < n && raw >= S) atomicAdd(&n_invalid, 1);
    // rank among the wave's rows of the same slot.  Few slots: one ballot per
    // bit of the slot number, a lane's group being the lanes that agree on
    // every bit; else one ballot per distinct slot present in the wave.
    int rank = 0;
    const bool few = S <= kSmallBallotSlots;
    if (few) {
        int group;
        rank = few_rank(key, active, S, group);
        if (active && rank == 0) tab[key * W + w] = group;  // the group's first lane
    } else {
        uint64_t pending = __ballot(active);
        while (pending) {
            const int leader = __builtin_ctzll(pending);
            const int k = __builtin_amdgcn_readlane(key, leader);
            const uint64_t same = __ballot(key == k);
            if (key == k) rank = __popcll(same & lanemask_lt());
            if (lane == leader) tab[k * W + w] = __popcll(same);
            pending &= ~same;
        }
    }
    __syncthreads();
    Int3 tot;
    if (few) {
        // wave 0 scans the slots, lane k holding slot k
        if (w == 0) {
            const int k = lane;
            int t = 0;
            if (k < S) {
#pragma unroll
                for (int ww = 0; ww < W; ++ww) t += tab[k * W + ww];
            }
            const Int3 v = {t, t > 0, seg_tiles(t, n)};
            const Int3 inc = wave_incl_scan3(v);
            const Int3 run = {inc.a - v.a, inc.b - v.b, inc.c - v.c};
            if (k < S) {
                int base = run.a;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) {
                    const int c = tab[k * W + ww];
                    tab[k * W + ww] = base;
                    base += c;
                }
                seg_idx[k] = run.b;
                tile_off[k] = run.c;
                start[k] = run.a;
                if (t > 0) {
                    out.seg_offsets[run.b] = run.a;
                    out.seg_slot[run.b] = k;
                }
            }
            const uint64_t lng = __ballot(k < S && t >= kTileRows);
            if (lane == kWave - 1) {
                scan3[0] = inc;  // the last lane's inclusive sums are the totals
                n_long = __popcll(lng);
            }
        }
        __syncthreads();
        tot = scan3[0];
    } else {
        // per-slot totals: {rows, segments, tiles}, scanned over the slots
        const int per = (S + NT - 1) / NT;
        const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
        Int3 loc = {0, 0, 0};
        for (int k = s0; k < s1; ++k) {
            int t = 0;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) t += tab[k * W + ww];
            loc = loc + Int3{t, t > 0, seg_tiles(t, n)};
            if (t >= kTileRows) atomicAdd(&n_long, 1);
        }
        Int3 run = block_excl_scan3<NT>(loc, scan3, tot);
        for (int k = s0; k < s1; ++k) {
            int t = 0;
            int base = run.a;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) {
                const int c = tab[k * W + ww];
                tab[k * W + ww] = base;
                base += c;
                t += c;
            }
            seg_idx[k] = run.b;
            tile_off[k] = run.c;
            start[k] = run.a;
            if (t > 0) {
                out.seg_offsets[run.b] = run.a;
                out.seg_slot[run.b] = k;
            }
            run = run + Int3{t, t > 0, seg_tiles(t, n)};
        }
        __syncthreads();
    }
    if (active) {
        const int pos = tab[key * W + w] + rank;
        const int st = start[key];
        const int len = (key + 1 < S ? start[key + 1] : tot.a) - st;
        const int q = pos - st;
        out.sorted_rows[pos] = tid;
        const int per = seg_tile_rows(len, n);
        const int t = tile_off[key] + q / per, j = q % per;
        int32_t *rec = out.tiles + (int64_t)t * kTileWords;
        rec[kRecRowIds + j] = tid;
        if (j == 0) write_tile_header(rec, key, pos, min(per, len - q), len, seg_idx[key], q / per);
    }
    if (tid == 0) {
        out.seg_offsets[tot.b] = tot.a;
        out.counts[0] = tot.a;
        out.counts[1] = tot.b;
        out.counts[2] = n_invalid;
        out.counts[3] = n_long;
        out.counts[4] = tot.c;
        out.counts[5] = out.counts[6] = out.counts[7] = 0;
    }
    for (int t = tot.c + tid; t < out.tile_bound; t += NT)
        write_tile_header(out.tiles + (int64_t)t * kTileWords, 0, 0, 0, 0, 0, 0);
}


// ------------------------------------------------------------ one tile's record
// The record of tile t (kTileWords words, as small_meta_build writes it into
// out.tiles) for a workgroup of kSlotThreads threads, n <= kSlotThreads rows
// and S <= kSmallBallotSlots slots, built from the slot array alone: each
// wave ranks its rows per slot (few_rank), wave 0 scans the per-slot counts
// (rows, segments, tiles) and writes the header of the slot that owns tile
// t, and the rows of tile t write their ids.  Unused words are zero (a tile
// past the last has an all-zero record).  Returns word (lane mod 32) of the
// record; n_tiles gets the batch's tile count.  Uses S * 7 + 33 ints of
// LDS at sm, free again when it returns.  (Spreading the rows over the four
// waves measured faster than wave 0 alone holding four rows per lane.)
__device__ __forceinline__ int slot_tile_record(const int32_t *slot, int n, int S, int t, int *sm, int &n_tiles) {
    constexpr int W = kSlotThreads / kWave;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    int *tab = sm;               // [S][W]: counts, then first sorted positions
    int *start = tab + S * W;    // [S] first sorted position of each slot
    int *toff = start + S;       // [S] first tile of each slot
    int *cnt = toff + S;         // [S] rows of each slot
    int *rec = cnt + S;          // [kTileWords]
    int *tot = rec + kTileWords;
    const int raw = tid < n ? slot[tid] : -1;
    const bool active = raw >= 0 && raw < S;
    const int key = active ? raw : -1;
    for (int i = tid; i < S * W; i += kSlotThreads) tab[i] = 0;
    if (tid < kTileWords) rec[tid] = 0;
    __syncthreads();
    int group;
    const int rank = few_rank(key, active, S, group);
    if (active && rank == 0) tab[key * W + w] = group;
    __syncthreads();
    if (w == 0) {
        const int k = lane;
        int c = 0;
        if (k < S) {
#pragma unroll
            for (int ww = 0; ww < W; ++ww) c += tab[k * W + ww];
        }
        const Int3 v = {c, c > 0, seg_tiles(c, n)};
        const Int3 inc = wave_incl_scan3(v);
        if (k < S) {
            int base = inc.a - v.a;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) {
                const int x = tab[k * W + ww];
                tab[k * W + ww] = base;
                base += x;
            }
            start[k] = inc.a - v.a;
            toff[k] = inc.c - v.c;
            cnt[k] = c;
            const int jt = t - (inc.c - v.c);
            if (jt >= 0 && jt < v.c) {  // the slot that owns tile t
                const int per = seg_tile_rows(c, n);
                rec[kRecSlot] = k;
                rec[kRecPos] = inc.a - v.a + jt * per;
                rec[kRecRows] = min(per, c - jt * per);
                rec[kRecSegRows] = c;
                rec[kRecSeg] = inc.b - v.b;
                rec[kRecSegTile] = jt;
            }
        }
        if (lane == kWave - 1) *tot = inc.c;
    }
    __syncthreads();
    if (active) {
        const int q = tab[key * W + w] + rank - start[key];
        const int per = seg_tile_rows(cnt[key], n);
        if (toff[key] + q / per == t) rec[kRecRowIds + q % per] = tid;
    }
    __syncthreads();
    n_tiles = *tot;
    const int word = rec[lane & (kTileWords - 1)];
    __syncthreads();
    return word;
}

}  // namespace tl
