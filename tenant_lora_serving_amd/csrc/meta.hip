// meta.hip -- per-step routing metadata: rows sorted by (slot, row), segment
// offsets, the active-slot list and 16-row tile records.
//
// What is computed follows vLLM punica_base.py (PunicaWrapperBase: per-token
// lora indices, -1 meaning no lora; prefill_metadata grouping the rows of one
// adapter into segments with their start and length) and metrale's lora_delta
// docs (apply_lora_bgmv: a negative slot gets no delta).  Rows are ordered by
// (slot, row), which makes the result unique, so it is compared bit-exactly.
//
// Design (gfx950): one 1024-thread workgroup per chunk of 1024 rows.
//  1. Each chunk is sorted by slot in LDS, stably: up to 512 slots in one
//     pass (per-wave ballots, one per key bit, give each lane its rank among
//     equal keys; a [key][wave] table is scanned for the positions), else
//     with 4-bit radix passes ranked the same way.  Inactive and invalid
//     rows get the key S and sort to the end.  A split build (below) with up
//     to 512 slots does not move the rows at all: each keeps its rank among
//     the chunk's rows of its slot, which is all its placement needs.
//  2. Runs of one slot in the sorted chunk are found with a block scan.
//  3. One chunk: the workgroup writes every output directly.
//     Several chunks: each writes its sorted chunk to the workspace.  When a
//     [chunk][slot] table of run lengths fits LDS and there are at most 64
//     chunks, a second launch of one workgroup per chunk follows: each reads
//     every chunk's slot counts from the workspace, scans them (rows of a slot in earlier
//     chunks come first, so rows keep ascending order within a slot) and
//     places its own chunk's rows.
//     Otherwise the last workgroup to finish the first launch (atomic ticket,
//     release/acquire at agent scope) scans the per-slot counts and scatters
//     every chunk in order.
// No step waits on another workgroup, so nothing can hang.
#include "common.h"
#include "kernels.h"
#include "slot_meta.h"

#include <algorithm>

namespace tl {

constexpr int kMT = kMetaChunk;  // threads per workgroup = rows per chunk
constexpr int kAsmBatch = 16;      // chunks whose entries the assembling workgroup loads at once



// MoE pair p = t*top_k + j: adapter l = lora_ids[t], expert e = topk_ids[p].
// key = l*E + e; -1 when l < 0; L*E (invalid) when l >= L or e outside [0, E).
struct SlotSrcMoe {
    const int32_t *topk;
    const int32_t *lora;
    int top_k, E, L;
    __device__ int32_t key(int p) const {
        const int l = lora[p / top_k];
        const int e = topk[p];
        if (l < 0) return -1;
        if (l >= L || e < 0 || e >= E) return L * E;
        return l * E + e;
    }
};

// Expert-sorted rows (metrale expert_apply.rs: expert e owns sorted rows
// offsets[e] .. offsets[e+1] of the expert_offsets prefix sum): key of row r
// = slot[e] of the expert whose block holds r, -1 when none does.  The block
// is found by binary search for the first offset above r, so every row gets
// at most one expert even when the offsets are not a prefix sum.
struct SlotSrcBlocks {
    const uint32_t *off;  // [nb + 1]
    const int32_t *slot;  // [nb]
    int nb;
    __device__ int32_t key(int r) const {
        const uint32_t ur = (uint32_t)r;
        int lo = 0, hi = nb + 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= ur)
                lo = mid + 1;
            else
                hi = mid;
        }
        const int e = lo - 1;
        if (e < 0 || e >= nb || off[e] > ur || ur >= off[e + 1]) return -1;
        return slot[e];
    }
};

struct MetaShared {
    uint32_t key[kMT];
    int32_t val[kMT];
    int32_t hist[256];
    int32_t run_start[kMT];
    int32_t run_tile[kMT];
    int32_t scan[kMT / kWave + 1];
    Int3 scan3[kMT / kWave + 1];
    int flag_last;
};

// One stable pass of the LDS radix sort on digit (key >> shift) & 15.
__device__ __forceinline__ void radix_pass(uint32_t &key, int32_t &val, int shift, MetaShared &sh) {
    const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
    const uint32_t d = (key >> shift) & 15u;
    const uint64_t lt = lanemask_lt();
    uint64_t mine = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const uint64_t m = __ballot(d == (uint32_t)b);
        if (d == (uint32_t)b) mine = m;
        if (lane == b) sh.hist[b * 16 + w] = __popcll(m);
    }
    const int rank = __popcll(mine & lt);
    __syncthreads();
    int tot;
    const int hv = tid < 256 ? sh.hist[tid] : 0;
    const int hx = block_excl_scan<kMT>(hv, sh.scan, tot);
    if (tid < 256) sh.hist[tid] = hx;
    __syncthreads();
    const int pos = sh.hist[d * 16 + w] + rank;
    sh.key[pos] = key;
    sh.val[pos] = val;
    __syncthreads();
    key = sh.key[tid];
    val = sh.val[tid];
    __syncthreads();
}


// The chunk sorted by key in one pass (stable, as the radix passes), for
// S <= kBallotSortSlots: each wave ranks its lanes among equal keys with one
// ballot per key bit (few_rank), a [key][wave] table of group sizes is
// scanned key-major in wave order, and every entry moves to its position.
// tab: (S + 1) * 16 ints of LDS.
constexpr int kBallotSortSlots = 512;
__device__ __forceinline__ void ballot_sort(uint32_t &key, int32_t &val, int S, MetaShared &sh, int *tab) {
    constexpr int W = kMT / kWave;
    const int tid = threadIdx.x, w = wave_id();
    const int n_ent = (S + 1) * W;
    for (int i = tid; i < n_ent; i += kMT) tab[i] = 0;
    __syncthreads();
    int group;
    const int rank = few_rank((int)key, true, S + 1, group);
    if (rank == 0) tab[key * W + w] = group;
    __syncthreads();
    const int per = (n_ent + kMT - 1) / kMT;  // contiguous entries per thread
    const int e0 = min(n_ent, tid * per), e1 = min(n_ent, e0 + per);
    int loc = 0;
    for (int i = e0; i < e1; ++i) loc += tab[i];
    int total;
    int base = block_excl_scan<kMT>(loc, sh.scan, total);
    for (int i = e0; i < e1; ++i) {
        const int v = tab[i];
        tab[i] = base;
        base += v;
    }
    __syncthreads();
    const int pos = tab[key * W + w] + rank;
    sh.key[pos] = key;
    sh.val[pos] = val;
    __syncthreads();
    key = sh.key[tid];
    val = sh.val[tid];
    __syncthreads();
}

// A chunk of a split build, ranked instead of sorted: the assembling launch
// places each row from its key, its rank among the chunk's rows of that key
// (rows keep ascending order) and every chunk's per-slot counts, all that
// the sorted order would have given it.  Each wave ranks its lanes with one
// ballot per key bit (few_rank); a [wave][slot] table of group sizes, scanned
// over the waves per slot, turns wave ranks into chunk ranks and gives the
// chunk's count of every slot.  tab: S * 16 ints of LDS.
__device__ __forceinline__ void rank_chunk(uint32_t key, int e, bool invalid, int S, int c, MetaWs ws, int *tab) {
    constexpr int W = kMT / kWave;
    const int tid = threadIdx.x, w = wave_id();
    for (int i = tid; i < S * W; i += kMT) tab[i] = 0;
    const int n_inv_chunk = __syncthreads_count(invalid);
    const bool act = key < (uint32_t)S;
    int group;
    const int rank = few_rank(act ? (int)key : -1, act, S, group);
    if (act && rank == 0) tab[w * S + key] = group;
    __syncthreads();
    for (int s = tid; s < S; s += kMT) {
        int acc = 0;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            const int v = tab[ww * S + s];
            tab[ww * S + s] = acc;
            acc += v;
        }
        ws.hist[(int64_t)c * S + s] = acc;
    }
    __syncthreads();
    const int64_t idx = (int64_t)c * kMT + tid;
    ws.rows[idx] = e;
    ws.keys[idx] = (int)key;
    ws.offlen[idx] = act ? tab[w * S + key] + rank : 0;
    if (tid == 0 && n_inv_chunk) atomicAdd(&ws.ctl[1], n_inv_chunk);
}

// Assembly of a multi-chunk build from the chunks' sorted entries in the
// workspace: rows per slot (and per chunk), a scan over slots, then the
// scatter of every chunk (only < 0) or of chunk `only` alone, which needs
// the [chunk][slot] table.  Workgroup `only == 0` (or the single assembler)
// writes the segment arrays and the counts.
__device__ void meta_assemble(int n, int S, int n_chunks, MetaOut out, MetaWs ws, MetaShared &sh, int *dyn,
                              int only) {
    const int tid = threadIdx.x;
    int *start = dyn, *segidx = dyn + S, *tileoff = dyn + 2 * S, *rc = dyn + 3 * S;
    // With a [chunk][slot] table in LDS, every chunk's rows are placed at once:
    // cb[c][s] = rows of slot s in chunks before c.  Otherwise the chunks are
    // scattered one after another, rc[s] counting the rows already placed.
    const bool table = meta_table_fits(n_chunks, S);
    const bool writer = only < 0 || only == 0;  // writes the per-segment outputs and counts
    int *cb = dyn + 4 * S;
    // One chunk's placement with the per-chunk slot counts at hand (a split
    // build): each slot's rows in all chunks and in the chunks before this
    // one, from [chunk][slot] counts, kAsmBatch chunks' loads in flight.
    const bool from_hist = only >= 0 && ws.hist && table;
    // a split assembler's own chunk entries, loaded with the slot counts
    // rather than after the scans
    uint32_t own_k = (uint32_t)S;
    int own_ol = 0, own_row = 0;
    if (from_hist) {
        const int64_t idx = (int64_t)only * kMT + tid;
        own_k = (uint32_t)ws.keys[idx];
        own_ol = ws.offlen[idx];
        own_row = ws.rows[idx];
    }
    if (from_hist) {
        for (int s = tid; s < S; s += kMT) {
            int acc = 0, before = 0;
            for (int c0 = 0; c0 < n_chunks; c0 += kAsmBatch) {
                int v[kAsmBatch];
#pragma unroll
                for (int u = 0; u < kAsmBatch; ++u) v[u] = c0 + u < n_chunks ? ws.hist[(int64_t)(c0 + u) * S + s] : 0;
#pragma unroll
                for (int u = 0; u < kAsmBatch; ++u) {
                    if (c0 + u == only) before = acc;
                    acc += v[u];
                }
            }
            rc[s] = acc;
            cb[(int64_t)only * S + s] = before;
        }
        __syncthreads();
    }
    if (table && !from_hist) {
        for (int i = tid; i < n_chunks * S; i += kMT) cb[i] = 0;
    }
    for (int s = tid; !from_hist && s < S; s += kMT) rc[s] = 0;
    __syncthreads();
    // rows per slot (and per chunk): each run's first entry carries its length;
    // the loads of kAsmBatch chunks are issued before any is used
    for (int c0 = 0; !from_hist && c0 < n_chunks; c0 += kAsmBatch) {
        uint32_t kb[kAsmBatch];
        int ob[kAsmBatch];
#pragma unroll
        for (int u = 0; u < kAsmBatch; ++u) {
            const int64_t idx = (int64_t)(c0 + u) * kMT + tid;
            kb[u] = c0 + u < n_chunks ? (uint32_t)ws.keys[idx] : (uint32_t)S;
            ob[u] = c0 + u < n_chunks ? ws.offlen[idx] : 1;
        }
#pragma unroll
        for (int u = 0; u < kAsmBatch; ++u) {
            if (kb[u] < (uint32_t)S && (ob[u] & 0xffff) == 0) {
                if (table)
                    cb[(c0 + u) * S + kb[u]] = ob[u] >> 16;
                else
                    atomicAdd(&rc[kb[u]], ob[u] >> 16);
            }
        }
    }
    __syncthreads();
    if (table && !from_hist) {
        for (int s2 = tid; s2 < S; s2 += kMT) {
            int acc = 0;
            for (int cc = 0; cc < n_chunks; ++cc) {
                const int v = cb[cc * S + s2];
                cb[cc * S + s2] = acc;
                acc += v;
            }
            rc[s2] = acc;
        }
        __syncthreads();
    }
    // scan {rows, segments, tiles} over slots, each thread a contiguous block
    const int per = (S + kMT - 1) / kMT;
    const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
    Int3 loc = {0, 0, 0};
    int lng = 0;
    for (int s = s0; s < s1; ++s) {
        const int v = rc[s];
        loc = loc + Int3{v, v > 0, seg_tiles(v, n)};
        lng += v >= kTileRows;
    }
    Int3 tot;
    Int3 run = block_excl_scan3<kMT>(loc, sh.scan3, tot);
    int n_long;
    block_excl_scan<kMT>(lng, sh.scan, n_long);
    for (int s = s0; s < s1; ++s) {
        const int v = rc[s];
        start[s] = run.a;
        segidx[s] = run.b;
        tileoff[s] = run.c;
        if (v > 0 && writer) {
            out.seg_offsets[run.b] = run.a;
            out.seg_slot[run.b] = s;
        }
        run = run + Int3{v, v > 0, seg_tiles(v, n)};
        rc[s] = 0;
    }
    __syncthreads();
    if (tid == 0 && writer) {
        out.seg_offsets[tot.b] = tot.a;
        out.counts[0] = tot.a;
        out.counts[1] = tot.b;
        out.counts[2] = __hip_atomic_load(&ws.ctl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        out.counts[3] = n_long;
        out.counts[4] = tot.c;
        out.counts[5] = out.counts[6] = out.counts[7] = 0;
    }
    // entry (key k2, offset+length ol, row) of chunk cc to its place
    auto place = [&](int cc, uint32_t k2, int ol, int row) {
        if (k2 >= (uint32_t)S) return;
        const int o = cb[cc * S + k2] + (ol & 0xffff);
        const int dest = start[k2] + o;
        const int seg_rows = (k2 + 1 < (uint32_t)S ? start[k2 + 1] : tot.a) - start[k2];
        out.sorted_rows[dest] = row;
        const int per = seg_tile_rows(seg_rows, n);
        const int t = tileoff[k2] + o / per, j = o % per;
        int32_t *rec = out.tiles + (int64_t)t * kTileWords;
        rec[kRecRowIds + j] = row;
        if (j == 0) write_tile_header(rec, (int)k2, dest, min(per, seg_rows - o), seg_rows, segidx[k2], o / per);
    };
    if (from_hist) {
        place(only, own_k, own_ol, own_row);
    } else if (table) {
        // every chunk, or only chunk `only`
        const int cbeg = only < 0 ? 0 : only, cend = only < 0 ? n_chunks : only + 1;
        for (int c0 = cbeg; c0 < cend; c0 += kAsmBatch) {
            uint32_t kb[kAsmBatch];
            int ob[kAsmBatch], rb[kAsmBatch];
#pragma unroll
            for (int u = 0; u < kAsmBatch; ++u) {
                const int64_t idx = (int64_t)(c0 + u) * kMT + tid;
                const bool in = c0 + u < cend;
                kb[u] = in ? (uint32_t)ws.keys[idx] : (uint32_t)S;
                ob[u] = in ? ws.offlen[idx] : 0;
                rb[u] = in ? ws.rows[idx] : 0;
            }
#pragma unroll
            for (int u = 0; u < kAsmBatch; ++u) place(c0 + u, kb[u], ob[u], rb[u]);
        }
    }
    // scatter the chunks in order; rc[s] counts the rows of slot s already placed
    for (int cc = 0; !table && cc < n_chunks; ++cc) {
        const int64_t idx = (int64_t)cc * kMT + tid;
        const uint32_t k2 = (uint32_t)ws.keys[idx];
        const int ol = ws.offlen[idx];
        const int off2 = ol & 0xffff, len2 = ol >> 16;
        const bool a2 = k2 < (uint32_t)S;
        if (a2) {
            const int row = ws.rows[idx];
            const int o = rc[k2] + off2;
            const int dest = start[k2] + o;
            const int seg_rows = (k2 + 1 < (uint32_t)S ? start[k2 + 1] : tot.a) - start[k2];
            out.sorted_rows[dest] = row;
            const int per = seg_tile_rows(seg_rows, n);
            const int t = tileoff[k2] + o / per, j = o % per;
            int32_t *rec = out.tiles + (int64_t)t * kTileWords;
            rec[kRecRowIds + j] = row;
            if (j == 0)
                write_tile_header(rec, (int)k2, dest, min(per, seg_rows - o), seg_rows, segidx[k2], o / per);
        }
        __syncthreads();
        if (a2 && off2 == 0) rc[k2] += len2;
        __syncthreads();
    }
    // empty records past the last tile, shared by the assembling workgroups
    const int g = only < 0 ? 0 : only, ng = only < 0 ? 1 : n_chunks;
    for (int t = tot.c + g * kMT + tid; t < out.tile_bound; t += ng * kMT)
        write_tile_header(out.tiles + (int64_t)t * kTileWords, 0, 0, 0, 0, 0, 0);
}

template <class Src>
__global__ __launch_bounds__(kMT) void meta_kernel(Src src, int n, int S, int n_chunks, MetaOut out,
                                                   MetaWs ws, int split) {
    __shared__ MetaShared sh;
    extern __shared__ int dyn[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    const int e = c * kMT + tid;
    const bool real = e < n;
    const int raw = real ? src.key(e) : -1;
    const bool invalid = real && raw >= S;
    uint32_t key = (real && raw >= 0 && raw < S) ? (uint32_t)raw : (uint32_t)S;
    int32_t val = e;

    if (split && ws.hist && S <= kBallotSortSlots) {  // meta_assemble_kernel follows in the same stream
        rank_chunk(key, e, invalid, S, c, ws, dyn);
        return;
    }
    if (S <= kBallotSortSlots) {
        ballot_sort(key, val, S, sh, dyn);
    } else {
        const int nbits = 32 - __clz(S);  // bits holding 0..S
        for (int shift = 0; shift < nbits; shift += 4) radix_pass(key, val, shift, sh);
    }

    // runs of equal keys in the sorted chunk
    const uint32_t prev = tid > 0 ? sh.key[tid - 1] : 0xFFFFFFFFu;
    const int leader = key != prev;
    int n_runs;
    const int run_id = block_excl_scan<kMT>(leader, sh.scan, n_runs) + leader - 1;
    if (leader) sh.run_start[run_id] = tid;
    __syncthreads();
    const int rstart = sh.run_start[run_id];
    const int rend = run_id + 1 < n_runs ? sh.run_start[run_id + 1] : kMT;
    const int off = tid - rstart, len = rend - rstart;
    const bool act = key < (uint32_t)S;
    const int n_inv_chunk = __syncthreads_count(invalid);

    if (n_chunks == 1) {
        const int seg_lead = leader && act;
        const int n_active = __syncthreads_count(act);
        const int n_long = __syncthreads_count(seg_lead && len >= kTileRows);
        int n_tiles;
        const int tile_x =
            block_excl_scan<kMT>(seg_lead ? seg_tiles(len, n) : 0, sh.scan, n_tiles);
        if (seg_lead) sh.run_tile[run_id] = tile_x;
        const int n_seg = __syncthreads_count(seg_lead);
        if (act) {
            out.sorted_rows[tid] = val;
            if (leader) {
                out.seg_offsets[run_id] = tid;
                out.seg_slot[run_id] = (int)key;
            }
            const int per = seg_tile_rows(len, n);
            const int t = sh.run_tile[run_id] + off / per, j = off % per;
            int32_t *rec = out.tiles + (int64_t)t * kTileWords;
            rec[kRecRowIds + j] = val;
            if (j == 0) write_tile_header(rec, (int)key, tid, min(per, len - off), len, run_id, off / per);
        }
        if (tid == 0) {
            out.seg_offsets[n_seg] = n_active;
            out.counts[0] = n_active;
            out.counts[1] = n_seg;
            out.counts[2] = n_inv_chunk;
            out.counts[3] = n_long;
            out.counts[4] = n_tiles;
            out.counts[5] = out.counts[6] = out.counts[7] = 0;
        }
        for (int t = n_tiles + tid; t < out.tile_bound; t += kMT)
            write_tile_header(out.tiles + (int64_t)t * kTileWords, 0, 0, 0, 0, 0, 0);
        return;
    }

    // ---- several chunks: publish this chunk, the last workgroup assembles
    {
        const int64_t idx = (int64_t)c * kMT + tid;
        ws.rows[idx] = val;
        ws.keys[idx] = (int)key;
        ws.offlen[idx] = off | (len << 16);
    }
    if (tid == 0 && n_inv_chunk) atomicAdd(&ws.ctl[1], n_inv_chunk);
    if (split) {  // meta_assemble_kernel follows in the same stream
        if (ws.hist) {  // this chunk's rows of every slot (the run lengths, zero for absent slots)
            for (int s = tid; s < S; s += kMT) dyn[s] = 0;
            __syncthreads();
            if (leader && act) dyn[key] = len;
            __syncthreads();
            for (int s = tid; s < S; s += kMT) ws.hist[(int64_t)c * S + s] = dyn[s];
        }
        return;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) sh.flag_last = atomic_add_acqrel(&ws.ctl[0], 1) == n_chunks - 1;
    __syncthreads();
    if (!sh.flag_last) return;
    __threadfence();

    meta_assemble(n, S, n_chunks, out, ws, sh, dyn, -1);
    if (tid == 0) {
        store_relaxed(&ws.ctl[0], 0);
        store_relaxed(&ws.ctl[1], 0);
    }
}

// Second launch of a split build: workgroup c places chunk c.  The invalid
// count is read (and cleared for the next call) by workgroup 0 alone.
__global__ __launch_bounds__(kMT) void meta_assemble_kernel(int n, int S, int n_chunks, MetaOut out, MetaWs ws) {
    __shared__ MetaShared sh;
    extern __shared__ int dyn[];
    meta_assemble(n, S, n_chunks, out, ws, sh, dyn, blockIdx.x);
    if (blockIdx.x == 0 && threadIdx.x == 0) store_relaxed(&ws.ctl[1], 0);
}

// ------------------------------------------------------------ small batches
// (small_meta_build, slot_meta.h) as a kernel of one workgroup.
template <int NT, class Src>
__global__ __launch_bounds__(NT) void meta_small_kernel(Src src, int n, int S, MetaOut out) {
    extern __shared__ int dyn[];
    __shared__ Int3 scan3[NT / kWave + 1];
    __shared__ int cnt2[2];
    small_meta_build<NT>(src, n, S, out, dyn, scan3, cnt2);
}

static int small_threads(int n) { return n <= 64 ? 64 : (n <= 256 ? 256 : 1024); }

// Past 256 rows with many slots, up to 64 distinct slots per wave make the
// per-wave ranking slower than the radix path.
static bool small_fits(int n, int S) {
    return n <= kMT && S <= kSmallMaxSlots && (long long)(small_threads(n) / kWave) * S <= kSmallTable &&
           (n <= 256 || S <= kSmallBallotSlots);
}

static size_t small_lds(int n, int S) { return ((size_t)S * (small_threads(n) / kWave) + 3 * (size_t)S) * sizeof(int); }


size_t meta_dyn_lds(int n, int S) {
    const int c = meta_chunks(n);
    if (c <= 1) return 0;
    return (size_t)(meta_table_fits(c, S) ? 4 + c : 4) * S * sizeof(int);
}

template <int NT, class Src>
static hipError_t launch_small(Src src, int n, int S, MetaOut out, hipStream_t st) {
    const size_t dyn = small_lds(n, S);
    if (dyn > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(meta_small_kernel<NT, Src>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    hipLaunchKernelGGL((meta_small_kernel<NT, Src>), dim3(1), dim3(NT), dyn, st, src, n, S, out);
    return hipGetLastError();
}

template <class Src>
static hipError_t launch_meta(Src src, int n, int S, MetaOut out, MetaWs ws, hipStream_t st) {
    if (small_fits(n, S)) {
        switch (small_threads(n)) {
        case 64: return launch_small<64>(src, n, S, out, st);
        case 256: return launch_small<256>(src, n, S, out, st);
        default: return launch_small<1024>(src, n, S, out, st);
        }
    }
    const int chunks = meta_chunks(n);
    // every chunk workgroup's LDS: the one-pass sort's table, the assembly's
    // table and slot arrays (the single assembler), the chunk's slot counts
    // (a split build)
    const int split = chunks > 1 && chunks <= kSplitMaxChunks && meta_table_fits(chunks, S);
    const size_t sort_lds = S <= kBallotSortSlots ? (size_t)(S + 1) * (kMT / kWave) * sizeof(int) : 0;
    const size_t dyn = meta_dyn_lds(n, S);
    const size_t first = std::max(sort_lds, split ? (size_t)S * sizeof(int) : dyn);
    if (first > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(meta_kernel<Src>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)first);
    // every workgroup of the second launch reads all chunks' slot counts
    // (work quadratic in the chunk count), so very long batches assemble alone
    hipLaunchKernelGGL(meta_kernel<Src>, dim3(chunks), dim3(kMT), first, st, src, n, S, chunks, out, ws, split);
    if (!split) return hipGetLastError();
    if (dyn > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(meta_assemble_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    hipLaunchKernelGGL(meta_assemble_kernel, dim3(chunks), dim3(kMT), dyn, st, n, S, chunks, out, ws);
    return hipGetLastError();
}

hipError_t launch_meta_dense(const int32_t *slot, int n, int S, MetaOut out, MetaWs ws, hipStream_t st) {
    return launch_meta(SlotSrcDense{slot}, n, S, out, ws, st);
}

hipError_t launch_meta_moe(const int32_t *topk, const int32_t *lora, int top_k, int E, int L, int n_pairs,
                           MetaOut out, MetaWs ws, hipStream_t st) {
    return launch_meta(SlotSrcMoe{topk, lora, top_k, E, L}, n_pairs, L * E, out, ws, st);
}

hipError_t launch_meta_blocks(const uint32_t *offsets, const int32_t *block_slot, int n_blocks, int n, int S,
                              MetaOut out, MetaWs ws, hipStream_t st) {
    return launch_meta(SlotSrcBlocks{offsets, block_slot, n_blocks}, n, S, out, ws, st);
}

}  // namespace tl
