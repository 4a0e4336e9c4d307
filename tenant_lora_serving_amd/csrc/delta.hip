// delta.hip -- standalone shrink and expand kernels (lora_shrink,
// lora_expand) for gfx950.  The one-launch fused delta lives in fused.hip.
//
// Semantics (vLLM punica_base.py, add_shrink / add_expand; metrale
// lora_delta docs, apply_lora_bgmv and LoraPair): rows of one adapter slot
// form a segment; the shrink gives xa = scale * x @ A^T in fp32, the expand
// adds xa @ B^T to the output window and rounds once to bf16.
//
// Work units.  The metadata cuts every segment into tiles of at most 16 rows
// (one 128-byte record each: slot, first sorted position, row count, segment
// size, row ids).  A workgroup takes one unit (4 waves; a shrink unit of a
// call with few units, 8 waves over 2048-wide k passes):
//   shrink unit  (tile, shrink slice): every rank row of the slice over all of k
//   expand unit  (tile, 512-column chunk): every row of the tile
// Segments with at least `mfma_min` rows (16 by default) run on
// v_mfma_f32_16x16x32_bf16; shorter ones on the vector ALU with
// v_dot2c_f32_bf16.  bf16 products are exact in fp32 on both paths.  The
// expand keeps xa's precision by splitting it into two bf16 terms
// (hi = bf16(xa), lo = bf16(xa - hi)) that both multiply B, so no bf16
// rounding of xa reaches the result beyond ~2^-16 relative.
#include "common.h"
#include "kernels.h"
#include "ops.h"

#include <algorithm>

namespace tl {

constexpr int kBT = 256;        // threads per expand workgroup
// Shrink units: 4 waves and 512-wide k passes when a call has enough units
// to fill the chip, else 8 waves and 2048-wide passes (a unit's k range in
// fewer dependent passes; one workgroup per CU at the larger LDS stage).
constexpr int kCW = 512;        // expand columns per unit
constexpr int kRRMfma = 128;    // shrink rank rows per pass on the MFMA path
constexpr int kRRValu = 64;     // shrink rank rows per pass on the vector ALU
// per-wave partial blocks when the NW waves split k: KW * n_rr * 16 floats, and
// KW * n_rr < 32 * NW rank rows (wave_split)
template <int NW>
constexpr int shrink_red_floats() { return 512 * NW; }
template <int KC>
constexpr int shrink_xs() { return KC + 8; }  // padded LDS row stride (elements) of the staged x tile
constexpr int kOutStride = 132;      // padded fp32 row stride of the MFMA output tile

// ============================================================ tile header
// The scalar fields of a tile record live in SGPRs (read through
// readfirstlane), so every branch on them is uniform; the row ids and x row
// pointers live in LDS.
struct TileLds {
    int hdr[4];
    int flag;
    int rows[kTileRows];
    const uint16_t *xrow[kTileRows];
};

struct Tile {
    int m, slot, pos0, mseg;
    const int *rows;               // LDS
    const uint16_t *const *xrow;   // LDS (null past m)
};

template <class Op>
__device__ __forceinline__ bool load_tile(const Op &op, const int32_t *tiles, int t, TileLds &sh, Tile &h) {
    const int tid = threadIdx.x;
    const int32_t *rec = tiles + (int64_t)t * kTileWords;
    if (tid < 4) sh.hdr[tid] = rec[tid == 0 ? kRecRows : tid == 1 ? kRecSlot : tid == 2 ? kRecPos : kRecSegRows];
    if (tid == 0) sh.flag = 0;
    __syncthreads();
    h.m = __builtin_amdgcn_readfirstlane(sh.hdr[0]);
    h.slot = __builtin_amdgcn_readfirstlane(sh.hdr[1]);
    h.pos0 = __builtin_amdgcn_readfirstlane(sh.hdr[2]);
    h.mseg = __builtin_amdgcn_readfirstlane(sh.hdr[3]);
    h.rows = sh.rows;
    h.xrow = sh.xrow;
    if (h.m == 0) return false;
    if (tid < kTileRows) {
        const int row = tid < h.m ? rec[kRecRowIds + tid] : 0;
        sh.rows[tid] = row;
        sh.xrow[tid] = tid < h.m ? op.xrow(row) : nullptr;
    }
    __syncthreads();
    return true;
}

__device__ __forceinline__ u32x4_t lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// How the NW waves of a shrink unit share it: GW waves (a power of two, at
// most the rank-row groups and NW) split the groups, KW = NW / GW split the
// k range (their partials are summed in wave order).  With GW the largest
// power of two <= groups (or NW), KW * n_rr stays below 32 * NW rank rows (16
// per MFMA group, 8 per vector-ALU group): the partial blocks fit
// shrink_red_floats<NW>().
template <int NW>
__device__ __forceinline__ void wave_split(int groups, int &GW, int &KW) {
    GW = (groups >= 8 && NW >= 8) ? 8 : (groups >= 4 ? 4 : (groups >= 2 ? 2 : 1));
    KW = NW / GW;
}

// Sum the KW per-wave partial blocks of `red` (n_rr * 16 floats each) into
// `res` in wave order.
template <int NT>
__device__ __forceinline__ void reduce_waves(int KW, int n_rr, float *res, const float *red) {
    __syncthreads();
    if (KW > 1) {
        for (int idx = threadIdx.x; idx < n_rr * 16; idx += NT) {
            float s = red[idx];
            for (int q = 1; q < KW; ++q) s += red[q * n_rr * 16 + idx];
            res[idx] = s;
        }
        __syncthreads();
    }
}

// ============================================================ shrink
// Every unit reads its x rows through LDS in chunks of KC columns (coalesced
// 16-byte loads, all issued before any is used) and streams the adapter's
// A rows straight from HBM into registers, eight 16-byte loads per lane in
// flight before the first is consumed.
//
// Stage x rows j < 16 (zero rows past m), columns [kc0, kc1), into xs[j][.].
template <int NT, int KC>
__device__ __forceinline__ void stage_x(const Tile &h, int kc0, int kc1, uint16_t *xs) {
    constexpr int kPerRow = KC / 8;                       // 16-byte chunks per staged row
    constexpr int kLoads = kTileRows * kPerRow / NT;      // per thread
    u32x4_t v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = threadIdx.x + NT * i;
        const int j = idx / kPerRow, k = kc0 + 8 * (idx % kPerRow);
        v[i] = (j < h.m && k < kc1) ? ld16(h.xrow[j] + k) : zero4();
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = threadIdx.x + NT * i;
        *reinterpret_cast<u32x4_t *>(xs + (idx / kPerRow) * shrink_xs<KC>() + 8 * (idx % kPerRow)) = v[i];
    }
}

// res[rl*16 + j] = sum_{k in [k0,k1)} x[row_j][k] * A[slot][rr0 + rl][k] for
// rl < n_rr <= kRRMfma, on v_mfma_f32_16x16x32_bf16 (tile rows = MFMA rows,
// rank rows = MFMA columns).
template <int NT, int KC, class Op>
__device__ __forceinline__ void shrink_mfma(const Op &op, const Tile &h, int rr0, int n_rr, int k0, int k1,
                                            float *res, float *red, uint16_t *xs) {
    constexpr int kXS = shrink_xs<KC>();
    const int lane = lane_id(), w = wave_id();
    const int groups = (n_rr + 15) >> 4;
    int GW, KW;
    wave_split<NT / kWave>(groups, GW, KW);
    const int gw = w % GW, kw = w / GW;
    const int col = lane & 15, kk = (lane >> 4) * 8;
    const bool has0 = gw < groups, has1 = gw + GW < groups;
    const int rl0 = 16 * gw + col, rl1 = 16 * (gw + GW) + col;
    const uint16_t *ap0 = (has0 && rl0 < n_rr) ? op.arow(h.slot, rr0 + rl0) : nullptr;
    const uint16_t *ap1 = (has1 && rl1 < n_rr) ? op.arow(h.slot, rr0 + rl1) : nullptr;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    u32x4_t a0[8], a1[8];
    auto load_a = [&](int kb0, int kb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = kb0 + 32 * u + kk;
            a0[u] = (ap0 && k < kb) ? ld16(ap0 + k) : zero4();
            a1[u] = (ap1 && k < kb) ? ld16(ap1 + k) : zero4();
        }
    };
    for (int kc0 = k0; kc0 < k1; kc0 += KC) {
        const int kc1 = min(k1, kc0 + KC);
        const int per = ((kc1 - kc0 + KW * 32 - 1) / (KW * 32)) * 32;
        const int ka = kc0 + kw * per, kb = min(kc1, ka + per);
        load_a(ka, kb);  // first A batch in flight while x is staged
        __syncthreads();
        stage_x<NT, KC>(h, kc0, kc1, xs);
        __syncthreads();
        for (int kb0 = ka; kb0 < kb; kb0 += 8 * 32) {
            if (kb0 > ka) load_a(kb0, kb);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = kb0 + 32 * u + kk;
                const u32x4_t xo = k < kb ? lds16(xs + col * kXS + (k - kc0)) : zero4();
                acc0 = mfma_16x16x32(xo, a0[u], acc0);  // absent groups multiply zeros
                acc1 = mfma_16x16x32(xo, a1[u], acc1);
            }
        }
    }
    // lane holds D[tile row 4*(lane>>4) + i][rank row rl]
    float *dst = KW == 1 ? res : red + kw * n_rr * 16;
    const int j0 = (lane >> 4) * 4;
    if (has0 && rl0 < n_rr) {
        dst[rl0 * 16 + j0 + 0] = acc0[0];
        dst[rl0 * 16 + j0 + 1] = acc0[1];
        dst[rl0 * 16 + j0 + 2] = acc0[2];
        dst[rl0 * 16 + j0 + 3] = acc0[3];
    }
    if (has1 && rl1 < n_rr) {
        dst[rl1 * 16 + j0 + 0] = acc1[0];
        dst[rl1 * 16 + j0 + 1] = acc1[1];
        dst[rl1 * 16 + j0 + 2] = acc1[2];
        dst[rl1 * 16 + j0 + 3] = acc1[3];
    }
    reduce_waves<NT>(KW, n_rr, res, red);
}

// Same result on the vector ALU (v_dot2c_f32_bf16) for n_rr <= kRRValu:
// a wave holds 8 rank rows x 8 k lanes; each lane dots 8 k per load and the
// 8 k lanes of a rank row are summed with xor shuffles at the end.
template <int NT, int KC, class Op>
__device__ __forceinline__ void shrink_valu(const Op &op, const Tile &h, int rr0, int n_rr, int k0, int k1,
                                            float *res, float *red, uint16_t *xs) {
    constexpr int kXS = shrink_xs<KC>();
    const int lane = lane_id(), w = wave_id();
    const int rsub = lane >> 3, kl = lane & 7;
    const int groups = n_rr >> 3;
    int GW, KW;
    wave_split<NT / kWave>(groups, GW, KW);
    const int gw = w % GW, kw = w / GW;
    const int m = h.m;
    float *dst = KW == 1 ? res : red + kw * n_rr * 16;
    u32x4_t a[8];
    for (int kc0 = k0; kc0 < k1; kc0 += KC) {
        const int kc1 = min(k1, kc0 + KC);
        const int per = ((kc1 - kc0 + KW * 64 - 1) / (KW * 64)) * 64;
        const int ka = kc0 + kw * per, kb = min(kc1, ka + per);
        // first A batch of this wave's first group in flight while x is staged
        const uint16_t *ap_first = gw < groups ? op.arow(h.slot, rr0 + 8 * gw + rsub) : nullptr;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = ka + 64 * u + 8 * kl;
            a[u] = (ap_first && k < kb) ? ld16_stream(ap_first + k) : zero4();
        }
        __syncthreads();
        stage_x<NT, KC>(h, kc0, kc1, xs);
        __syncthreads();
        for (int q = gw; q < groups; q += GW) {
            const int rl = 8 * q + rsub;
            const uint16_t *ap = op.arow(h.slot, rr0 + rl);
            float acc[kTileRows];
#pragma unroll
            for (int j = 0; j < kTileRows; ++j) acc[j] = 0.f;
            for (int kb0 = ka; kb0 < kb; kb0 += 8 * 64) {
                if (q != gw || kb0 != ka) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int k = kb0 + 64 * u + 8 * kl;
                        a[u] = k < kb ? ld16_stream(ap + k) : zero4();
                    }
                }
                // x rows past m are zero in LDS, so whole 4-row blocks run
                // without per-row branches; lanes past kb read chunk 0 and
                // multiply a zero A chunk
#pragma unroll
                for (int jb = 0; jb < kTileRows; jb += 4) {
                    if (jb < m) {
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int k = kb0 + 64 * u + 8 * kl;
                            const uint16_t *xp = xs + (k < kb ? k - kc0 : 0) + jb * kXS;
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) acc[jb + jj] = dot8(a[u], lds16(xp + jj * kXS), acc[jb + jj]);
                        }
                    }
                }
            }
            // sum the 8 k lanes of each rank row; accumulate over x chunks in dst
#pragma unroll
            for (int jb = 0; jb < kTileRows; jb += 4) {
                if (jb < m) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float v = group_sum(acc[jb + jj], 3);
                        if (kl == 0 && jb + jj < m)
                            dst[rl * 16 + jb + jj] = (kc0 == k0 ? 0.f : dst[rl * 16 + jb + jj]) + v;
                    }
                }
            }
        }
    }
    reduce_waves<NT>(KW, n_rr, res, red);
}

// Rank rows [rr0, rr0 + n_rr) of one tile over k in [k0, k1) into res
// (n_rr <= kRRMfma on the MFMA path, <= kRRValu on the vector ALU).
template <int NT, int KC, class Op>
__device__ __forceinline__ void shrink_compute(const Op &op, const Tile &h, bool mf, int rr0, int n_rr,
                                               int k0, int k1, float *res, float *red, uint16_t *xs) {
    if (mf)
        shrink_mfma<NT, KC>(op, h, rr0, n_rr, k0, k1, res, red, xs);
    else
        shrink_valu<NT, KC>(op, h, rr0, n_rr, k0, k1, res, red, xs);
}

// ============================================================ expand
// xa sources: get(slice, row id, sorted position, rank) -> fp32 xa
struct XaDirect {  // caller's xa[slice][n][R], already scaled
    const float *xa;
    int n, R;
    __device__ float get(int sg, int row, int, int r) const { return xa[((int64_t)sg * n + row) * R + r]; }
};
struct NoWait {
    __device__ bool operator()() const { return true; }
};

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// xl[sl][j][0..R) = bf16(xa), xl[sl][j][R..2R) = bf16(xa - bf16(xa)) for the
// tile rows j (zero past m) and xa slices sg_lo .. sg_lo + ns - 1.
template <class Xa>
__device__ __forceinline__ void stage_xa(const Tile &h, const Xa &xs, int sg_lo, int ns, int R, uint16_t *xl) {
    const int total = ns * kTileRows * R;
    for (int base = 0; base < total; base += 4 * kBT) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = base + threadIdx.x + kBT * i;
            const int r = idx % R, j = (idx / R) % kTileRows, sl = idx / (kTileRows * R);
            v[i] = (idx < total && j < h.m) ? xs.get(sg_lo + sl, h.rows[j], h.pos0 + j, r) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = base + threadIdx.x + kBT * i;
            if (idx < total) {
                const int r = idx % R, j = (idx / R) % kTileRows, sl = idx / (kTileRows * R);
                const float hi = bf16_round(v[i]);
                uint16_t *d = xl + (sl * kTileRows + j) * 2 * R;
                d[r] = bf16_bits(hi);
                d[R + r] = bf16_bits(v[i] - hi);
            }
        }
    }
}

// y of the 16 x 128 output tile of wave w: lane reads rows 4p + lane/16 (p < 4),
// columns cw0 + 8*(lane%16) .. +8, as 16-byte loads (issued early).
template <class Op>
__device__ __forceinline__ void prefetch_y(const Op &op, const Tile &h, int cw0, int cend, bool add_inputs,
                                           u32x4_t (&yv)[4]) {
    const int lane = lane_id();
    const int cy = cw0 + 8 * (lane & 15);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int j = 4 * p + (lane >> 4);
        yv[p] = (add_inputs && j < h.m && cy < cend) ? ld16_stream(op.yrow(h.rows[j]) + cy) : zero4();
    }
}

// y[row j][cw0 + c] = (add_inputs ? y : 0) + ol[j][c], rounded once to bf16, for
// the wave's 16 x 128 tile held in LDS (fp32, row stride kOutStride).
template <class Op>
__device__ __forceinline__ void store_tile(const Op &op, const Tile &h, const float *ol, int cw0, int cend,
                                           bool add_inputs, const u32x4_t (&yv)[4]) {
    const int lane = lane_id();
    const int cy = cw0 + 8 * (lane & 15);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int j = 4 * p + (lane >> 4);
        if (j < h.m && cy < cend) {
            const float *src = ol + j * kOutStride + 8 * (lane & 15);
            float o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = src[q];
            if (add_inputs) {
                o[0] += bf_lo(yv[p].x);
                o[1] += bf_hi(yv[p].x);
                o[2] += bf_lo(yv[p].y);
                o[3] += bf_hi(yv[p].y);
                o[4] += bf_lo(yv[p].z);
                o[5] += bf_hi(yv[p].z);
                o[6] += bf_lo(yv[p].w);
                o[7] += bf_hi(yv[p].w);
            }
            st16_stream(op.yrow(h.rows[j]) + cy,
                        u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                pack_bf16x2(o[6], o[7])});
        }
    }
}

// B chunks of instructions i0 .. i0+7 of a wave's vector-ALU expand.
template <class Op>
__device__ __forceinline__ void valu_load_b(const Op &op, const Tile &h, u32x4_t (&bv)[8], int i0, int cw0,
                                            int cpi, int lg, int n_ins, int cend, int q, int nq) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = cw0 + (i0 + i) * cpi + (lane >> lg);
        const bool ok = i0 + i < n_ins && c < cend && q < nq;
        bv[i] = ok ? ld16(op.brow(h.slot, c) + 8 * q) : zero4();
    }
}

// Vector-ALU expand of one unit.  Each B row (one output column, R ranks)
// is split over 2^lg lanes holding 8 ranks each, so every load instruction of
// a wave reads 1 KB of consecutive B rows; the per-lane partial dots are
// summed over those lanes with xor shuffles and land in the wave's 16 x 128
// fp32 tile in LDS, which is added to y with 16-byte accesses.  Wave w owns
// columns c0 + 128w .. +128, in n_ins = 128 / (64 >> lg) load instructions.
template <class Op, class Xa, class Wait>
__device__ __forceinline__ void expand_valu(const Op &op, const Tile &h, int c0, const Xa &xs, bool add_inputs,
                                            const Wait &wait, char *smem) {
    const int lane = lane_id(), w = wave_id();
    const int R = op.R, m = h.m;
    const int cend = min(c0 + kCW, op.n_out);
    const int sg_lo = op.xslice(c0), ns = op.xslice(cend - 1) - sg_lo + 1;
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);
    const size_t xl_bytes = ((size_t)ns * kTileRows * 2 * R * 2 + 15) & ~(size_t)15;
    float *ol = reinterpret_cast<float *>(smem + xl_bytes) + w * (kTileRows * kOutStride);
    const int nq = R >> 3;  // 16-byte chunks per B row
    int lg = 0;
    while ((1 << lg) < nq) ++lg;
    const int q = lane & ((1 << lg) - 1);
    const int cpi = 64 >> lg;         // columns per instruction
    const int n_ins = 128 / cpi;      // 2 .. 32
    const int cw0 = c0 + 128 * w;
    const int sg_w0 = op.xslice(min(cw0, cend - 1)), sg_w1 = op.xslice(min(cw0 + 127, cend - 1));
    const bool straddle = sg_w0 != sg_w1;
    u32x4_t bv[8];
    valu_load_b(op, h, bv, 0, cw0, cpi, lg, n_ins, cend, q, nq);
    u32x4_t yv[4];
    prefetch_y(op, h, cw0, cend, add_inputs, yv);
    if (!wait()) return;
    stage_xa(h, xs, sg_lo, ns, R, xl);
    __syncthreads();
    for (int i0 = 0; i0 < n_ins; i0 += 8) {
        if (i0 > 0) valu_load_b(op, h, bv, i0, cw0, cpi, lg, n_ins, cend, q, nq);
        if (!straddle) {
            // one xa slice under the wave's columns: each xa row chunk is read
            // once and multiplies all 8 B chunks; xa rows past m are zero in
            // LDS, so 4-row blocks run without per-row branches
            const uint16_t *xr = xl + (sg_w0 - sg_lo) * kTileRows * 2 * R + 8 * (q < nq ? q : 0);
#pragma unroll
            for (int jb = 0; jb < kTileRows; jb += 4) {
                if (jb < m) {
                    u32x4_t hv[4], lv[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        hv[jj] = lds16(xr + (jb + jj) * 2 * R);
                        lv[jj] = lds16(xr + (jb + jj) * 2 * R + R);
                    }
                    float v[8][4];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            v[i][jj] = group_sum(dot8(bv[i], lv[jj], dot8(bv[i], hv[jj], 0.f)), lg);
                    if (q == 0) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int cl = (i0 + i) * cpi + (lane >> lg);
                            if (i0 + i < n_ins)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj) ol[(jb + jj) * kOutStride + cl] = v[i][jj];
                        }
                    }
                }
            }
        } else {
            // columns straddle a slice boundary: per-instruction slice lookup
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int cl = (i0 + i) * cpi + (lane >> lg);
                const int c = cw0 + cl;
                const int sg = c < cend ? op.xslice(c) : sg_lo;
                const uint16_t *xr = xl + (sg - sg_lo) * kTileRows * 2 * R + 8 * (q < nq ? q : 0);
                for (int j = 0; j < m; ++j) {
                    const float v = group_sum(
                        dot8(bv[i], lds16(xr + j * 2 * R + R), dot8(bv[i], lds16(xr + j * 2 * R), 0.f)), lg);
                    if (q == 0 && i0 + i < n_ins) ol[j * kOutStride + cl] = v;
                }
            }
        }
    }
    __syncthreads();
    store_tile(op, h, ol, cw0, cend, add_inputs, yv);
}

// B operands of column tiles ct0 .. ct0+CTB-1 of a wave's MFMA expand; rows
// of columns outside xa slice `only` (when >= 0) are zeroed.
template <int NRS, int CTB, class Op>
__device__ __forceinline__ void mfma_load_b(const Op &op, const Tile &h, u32x4_t (&bo)[CTB][NRS], int ct0,
                                            int only, int cw0, int cend, int R) {
    const int lane = lane_id();
    const int col_l = lane & 15, kk = (lane >> 4) * 8;
#pragma unroll
    for (int i = 0; i < CTB; ++i) {
        const int c = cw0 + 16 * (ct0 + i) + col_l;
        const bool cok = c < cend && (only < 0 || op.xslice(c) == only);
        const uint16_t *b = cok ? op.brow(h.slot, c) : nullptr;
#pragma unroll
        for (int s = 0; s < NRS; ++s) {
            const int rk = 32 * s + kk;
            bo[i][s] = (cok && rk < R) ? ld16(b + rk) : zero4();
        }
    }
}

// MFMA expand of one unit: D[column][tile row] = B[column][ranks] .
// (xa_hi + xa_lo)[tile row][ranks] as two bf16 MFMAs per 32 ranks; wave w owns
// columns c0 + 128w .. +128 (8 tiles of 16).  NRS = rank steps of 32.
template <int NRS, class Op, class Xa, class Wait>
__device__ __forceinline__ void expand_mfma(const Op &op, const Tile &h, int c0, const Xa &xs, bool add_inputs,
                            const Wait &wait, char *smem) {
    constexpr int CTB = 8 / NRS;  // column tiles whose B operands are in flight together (8 loads)
    const int lane = lane_id(), w = wave_id();
    const int R = op.R, R2 = 2 * R;
    const int cend = min(c0 + kCW, op.n_out);
    const int sg_lo = op.xslice(c0), ns = op.xslice(cend - 1) - sg_lo + 1;
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);
    const size_t xl_bytes = ((size_t)ns * kTileRows * R2 * 2 + 15) & ~(size_t)15;
    float *ol = reinterpret_cast<float *>(smem + xl_bytes) + w * (kTileRows * kOutStride);
    const int cw0 = c0 + 128 * w;
    const int col_l = lane & 15, kk = (lane >> 4) * 8;

    u32x4_t bo[CTB][NRS];
    mfma_load_b<NRS, CTB>(op, h, bo, 0, -1, cw0, cend, R);
    u32x4_t yv[4];
    prefetch_y(op, h, cw0, cend, add_inputs, yv);
    if (!wait()) return;
    stage_xa(h, xs, sg_lo, ns, R, xl);
    __syncthreads();

    f32x4_t d[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) d[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int sg_w0 = op.xslice(min(cw0, cend - 1)), sg_w1 = op.xslice(min(cw0 + 127, cend - 1));
    const bool straddle = sg_w0 != sg_w1;
    // one pass per xa slice under this wave's columns (almost always one);
    // when they straddle a slice boundary each pass masks the other slice's rows
    for (int sg = sg_w0; cw0 < cend && sg <= sg_w1; ++sg) {
        const uint16_t *xr = xl + ((sg - sg_lo) * kTileRows + col_l) * R2;  // MFMA-B column = tile row
        u32x4_t hv[NRS], lv[NRS];
#pragma unroll
        for (int s = 0; s < NRS; ++s) {
            const int rk = 32 * s + kk;
            hv[s] = rk < R ? lds16(xr + rk) : zero4();
            lv[s] = rk < R ? lds16(xr + R + rk) : zero4();
        }
#pragma unroll
        for (int cb = 0; cb < 8; cb += CTB) {
            if (cb > 0 || straddle) mfma_load_b<NRS, CTB>(op, h, bo, cb, straddle ? sg : -1, cw0, cend, R);
#pragma unroll
            for (int i = 0; i < CTB; ++i) {
#pragma unroll
                for (int s = 0; s < NRS; ++s) {
                    d[cb + i] = mfma_16x16x32(bo[i][s], hv[s], d[cb + i]);
                    d[cb + i] = mfma_16x16x32(bo[i][s], lv[s], d[cb + i]);
                }
            }
        }
    }
    // lane holds D[column cw0 + 16ct + 4*(lane>>4) + q][tile row lane & 15]
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        float *o = ol + col_l * kOutStride + 16 * ct + 4 * (lane >> 4);
        o[0] = d[ct][0];
        o[1] = d[ct][1];
        o[2] = d[ct][2];
        o[3] = d[ct][3];
    }
    __syncthreads();
    store_tile(op, h, ol, cw0, cend, add_inputs, yv);
}

template <int NRS, class Op, class Xa, class Wait>
__device__ __forceinline__ void expand_unit(const Op &op, const Tile &h, bool mf, int c0, const Xa &xs,
                                            bool add_inputs, const Wait &wait, char *smem) {
    if (mf)
        expand_mfma<NRS>(op, h, c0, xs, add_inputs, wait, smem);
    else
        expand_valu(op, h, c0, xs, add_inputs, wait, smem);
}

// ============================================================ kernels
template <int NT, int KC, class Op>
__global__ __launch_bounds__(NT) void shrink_kernel(Op op, const int32_t *tiles, float *xa, int n, int mfma_min) {
    extern __shared__ __align__(16) char smem[];
    __shared__ TileLds tl_sh;
    Tile h;
    const int n_sl = op.n_sh;
    const int t = blockIdx.x / n_sl, sl = blockIdx.x % n_sl;
    if (!load_tile(op, tiles, t, tl_sh, h)) return;
    const bool mf = h.mseg >= mfma_min;
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    float *res = reinterpret_cast<float *>(smem + kTileRows * shrink_xs<KC>() * 2);
    float *red = res + kRRMfma * 16;
    const int R = op.R;
    const float sc = op.scale_of(h.slot);
    const int chunk = mf ? kRRMfma : kRRValu;
    for (int r0 = 0; r0 < R; r0 += chunk) {
        const int cnt = min(chunk, R - r0);
        shrink_compute<NT, KC>(op, h, mf, sl * R + r0, cnt, 0, op.k_in, res, red, xs);
        for (int idx = threadIdx.x; idx < h.m * cnt; idx += NT) {
            const int j = idx / cnt, r = idx % cnt;
            xa[((int64_t)sl * n + h.rows[j]) * R + r0 + r] = sc * res[r * 16 + j];
        }
        __syncthreads();
    }
}

template <int NRS, class Op>
__global__ __launch_bounds__(kBT) void expand_kernel(Op op, const int32_t *tiles, const float *xa, int n, int C,
                                                     int add_inputs, int mfma_min) {
    extern __shared__ __align__(16) char smem[];
    __shared__ TileLds tl_sh;
    Tile h;
    const int t = blockIdx.x / C, cc = blockIdx.x % C;
    if (!load_tile(op, tiles, t, tl_sh, h)) return;
    const bool mf = h.mseg >= mfma_min;
    expand_unit<NRS>(op, h, mf, cc * kCW, XaDirect{xa, n, op.R}, add_inputs != 0, NoWait{}, smem);
}

// ============================================================ host side
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

template <int NT, int KC>
static size_t shrink_lds() {
    return (size_t)kTileRows * shrink_xs<KC>() * 2 +
           (size_t)(kRRMfma * 16 + shrink_red_floats<NT / kWave>()) * sizeof(float);
}

static size_t expand_lds(int n_xa_slices, int R) {
    return align_up((size_t)n_xa_slices * kTileRows * 2 * R * 2, 16) +
           (size_t)4 * kTileRows * kOutStride * sizeof(float);
}

// rank steps of 32 of the MFMA expand
static int nrs_of(int R) { return R <= 32 ? 1 : (R <= 64 ? 2 : 4); }

template <class K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

static DenseOp dense_op(const DenseShape &d) {
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
    return op;
}

hipError_t launch_shrink(const DenseShape &d, const int32_t *tiles, int tile_bound, float *xa, int mfma_min,
                         hipStream_t st) {
    if (tile_bound == 0) return hipSuccess;
    const DenseOp op = dense_op(d);
    const long long units = (long long)tile_bound * d.num_slices;
    if (units >= 512) {  // enough units for two per CU: 4 waves, 512-wide k passes
        const size_t lds = shrink_lds<256, 512>();
        hipLaunchKernelGGL((shrink_kernel<256, 512, DenseOp>), dim3(units), dim3(256), lds, st, op, tiles, xa,
                           d.n, mfma_min);
    } else {
        const size_t lds = shrink_lds<512, 2048>();
        allow_lds(shrink_kernel<512, 2048, DenseOp>, lds);
        hipLaunchKernelGGL((shrink_kernel<512, 2048, DenseOp>), dim3(units), dim3(512), lds, st, op, tiles, xa,
                           d.n, mfma_min);
    }
    return hipGetLastError();
}

template <int NRS>
static hipError_t launch_expand_nrs(const DenseOp &op, const float *xa, const int32_t *tiles, int tile_bound,
                                    int n, int add_inputs, int mfma_min, size_t lds, hipStream_t st) {
    const int C = (op.n_out + kCW - 1) / kCW;
    allow_lds(expand_kernel<NRS, DenseOp>, lds);
    hipLaunchKernelGGL((expand_kernel<NRS, DenseOp>), dim3(tile_bound * C), dim3(kBT), lds, st, op, tiles, xa, n,
                       C, add_inputs, mfma_min);
    return hipGetLastError();
}

hipError_t launch_expand(const DenseShape &d, const float *xa, const int32_t *tiles, int tile_bound,
                         int add_inputs, int mfma_min, hipStream_t st) {
    if (tile_bound == 0) return hipSuccess;
    const DenseOp op = dense_op(d);
    const size_t lds = expand_lds(d.num_slices, d.R);
    switch (nrs_of(d.R)) {
    case 1: return launch_expand_nrs<1>(op, xa, tiles, tile_bound, d.n, add_inputs, mfma_min, lds, st);
    case 2: return launch_expand_nrs<2>(op, xa, tiles, tile_bound, d.n, add_inputs, mfma_min, lds, st);
    default: return launch_expand_nrs<4>(op, xa, tiles, tile_bound, d.n, add_inputs, mfma_min, lds, st);
    }
}

}  // namespace tl
