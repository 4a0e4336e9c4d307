// delta.hip -- shrink, expand and fused routed LoRA delta for gfx950.
//
// Semantics (vLLM punica_base.py, add_shrink / add_expand / add_lora_linear;
// metrale lora_delta docs, apply_lora_bgmv and LoraPair; FlashInfer
// bgmv_moe_gemm1_lora_delta): rows of one adapter slot form a segment; the
// shrink gives xa = scale * x @ A^T in fp32, the expand adds xa @ B^T to the
// output window and rounds once to bf16.
//
// Work units.  The metadata cuts every segment into tiles of at most 16 rows
// (one 128-byte record each: slot, first sorted position, row count, segment
// size, row ids).  A workgroup (4 waves) takes one unit:
//   shrink unit  (tile, k piece): every rank row of the adapter over a k range
//   expand unit  (tile, 512-column chunk): every row of the tile
// Segments with at least `mfma_min` rows (16 by default) run on
// v_mfma_f32_16x16x32_bf16; shorter ones on the vector ALU with
// v_dot2c_f32_bf16.  bf16 products are exact in fp32 on both paths.  The
// expand keeps xa's precision by splitting it into two bf16 terms
// (hi = bf16(xa), lo = bf16(xa - hi)) that both multiply B, so no bf16
// rounding of xa reaches the result beyond ~2^-16 relative.
//
// The fused kernel runs all shrink units (lower workgroup ids) and all expand
// units in one launch.  A shrink unit stores an fp32 partial for its k piece
// and bumps its tile's counter (agent-scope release); an expand unit waits on
// that counter (agent-scope acquire) and sums the P partials in a fixed
// order, so results are bitwise reproducible.  Workgroups are dispatched in
// id order, so every awaited shrink unit is already running or done; the wait
// is bounded anyway and reports a flag instead of hanging.
#include "common.h"
#include "kernels.h"

namespace tl {

constexpr int kBT = 256;        // threads per compute workgroup
constexpr int kCW = 512;        // expand columns per unit
constexpr int kRRChunk = 256;   // shrink rank rows per pass
constexpr int kRedStride = 48 * 16;  // per-wave partial block when waves split k
constexpr int kOutStride = 132;      // padded fp32 row stride of the MFMA output tile
constexpr int kSpinLimit = 1 << 24;

// ============================================================ addressing
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

    __device__ const uint16_t *xrow(int row) const { return x + (int64_t)row * ldx; }
    // rank row rr = l*R + r of slot s: a_pool[s][l][r][:]
    __device__ const uint16_t *arow(int slot, int rr) const {
        return a_pool + ((int64_t)slot * n_sh * R + rr) * k_in;
    }
    __device__ int xslice(int c) const {
        int l = 0;
        while (l + 1 < n_sl && c >= off[l + 1]) ++l;
        return l;
    }
    __device__ const uint16_t *brow(int slot, int c) const {
        return b_pool + ((int64_t)slot * n_out + c) * R;
    }
    __device__ uint16_t *yrow(int row) const { return y + (int64_t)row * ldy + col0; }
    __device__ float scale_of(int slot) const { return scale[slot]; }
};

// Routed MoE gemm1: key = l*E + e, rows are (token, slot) pairs.
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

    __device__ const uint16_t *xrow(int pair) const { return x + (int64_t)(pair / top_k) * ldx; }
    __device__ const uint16_t *arow(int key, int rr) const {
        const int l = key / E, e = key - l * E;
        const int sg = rr / R, r = rr - sg * R;
        const uint16_t *base = reinterpret_cast<const uint16_t *>(wa[shared ? e : sg * E + e]);
        return base + (int64_t)l * lsa + (int64_t)r * k_in;
    }
    __device__ int xslice(int c) const { return shared ? 0 : (c >= inter ? 1 : 0); }
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
};

// ============================================================ tile header
struct UnitHdr {
    int m, slot, pos0, mseg, flag;
    int rows[kTileRows];
    const uint16_t *xrow[kTileRows];
};

template <class Op>
__device__ bool load_tile(const Op &op, const int32_t *tiles, int t, UnitHdr &h) {
    const int tid = threadIdx.x;
    const int32_t *rec = tiles + (int64_t)t * kTileWords;
    if (tid == 0) {
        h.m = rec[kRecRows];
        h.slot = rec[kRecSlot];
        h.pos0 = rec[kRecPos];
        h.mseg = rec[kRecSegRows];
        h.flag = 0;
    }
    __syncthreads();
    const int m = h.m;
    if (m == 0) return false;
    if (tid < kTileRows) {
        const int row = tid < m ? rec[kRecRowIds + tid] : 0;
        h.rows[tid] = row;
        h.xrow[tid] = tid < m ? op.xrow(row) : nullptr;
    }
    __syncthreads();
    return true;
}

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// How the 4 waves share a unit: GW waves split the rank-row groups, KW = 4/GW
// split the k range (their partials are summed in wave order).
__device__ __forceinline__ void wave_split(int groups, int &GW, int &KW) {
    GW = groups >= 4 ? 4 : (groups >= 2 ? 2 : 1);
    KW = 4 / GW;
}

// ============================================================ shrink
// res[rl*16 + j] = sum_{k in [k0,k1)} x[row_j][k] * A[slot][rr0 + rl][k], rl < n_rr.
template <class Op>
__device__ void shrink_mfma(const Op &op, const UnitHdr &h, int rr0, int n_rr, int k0, int k1, float *res,
                            float *red) {
    const int lane = lane_id(), w = wave_id();
    const int groups = (n_rr + 15) >> 4;
    int GW, KW;
    wave_split(groups, GW, KW);
    const int gw = w % GW, kw = w / GW;
    const int per = ((k1 - k0 + KW * 32 - 1) / (KW * 32)) * 32;
    const int ka = k0 + kw * per, kb = min(k1, ka + per);
    const int col = lane & 15, kk = (lane >> 4) * 8;
    const uint16_t *xr = h.xrow[col];  // MFMA-A row = tile row (null past m)
    float *dst = KW == 1 ? res : red + kw * kRedStride;
    for (int g = gw; g < groups; g += GW) {
        const int rl = 16 * g + col;  // MFMA-B column = rank row
        const uint16_t *ap = rl < n_rr ? op.arow(h.slot, rr0 + rl) : nullptr;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};

        for (int k = ka; k < kb; k += 32) {
            const int kx = k + kk;
            const bool in = kx < kb;
            const u32x4_t xo = (xr && in) ? ld16(xr + kx) : zero4();
            const u32x4_t ao = (ap && in) ? ld16_stream(ap + kx) : zero4();
            acc = mfma_16x16x32(xo, ao, acc);
        }
        if (rl < n_rr) {
            const int j0 = (lane >> 4) * 4;
            dst[rl * 16 + j0 + 0] = acc[0];
            dst[rl * 16 + j0 + 1] = acc[1];
            dst[rl * 16 + j0 + 2] = acc[2];
            dst[rl * 16 + j0 + 3] = acc[3];
        }
    }
    __syncthreads();
    if (KW > 1) {
        for (int idx = threadIdx.x; idx < n_rr * 16; idx += kBT) {
            float s = red[idx];
            for (int q = 1; q < KW; ++q) s += red[q * kRedStride + idx];
            res[idx] = s;
        }
        __syncthreads();
    }
}

template <class Op>
__device__ void shrink_valu(const Op &op, const UnitHdr &h, int rr0, int n_rr, int k0, int k1, float *res,
                            float *red) {
    const int lane = lane_id(), w = wave_id();
    const int rsub = lane >> 3, kl = lane & 7;
    const int groups = n_rr >> 3;
    int GW, KW;
    wave_split(groups, GW, KW);
    const int gw = w % GW, kw = w / GW;
    const int per = ((k1 - k0 + KW * 64 - 1) / (KW * 64)) * 64;
    const int ka = k0 + kw * per, kb = min(k1, ka + per);
    const int m = h.m;
    float *dst = KW == 1 ? res : red + kw * kRedStride;
    for (int q = gw; q < groups; q += GW) {
        const int rl = 8 * q + rsub;
        const uint16_t *ap = op.arow(h.slot, rr0 + rl);
        float acc[kTileRows];
#pragma unroll
        for (int j = 0; j < kTileRows; ++j) acc[j] = 0.f;
        for (int k = ka + 8 * kl; k < kb; k += 64) {
            const u32x4_t av = ld16_stream(ap + k);
#pragma unroll
            for (int j = 0; j < kTileRows; ++j)
                if (j < m) acc[j] = dot8(av, ld16(h.xrow[j] + k), acc[j]);
        }
#pragma unroll
        for (int j = 0; j < kTileRows; ++j) {
            if (j < m) {
                float v = acc[j];
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 4);
                if (kl == 0) dst[rl * 16 + j] = v;
            }
        }
    }
    __syncthreads();
    if (KW > 1) {
        for (int idx = threadIdx.x; idx < n_rr * 16; idx += kBT) {
            float s = red[idx];
            for (int q = 1; q < KW; ++q) s += red[q * kRedStride + idx];
            res[idx] = s;
        }
        __syncthreads();
    }
}

template <class Op>
__device__ __forceinline__ void shrink_compute(const Op &op, const UnitHdr &h, bool mf, int rr0, int n_rr,
                                               int k0, int k1, float *res, float *red) {
    if (mf)
        shrink_mfma(op, h, rr0, n_rr, k0, k1, res, red);
    else
        shrink_valu(op, h, rr0, n_rr, k0, k1, res, red);
}

// ============================================================ expand
// xa sources: get(slice, row id, sorted position, rank) -> fp32 xa
struct XaDirect {  // caller's xa[slice][n][R], already scaled
    const float *xa;
    int n, R;
    __device__ float get(int sg, int row, int, int r) const { return xa[((int64_t)sg * n + row) * R + r]; }
};
struct XaPartials {  // fused workspace part[p][pos][n_rr], scaled here
    const float *part;
    int n, P, n_rr, R;
    float scale;
    __device__ float get(int sg, int, int pos, int r) const {
        float s = 0.f;
        for (int p = 0; p < P; ++p) s += part[((int64_t)p * n + pos) * n_rr + sg * R + r];
        return scale * s;
    }
};

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

template <class Op>
__device__ __forceinline__ void store_row8(const Op &op, uint16_t *yp, const float *v, bool add_inputs) {
    float o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = v[q];
    if (add_inputs) {
        const u32x4_t yv = ld16(yp);
        o[0] += bf_lo(yv.x);
        o[1] += bf_hi(yv.x);
        o[2] += bf_lo(yv.y);
        o[3] += bf_hi(yv.y);
        o[4] += bf_lo(yv.z);
        o[5] += bf_hi(yv.z);
        o[6] += bf_lo(yv.w);
        o[7] += bf_hi(yv.w);
    }
    st16(yp, u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                     pack_bf16x2(o[6], o[7])});
}

template <class Op, class Xa>
__device__ void expand_unit(const Op &op, const UnitHdr &h, bool mf, int c0, const Xa &xs, bool add_inputs,
                            char *smem) {
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int R = op.R, R2 = 2 * R;
    const int cend = min(c0 + kCW, op.n_out);
    const int sg_lo = op.xslice(c0), sg_hi = op.xslice(cend - 1);
    const int ns = sg_hi - sg_lo + 1;
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);  // [ns][16][hi R | lo R]
    for (int idx = tid; idx < ns * kTileRows * R; idx += kBT) {
        const int r = idx % R, j = (idx / R) % kTileRows, sl = idx / (kTileRows * R);
        const float v = j < h.m ? xs.get(sg_lo + sl, h.rows[j], h.pos0 + j, r) : 0.f;
        const float hi = bf16_round(v);
        uint16_t *d = xl + (sl * kTileRows + j) * R2;
        d[r] = bf16_bits(hi);
        d[R + r] = bf16_bits(v - hi);
    }
    __syncthreads();

    if (!mf) {
        // vector ALU: lane -> 8 columns, wave w -> rows w, w+4, w+8, w+12
        const int c = c0 + 8 * lane;
        if (c < cend) {
            const int sl = op.xslice(c) - sg_lo;
            const uint16_t *b = op.brow(h.slot, c);
            float acc[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
            for (int r8 = 0; r8 < R; r8 += 8) {
                u32x4_t bv[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) bv[q] = ld16_stream(b + q * R + r8);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = w + 4 * i;
                    if (j < h.m) {
                        const uint16_t *xr = xl + (sl * kTileRows + j) * R2;
                        const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(xr + r8);
                        const u32x4_t lv = *reinterpret_cast<const u32x4_t *>(xr + R + r8);
#pragma unroll
                        for (int q = 0; q < 8; ++q) acc[i][q] = dot8(bv[q], lv, dot8(bv[q], hv, acc[i][q]));
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = w + 4 * i;
                if (j < h.m) store_row8(op, op.yrow(h.rows[j]) + c, acc[i], add_inputs);
            }
        }
        return;
    }

    // MFMA: D[col][row] = B[col][hi|lo ranks] . [xa_hi | xa_lo][row]; wave w -> 128 columns
    const size_t xl_bytes = ((size_t)ns * kTileRows * R2 * 2 + 15) & ~(size_t)15;
    float *ol = reinterpret_cast<float *>(smem + xl_bytes) + w * (kTileRows * kOutStride);
    const int cw0 = c0 + 128 * w;
    const int col_l = lane & 15, kk = (lane >> 4) * 8;
    for (int ct = 0; ct < 8; ++ct) {
        const int cb = cw0 + 16 * ct;
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
        if (cb < cend) {
            const int c = cb + col_l;
            const bool cok = c < cend;
            const int sgc = cok ? op.xslice(c) : -1;
            const int s_first = op.xslice(cb), s_last = op.xslice(min(cb + 15, cend - 1));
            const uint16_t *b = cok ? op.brow(h.slot, c) : nullptr;
            for (int sg = s_first; sg <= s_last; ++sg) {
                const bool use = cok && sgc == sg;
                const uint16_t *xr = xl + ((sg - sg_lo) * kTileRows + col_l) * R2;  // MFMA-B column = tile row
                for (int kb = 0; kb < R2; kb += 32) {
                    const int kap = kb + kk;
                    const bool kin = kap < R2;
                    const int r = kap < R ? kap : kap - R;
                    const u32x4_t ao = (use && kin) ? ld16_stream(b + r) : zero4();
                    const u32x4_t bo = kin ? *reinterpret_cast<const u32x4_t *>(xr + kap) : zero4();
                    d = mfma_16x16x32(ao, bo, d);
                }
            }
        }
        // lane holds D[column cb + 4*(lane>>4) + i][tile row lane & 15]
        float *o = ol + col_l * kOutStride + 16 * ct + 4 * (lane >> 4);
        o[0] = d[0];
        o[1] = d[1];
        o[2] = d[2];
        o[3] = d[3];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int j = 4 * p + (lane >> 4);
        const int c = cw0 + 8 * (lane & 15);
        if (j < h.m && c < cend) {
            const float *src = ol + j * kOutStride + 8 * (lane & 15);
            store_row8(op, op.yrow(h.rows[j]) + c, src, add_inputs);
        }
    }
}

// ============================================================ kernels
template <class Op>
__global__ __launch_bounds__(kBT) void shrink_kernel(Op op, const int32_t *tiles, float *xa, int n, int mfma_min) {
    extern __shared__ __align__(16) char smem[];
    __shared__ UnitHdr h;
    const int n_sl = op.n_sh;
    const int t = blockIdx.x / n_sl, sl = blockIdx.x % n_sl;
    if (!load_tile(op, tiles, t, h)) return;
    const bool mf = h.mseg >= mfma_min;
    float *res = reinterpret_cast<float *>(smem);
    float *red = res + kRRChunk * 16;
    const int R = op.R;
    shrink_compute(op, h, mf, sl * R, R, 0, op.k_in, res, red);
    const float sc = op.scale_of(h.slot);
    for (int idx = threadIdx.x; idx < h.m * R; idx += kBT) {
        const int j = idx / R, r = idx % R;
        xa[((int64_t)sl * n + h.rows[j]) * R + r] = sc * res[r * 16 + j];
    }
}

template <class Op>
__global__ __launch_bounds__(kBT) void expand_kernel(Op op, const int32_t *tiles, const float *xa, int n, int C,
                                                     int add_inputs, int mfma_min) {
    extern __shared__ __align__(16) char smem[];
    __shared__ UnitHdr h;
    const int t = blockIdx.x / C, cc = blockIdx.x % C;
    if (!load_tile(op, tiles, t, h)) return;
    const bool mf = h.mseg >= mfma_min;
    expand_unit(op, h, mf, cc * kCW, XaDirect{xa, n, op.R}, add_inputs != 0, smem);
}

struct ZeroFill {  // MoE: rows of pairs without a valid (adapter, expert) are zeroed
    const int32_t *topk;
    const int32_t *lora;
    int top_k, E, L, n_pairs;
};

template <class Op>
__global__ __launch_bounds__(kBT) void fused_kernel(Op op, const int32_t *tiles, int tile_bound, int P, int C,
                                                    int n_pos, float *part, int *ctl, int *ctr, int *done,
                                                    int mfma_min, int add_inputs, ZeroFill zf) {
    extern __shared__ __align__(16) char smem[];
    __shared__ UnitHdr h;
    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    const int n_shr = tile_bound * P, n_exp = tile_bound * C;
    const int n_rr = op.n_sh * op.R;
    if (bid < n_shr) {
        const int t = bid / P, p = bid % P;
        if (!load_tile(op, tiles, t, h)) return;
        const bool mf = h.mseg >= mfma_min;
        const int KP = (((op.k_in + P - 1) / P + 63) / 64) * 64;
        const int k0 = min(op.k_in, p * KP), k1 = min(op.k_in, k0 + KP);
        float *res = reinterpret_cast<float *>(smem);
        float *red = res + kRRChunk * 16;
        for (int rr0 = 0; rr0 < n_rr; rr0 += kRRChunk) {
            const int cnt = min(kRRChunk, n_rr - rr0);
            shrink_compute(op, h, mf, rr0, cnt, k0, k1, res, red);
            for (int idx = tid; idx < h.m * cnt; idx += kBT) {
                const int j = idx / cnt, rl = idx % cnt;
                part[((int64_t)p * n_pos + h.pos0 + j) * n_rr + rr0 + rl] = res[rl * 16 + j];
            }
            __syncthreads();
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) atomic_add_release(&ctr[t], 1);
        return;
    }
    if (bid < n_shr + n_exp) {
        const int e = bid - n_shr;
        const int t = e / C, cc = e % C;
        if (!load_tile(op, tiles, t, h)) return;
        if (tid == 0) {
            int spins = 0;
            while (load_acquire(&ctr[t]) < P) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinLimit) {
                    atomicExch(&ctl[0], 1);
                    h.flag = 1;
                    break;
                }
            }
            if (!h.flag && atomicAdd(&done[t], 1) == C - 1) {
                store_relaxed(&ctr[t], 0);
                store_relaxed(&done[t], 0);
            }
        }
        __syncthreads();
        if (h.flag) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool mf = h.mseg >= mfma_min;
        expand_unit(op, h, mf, cc * kCW, XaPartials{part, n_pos, P, n_rr, op.R, op.scale_of(h.slot)},
                    add_inputs != 0, smem);
        return;
    }
    // zero rows of pairs that get no delta (MoE only)
    const int u = bid - n_shr - n_exp;
    const int pair = u * 16 + (tid >> 4);
    if (pair >= zf.n_pairs) return;
    const int l = zf.lora[pair / zf.top_k], ex = zf.topk[pair];
    if (l >= 0 && l < zf.L && ex >= 0 && ex < zf.E) return;
    uint16_t *o = op.yrow(pair);
    for (int c = (tid & 15) * 8; c < op.n_out; c += 128) st16(o + c, zero4());
}

// ============================================================ host side
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static size_t shrink_lds() { return (size_t)(kRRChunk * 16 + 4 * kRedStride) * sizeof(float); }

static size_t expand_lds(int n_xa_slices, int R) {
    return align_up((size_t)n_xa_slices * kTileRows * 2 * R * 2, 16) +
           (size_t)4 * kTileRows * kOutStride * sizeof(float);
}

static int tile_bound_of(int n, int S) {
    if (n <= 0) return 0;
    const long long a = (n + kTileRows - 1) / kTileRows + (long long)(n < S ? n : S);
    return (int)(a < n ? a : n);
}

FusedPlan fused_plan(int n, int num_slots, int n_sh, int R, int k_in, int n_out) {
    FusedPlan p{};
    p.tile_bound = tile_bound_of(n, num_slots);
    p.P = 1;
    const int target_units = 512;  // about two units per CU of the shrink over the k dimension
    while (p.tile_bound > 0 && (long long)p.P * 2 * p.tile_bound <= target_units && p.P * 2 <= k_in / 256)
        p.P *= 2;
    p.C = (n_out + kCW - 1) / kCW;
    p.ctr_bytes = align_up(64 + (size_t)2 * p.tile_bound * sizeof(int), 256);
    p.part_bytes = align_up((size_t)p.P * n * n_sh * R * sizeof(float), 256);
    p.total_bytes = p.ctr_bytes + p.part_bytes;
    return p;
}

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
    const size_t lds = shrink_lds();
    hipLaunchKernelGGL(shrink_kernel<DenseOp>, dim3(tile_bound * d.num_slices), dim3(kBT), lds, st, op, tiles, xa,
                       d.n, mfma_min);
    return hipGetLastError();
}

hipError_t launch_expand(const DenseShape &d, const float *xa, const int32_t *tiles, int tile_bound,
                         int add_inputs, int mfma_min, hipStream_t st) {
    if (tile_bound == 0) return hipSuccess;
    const DenseOp op = dense_op(d);
    const int C = (op.n_out + kCW - 1) / kCW;
    const size_t lds = expand_lds(d.num_slices, d.R);
    allow_lds(expand_kernel<DenseOp>, lds);
    hipLaunchKernelGGL(expand_kernel<DenseOp>, dim3(tile_bound * C), dim3(kBT), lds, st, op, tiles, xa, d.n, C,
                       add_inputs, mfma_min);
    return hipGetLastError();
}

template <class Op>
static hipError_t launch_fused_op(const Op &op, int n_pos, int n_xa_slices, const int32_t *tiles,
                                  const FusedPlan &plan, void *ws, int mfma_min, int add_inputs, ZeroFill zf,
                                  int zero_units, hipStream_t st) {
    char *w = static_cast<char *>(ws);
    int *ctl = reinterpret_cast<int *>(w);
    int *ctr = ctl + 16;
    int *done = ctr + plan.tile_bound;
    float *part = reinterpret_cast<float *>(w + plan.ctr_bytes);
    const size_t lds = shrink_lds() > expand_lds(n_xa_slices, op.R) ? shrink_lds() : expand_lds(n_xa_slices, op.R);
    allow_lds(fused_kernel<Op>, lds);
    const long long grid = (long long)plan.tile_bound * (plan.P + plan.C) + zero_units;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(fused_kernel<Op>, dim3((unsigned)grid), dim3(kBT), lds, st, op, tiles, plan.tile_bound,
                       plan.P, plan.C, n_pos, part, ctl, ctr, done, mfma_min, add_inputs, zf);
    return hipGetLastError();
}

hipError_t launch_fused(const DenseShape &d, const int32_t *tiles, const FusedPlan &plan, void *ws, int mfma_min,
                        hipStream_t st) {
    const DenseOp op = dense_op(d);
    return launch_fused_op(op, d.n, d.num_slices, tiles, plan, ws, mfma_min, 1, ZeroFill{nullptr, nullptr, 1, 1, 1, 0},
                           0, st);
}

hipError_t launch_moe_delta(const MoeShape &m, const int32_t *tiles, const FusedPlan &plan, void *ws,
                            int mfma_min, hipStream_t st) {
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
    return launch_fused_op(op, n_pairs, op.n_sh, tiles, plan, ws, mfma_min, 0, zf, zero_units, st);
}

}  // namespace tl
