/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the routed LoRA
 * delta.  TEST INFRASTRUCTURE ONLY: it is called by tests/, by the package's
 * smoke check and by the benchmark's CPU-baseline leg, never by the product
 * path.  It shares no code, header, table or helper with the HIP library.
 *
 * Every floating-point input (bf16 bit patterns, float32 scales, float32 xa)
 * is widened exactly to double and every sum runs in double, in ascending
 * index order.  No blocking, no fusion, no reordering beyond the definitions.
 *
 * Sources of the definitions (web pages, cited by title and section):
 *  - vLLM "punica_base.py" (PunicaWrapperBase): add_shrink and add_expand
 *    semantics docstrings; add_lora_linear semantics; prefill_metadata
 *    ("-1 means no lora"; lora indices grouped into segments).
 *  - metrale docs, module lora_delta: apply_lora_bgmv (routed delta, negative
 *    slot gets no delta), LoraPair (A is [max_rank, k_in], B is [n_out,
 *    max_rank], row-major, scale applied in the fold), module invariants
 *    (both stages contract at the padded max_rank; pad rows/cols are zero).
 *  - FlashInfer docs, flashinfer.fused_moe.bgmv_moe_gemm1_lora_delta: the
 *    per-(token, slot) gate/up formula, the shared-A form, the w_ptr tables
 *    and lora_stride, lora_ids = -1 meaning no adapter.
 *  - vLLM "punica_base.py", PunicaWrapperBase.add_lora_w2: the w2 LoRA
 *    applied in place to the per-(token, slot) down-projection output
 *    (intermediate_cache3) before moe_sum, routed as add_lora_w13.
 *  - metrale source "lora/expert_apply.rs": expert_delta_workitems (one
 *    work item per adapted expert with a non-empty block of the
 *    expert-sorted rows, from the expert_offsets prefix sum),
 *    apply_expert_lora_sorted and apply_router_lora (the delta of one pair
 *    folded over a contiguous block of rows, in place).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): a slot >= num_slots is excluded and counted as invalid; segments
 * are runs of equal slot after sorting rows by (slot, row); a MoE pair whose
 * adapter id is >= L or whose expert id is outside [0, E) yields a zero row
 * and is counted as invalid, a negative adapter id yields a zero row and is
 * not counted.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -fPIC -shared oracle.c -o liboracle.so
 * (no fast-math: the fp64 sums must not be reassociated).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * O-meta.  Row i is active when 0 <= slot[i] < num_slots, invalid when
 * slot[i] >= num_slots, and unadapted when slot[i] < 0.  Active rows are
 * listed in ascending (slot, row) order; a segment is a maximal run of one
 * slot in that list.
 *   sorted_rows[0 .. n_active)       the listed rows
 *   seg_offsets[0 .. n_seg]          start of each segment, then n_active
 *   seg_slot[0 .. n_seg)             the slot of each segment (ascending)
 *   counts = {n_active, n_seg, n_invalid, n_seg_with_at_least_16_rows}
 * Written as the plainest possible definition: one pass over all rows per
 * slot value, which is stable by construction.
 * ------------------------------------------------------------------------ */
void oracle_meta_build(const int32_t *slot, int32_t n, int32_t num_slots,
                       int32_t *sorted_rows, int32_t *seg_offsets,
                       int32_t *seg_slot, int32_t *counts)
{
    int32_t pos = 0, nseg = 0, nlong = 0, ninvalid = 0;
    for (int32_t i = 0; i < n; ++i)
        if (slot[i] >= num_slots)
            ++ninvalid;
    for (int32_t s = 0; s < num_slots; ++s) {
        int32_t start = pos;
        for (int32_t i = 0; i < n; ++i)
            if (slot[i] == s)
                sorted_rows[pos++] = i;
        if (pos > start) {
            seg_offsets[nseg] = start;
            seg_slot[nseg] = s;
            if (pos - start >= 16)
                ++nlong;
            ++nseg;
        }
    }
    seg_offsets[nseg] = pos;
    counts[0] = pos;
    counts[1] = nseg;
    counts[2] = ninvalid;
    counts[3] = nlong;
}

/* ------------------------------------------------------------------------
 * MoE pair keys.  Pair p = t*top_k + j routes token t to expert
 * e = topk_ids[p] under adapter l = lora_ids[t].  key = l*E + e for a valid
 * pair, -1 when l < 0 (no adapter), and L*E (an invalid slot, counted by
 * O-meta) when l >= L or e is outside [0, E).  O-meta over these keys with
 * num_slots = L*E gives the pair segments, one per (adapter, expert).
 * ------------------------------------------------------------------------ */
void oracle_moe_keys(const int32_t *topk_ids, int32_t T, int32_t top_k,
                     const int32_t *lora_ids, int32_t num_experts, int32_t num_loras,
                     int32_t *key)
{
    const int32_t S = num_loras * num_experts;
    for (int32_t t = 0; t < T; ++t) {
        const int32_t l = lora_ids[t];
        for (int32_t j = 0; j < top_k; ++j) {
            const int32_t e = topk_ids[(int64_t)t * top_k + j];
            int32_t k;
            if (l < 0)
                k = -1;
            else if (l >= num_loras || e < 0 || e >= num_experts)
                k = S;
            else
                k = l * num_experts + e;
            key[(int64_t)t * top_k + j] = k;
        }
    }
}

/* ------------------------------------------------------------------------
 * O-shrink, evaluated at the listed rows.  For listed row i with active slot
 * s, every slice l and every rank r:
 *     xa[q][l][r] = scale[s] * sum_{k ascending} x[i][k] * A[s][l][r][k]
 * with A_pool laid out [num_slots][num_slices][max_rank][k_in].  The output
 * of an inactive or invalid listed row is left unwritten.
 * ------------------------------------------------------------------------ */
void oracle_shrink_rows(const uint16_t *x, int64_t ldx, int32_t k_in,
                        const uint16_t *a_pool, const float *scale,
                        int32_t num_slots, int32_t num_slices, int32_t max_rank,
                        const int32_t *slot, const int32_t *rows, int32_t nr,
                        double *xa_out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < nr; ++q) {
        const int32_t i = rows[q];
        const int32_t s = slot[i];
        if (s < 0 || s >= num_slots)
            continue;
        for (int32_t l = 0; l < num_slices; ++l)
            for (int32_t r = 0; r < max_rank; ++r) {
                const uint16_t *a = a_pool +
                    (((int64_t)s * num_slices + l) * max_rank + r) * (int64_t)k_in;
                double acc = 0.0;
                for (int32_t k = 0; k < k_in; ++k)
                    acc += bf(x[(int64_t)i * ldx + k]) * bf(a[k]);
                xa_out[((int64_t)q * num_slices + l) * max_rank + r] =
                    (double)scale[s] * acc;
            }
    }
}

/* ------------------------------------------------------------------------
 * O-expand, evaluated at the listed rows.  y_out row q starts as a copy of
 * y_in row rows[q].  For an active row with slot s, slice l of width w_l at
 * offset off_l = w_0 + ... + w_{l-1}, and column c < w_l:
 *     d   = sum_{r ascending} xa[q][l][r] * B[s][off_l + c][r]
 *     col = offset_start + off_l + c
 *     y_out[q][col] = (add_inputs ? y_in[i][col] : 0) + d
 * with B_pool laid out [num_slots][N][max_rank], N = sum of slice widths.
 * Every other element of the row keeps its input value.
 * ------------------------------------------------------------------------ */
void oracle_expand_rows(const double *xa_rows, const uint16_t *b_pool,
                        int32_t num_slots, int32_t num_slices,
                        const int32_t *slice_sizes, int32_t max_rank,
                        const int32_t *slot, const int32_t *rows, int32_t nr,
                        const uint16_t *y_in, int64_t ldy, int32_t offset_start,
                        int32_t add_inputs, double *y_out)
{
    int64_t n_out = 0;
    for (int32_t l = 0; l < num_slices; ++l)
        n_out += slice_sizes[l];
    #pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < nr; ++q) {
        const int32_t i = rows[q];
        const int32_t s = slot[i];
        double *yo = y_out + (int64_t)q * ldy;
        const uint16_t *yi = y_in + (int64_t)i * ldy;
        for (int64_t c = 0; c < ldy; ++c)
            yo[c] = bf(yi[c]);
        if (s < 0 || s >= num_slots)
            continue;
        int64_t off = 0;
        for (int32_t l = 0; l < num_slices; ++l) {
            const double *u = xa_rows + ((int64_t)q * num_slices + l) * max_rank;
            for (int64_t c = 0; c < slice_sizes[l]; ++c) {
                const uint16_t *b = b_pool + ((int64_t)s * n_out + off + c) * max_rank;
                double d = 0.0;
                for (int32_t r = 0; r < max_rank; ++r)
                    d += u[r] * bf(b[r]);
                const int64_t col = offset_start + off + c;
                yo[col] = (add_inputs ? bf(yi[col]) : 0.0) + d;
            }
            off += slice_sizes[l];
        }
    }
}

/* ------------------------------------------------------------------------
 * O-moe, evaluated at the listed pairs p = t*top_k + j.  With l = lora_ids[t]
 * and e = topk_ids[p]:
 *   l < 0, l >= L, e < 0 or e >= E:  out[q][:] = 0
 *   regular (shared_a == 0): for slice sigma in {gate = 0, up = 1}
 *       A_sigma = w_ptr_a[sigma*E + e] + l*lora_stride_a   ([rank][H])
 *       B_sigma = w_ptr_b[sigma*E + e] + l*lora_stride_b   ([I][rank])
 *       u[r]    = sum_k A_sigma[r][k] * x[t][k]
 *       out[q][sigma*I + c] = scale * sum_r B_sigma[c][r] * u[r]
 *   shared (shared_a != 0):
 *       A = w_ptr_a[e] + l*lora_stride_a ([rank][H]),
 *       B = w_ptr_b[e] + l*lora_stride_b ([2I][rank], gate rows then up rows)
 *       out[q][c] = scale * sum_r B[c][r] * (sum_k A[r][k] * x[t][k]),  c < 2I
 * The pointer tables hold host addresses of bf16 matrices here; strides are
 * in elements.
 * ------------------------------------------------------------------------ */
void oracle_moe_gemm1_pairs(const uint16_t *x, int64_t ldx, int32_t H,
                            const int64_t *w_ptr_a, int64_t lora_stride_a,
                            const int64_t *w_ptr_b, int64_t lora_stride_b,
                            int32_t shared_a, const int32_t *topk_ids, int32_t top_k,
                            const int32_t *lora_ids, int32_t num_experts,
                            int32_t num_loras, int32_t rank, int32_t inter,
                            double scale, const int32_t *pairs, int32_t np,
                            double *out)
{
    const int64_t width = 2 * (int64_t)inter;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < np; ++q) {
        const int32_t p = pairs[q];
        const int32_t t = p / top_k;
        const int32_t l = lora_ids[t];
        const int32_t e = topk_ids[p];
        double *o = out + (int64_t)q * width;
        for (int64_t c = 0; c < width; ++c)
            o[c] = 0.0;
        if (l < 0 || l >= num_loras || e < 0 || e >= num_experts)
            continue;
        const uint16_t *xt = x + (int64_t)t * ldx;
        double u[256];
        if (!shared_a) {
            for (int32_t sigma = 0; sigma < 2; ++sigma) {
                const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[sigma * num_experts + e]
                                    + (int64_t)l * lora_stride_a;
                const uint16_t *B = (const uint16_t *)(intptr_t)w_ptr_b[sigma * num_experts + e]
                                    + (int64_t)l * lora_stride_b;
                for (int32_t r = 0; r < rank; ++r) {
                    double acc = 0.0;
                    for (int32_t k = 0; k < H; ++k)
                        acc += bf(A[(int64_t)r * H + k]) * bf(xt[k]);
                    u[r] = acc;
                }
                for (int32_t c = 0; c < inter; ++c) {
                    double d = 0.0;
                    for (int32_t r = 0; r < rank; ++r)
                        d += bf(B[(int64_t)c * rank + r]) * u[r];
                    o[(int64_t)sigma * inter + c] = scale * d;
                }
            }
        } else {
            const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[e] + (int64_t)l * lora_stride_a;
            const uint16_t *B = (const uint16_t *)(intptr_t)w_ptr_b[e] + (int64_t)l * lora_stride_b;
            for (int32_t r = 0; r < rank; ++r) {
                double acc = 0.0;
                for (int32_t k = 0; k < H; ++k)
                    acc += bf(A[(int64_t)r * H + k]) * bf(xt[k]);
                u[r] = acc;
            }
            for (int64_t c = 0; c < width; ++c) {
                double d = 0.0;
                for (int32_t r = 0; r < rank; ++r)
                    d += bf(B[c * rank + r]) * u[r];
                o[c] = scale * d;
            }
        }
    }
}

/* ------------------------------------------------------------------------
 * O-moe-w2, evaluated at the listed pairs p = t*top_k + j.  With l =
 * lora_ids[t], e = topk_ids[p] and w = topk_weights[p] (1 when no weights
 * are given):
 *   l < 0, l >= L, e < 0 or e >= E:  out[q][:] = y[p][:]
 *   otherwise, A = w_ptr_a[e] + l*lora_stride_a ([rank][I]),
 *              B = w_ptr_b[e] + l*lora_stride_b ([H][rank]):
 *       xa[r]      = (w * scale) * sum_i A[r][i] * x2[p][i]
 *       out[q][c]  = y[p][c] + sum_r xa[r] * B[c][r],   c < H
 * (the same association as O-shrink then O-expand, so with E = 1, top_k = 1
 * and no weights it is the dense delta bit for bit).
 * ------------------------------------------------------------------------ */
void oracle_moe_w2_pairs(const uint16_t *x2, int64_t ldx, int32_t I,
                         const int64_t *w_ptr_a, int64_t lora_stride_a,
                         const int64_t *w_ptr_b, int64_t lora_stride_b,
                         const int32_t *topk_ids, int32_t top_k, const int32_t *lora_ids,
                         const float *topk_weights, int32_t num_experts, int32_t num_loras,
                         int32_t rank, int32_t H, double scale, const uint16_t *y, int64_t ldy,
                         const int32_t *pairs, int32_t np, double *out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < np; ++q) {
        const int32_t p = pairs[q];
        const int32_t t = p / top_k;
        const int32_t l = lora_ids[t];
        const int32_t e = topk_ids[p];
        const uint16_t *yp = y + (int64_t)p * ldy;
        double *o = out + (int64_t)q * H;
        for (int32_t c = 0; c < H; ++c)
            o[c] = bf(yp[c]);
        if (l < 0 || l >= num_loras || e < 0 || e >= num_experts)
            continue;
        const double w = topk_weights ? (double)topk_weights[p] : 1.0;
        const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[e] + (int64_t)l * lora_stride_a;
        const uint16_t *B = (const uint16_t *)(intptr_t)w_ptr_b[e] + (int64_t)l * lora_stride_b;
        const uint16_t *xp = x2 + (int64_t)p * ldx;
        double xa[256];
        for (int32_t r = 0; r < rank; ++r) {
            double acc = 0.0;
            for (int32_t i = 0; i < I; ++i)
                acc += bf(xp[i]) * bf(A[(int64_t)r * I + i]);
            xa[r] = (w * scale) * acc;
        }
        for (int32_t c = 0; c < H; ++c) {
            double d = 0.0;
            for (int32_t r = 0; r < rank; ++r)
                d += xa[r] * bf(B[(int64_t)c * rank + r]);
            o[c] += d;
        }
    }
}

/* ------------------------------------------------------------------------
 * O-expert-work: the work items of the expert-sorted fold.  expert_offsets
 * has n_offsets entries, the prefix sum of rows per expert in the sorted
 * layout, so there are n_experts = max(n_offsets - 1, 0) experts and expert
 * e owns sorted rows offsets[e] .. offsets[e+1].  For each entry e of
 * `adapted`, in order: no item when e >= n_experts or when
 * offsets[e+1] <= offsets[e]; otherwise the item (e, offsets[e],
 * offsets[e+1] - offsets[e]).  Returns the number of items written.
 * ------------------------------------------------------------------------ */
int32_t oracle_expert_workitems(const uint32_t *expert_offsets, int32_t n_offsets,
                                const uint16_t *adapted, int32_t n_adapted,
                                int32_t *item_expert, uint32_t *item_row_off,
                                uint32_t *item_rows)
{
    const int32_t n_experts = n_offsets > 0 ? n_offsets - 1 : 0;
    int32_t n_items = 0;
    for (int32_t i = 0; i < n_adapted; ++i) {
        const int32_t e = (int32_t)adapted[i];
        if (e >= n_experts)
            continue;
        const uint32_t start = expert_offsets[e];
        const uint32_t end = expert_offsets[e + 1];
        if (end <= start)
            continue;
        item_expert[n_items] = e;
        item_row_off[n_items] = start;
        item_rows[n_items] = end - start;
        ++n_items;
    }
    return n_items;
}
