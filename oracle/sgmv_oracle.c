/*
 * sgmv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference of the SGMV LoRA add-on,
 * computed in IEEE double precision.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library; the product
 * path (the HIP library under segmented_gather_gemv_sgmv_amd/) never does, and
 * the two share no code.
 *
 * What is computed (plain definition, no blocking, no reordering):
 *
 *   LoRA forward: the output of an adapted linear layer is the base product
 *   plus a low-rank correction, y = xW + xAB, with A of shape [H1, r] and B of
 *   shape [r, H2]  (Punica walkthrough, omica.com.cn/news/959180, section 2.1).
 *   The shrink, expand and lora_apply functions compute only the correction
 *   xAB: the base xW belongs to the caller and is already inside y on entry.
 *   sgmv_oracle_lora_linear computes the whole layer, base product included.
 *
 *   Many requests, each with its own adapter, are served in one batch: the
 *   correction for request i is x_i A_i B_i, evaluated in two steps, first the
 *   rank-r vector v_i = x_i A_i (the segmented-gather step) and then v_i B_i
 *   (the batched matrix-vector step)  (same page, section 2.2).
 *
 *   All A matrices share one rank and sit back to back in one buffer, and the
 *   same holds for all B matrices (same page, section 2.2; aivaro.ru answer
 *   959, section 3.2), so the stacks are A_stack[N][H1][r] and
 *   B_stack[N][r][H2], row-major, adapter a at offset a*H1*r and a*r*H2.
 *
 *   The batch is cut into contiguous row segments, segment s covering rows
 *   [seg_indptr[s], seg_indptr[s+1]) and naming adapter adapter_ids[s]
 *   (segmented inputs and outputs: Punica review, nubint.ai, "Proposed
 *   method"; the CSR form of the segment table is this library's reading).
 *
 *   A scale s multiplies the correction: y_i += s * (x_i A) B.  The pages
 *   write the correction without a factor, which is the case s = 1.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - shrink overwrites v for covered rows; expand and lora_apply accumulate
 *     into y; rows outside every segment are left exactly as they were;
 *   - the reduction order is ascending h for the shrink and ascending k for
 *     the expand; v is kept in double and never rounded;
 *   - an empty segment does nothing; one adapter may name several segments.
 *
 * Inputs arrive as float arrays that already hold the dtype-rounded values
 * (fp16/bf16/fp32 values are exact in float); every product and sum below is
 * taken in double.  Returns 0 on success and -1 for a malformed segment table
 * or shape (the oracle does not guess what a malformed table means).
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

static int check_segments(const int32_t* seg_indptr, const int32_t* adapter_ids,
                          int32_t num_segments, int32_t num_rows, int32_t num_adapters)
{
    if (num_segments < 0 || num_rows < 0 || num_adapters < 0) return -1;
    if (num_segments == 0) return 0;
    if (seg_indptr[0] < 0) return -1;
    for (int32_t s = 0; s < num_segments; ++s) {
        if (seg_indptr[s + 1] < seg_indptr[s]) return -1;
        if (adapter_ids[s] < 0 || adapter_ids[s] >= num_adapters) return -1;
    }
    if (seg_indptr[num_segments] > num_rows) return -1;
    return 0;
}

/* v[i][k] = sum over h of x[i][h] * A_stack[a][h][k], for every row i of
 * every segment (adapter a = adapter_ids of that segment).  Rows outside all
 * segments keep the value v held on entry.                                  */
int sgmv_oracle_shrink(double* v, const float* x, const float* A_stack,
                       const int32_t* seg_indptr, const int32_t* adapter_ids,
                       int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                       int32_t H1, int32_t r)
{
    if (H1 < 0 || r < 0) return -1;
    if (check_segments(seg_indptr, adapter_ids, num_segments, num_rows, num_adapters)) return -1;
    for (int32_t s = 0; s < num_segments; ++s) {
        const int64_t a = adapter_ids[s];
        const float* A = A_stack + a * (int64_t)H1 * r;
        for (int64_t i = seg_indptr[s]; i < seg_indptr[s + 1]; ++i) {
            for (int64_t k = 0; k < r; ++k) {
                double acc = 0.0;
                for (int64_t h = 0; h < H1; ++h)
                    acc += (double)x[i * H1 + h] * (double)A[h * r + k];
                v[i * r + k] = acc;
            }
        }
    }
    return 0;
}

/* y[i][j] += scale * sum over k of v[i][k] * B_stack[a][k][j].              */
int sgmv_oracle_expand(double* y, const double* v, const float* B_stack,
                       const int32_t* seg_indptr, const int32_t* adapter_ids,
                       int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                       int32_t r, int32_t H2, double scale)
{
    if (H2 < 0 || r < 0) return -1;
    if (check_segments(seg_indptr, adapter_ids, num_segments, num_rows, num_adapters)) return -1;
    for (int32_t s = 0; s < num_segments; ++s) {
        const int64_t a = adapter_ids[s];
        const float* B = B_stack + a * (int64_t)r * H2;
        for (int64_t i = seg_indptr[s]; i < seg_indptr[s + 1]; ++i) {
            for (int64_t j = 0; j < H2; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < r; ++k)
                    acc += v[i * r + k] * (double)B[k * H2 + j];
                y[i * H2 + j] = y[i * H2 + j] + scale * acc;
            }
        }
    }
    return 0;
}

/* The whole add-on for one batch: y := y0, then per row the shrink followed
 * by the expand.  y (double, [num_rows][H2]) is filled from y0 here; v
 * (double, [num_rows][r]) receives the intermediate for covered rows and is
 * zero elsewhere.                                                            */
int sgmv_oracle_lora_apply(double* y, double* v, const float* y0, const float* x,
                           const float* A_stack, const float* B_stack,
                           const int32_t* seg_indptr, const int32_t* adapter_ids,
                           int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                           int32_t H1, int32_t H2, int32_t r, double scale)
{
    if (H1 < 0 || H2 < 0 || r < 0) return -1;
    if (check_segments(seg_indptr, adapter_ids, num_segments, num_rows, num_adapters)) return -1;
    for (int64_t e = 0; e < (int64_t)num_rows * H2; ++e) y[e] = (double)y0[e];
    for (int64_t e = 0; e < (int64_t)num_rows * r; ++e) v[e] = 0.0;
    if (sgmv_oracle_shrink(v, x, A_stack, seg_indptr, adapter_ids, num_segments,
                           num_rows, num_adapters, H1, r)) return -1;
    return sgmv_oracle_expand(y, v, B_stack, seg_indptr, adapter_ids, num_segments,
                              num_rows, num_adapters, r, H2, scale);
}

/* An adapted linear layer for one batch, base product included: for every
 * row i and column j
 *     y[i][j] = sum over h of x[i][h] * W[j][h]  (+ bias[j])
 * and then, for the rows of each segment, the add-on scale * (x_i A_a) B_a,
 * i.e. y = xW + xAB of Punica walkthrough (omica.com.cn/news/959180, section
 * 2.1) with the base layer folded in, as the fused kernel of aivaro.ru answer
 * 959 (section 3.2) does.  W is stored [H2][H1] (output feature major, each
 * row the weights of one output), so the page's W is its transpose; bias may
 * be NULL.  Rows outside every segment receive the base product only.      */
int sgmv_oracle_lora_linear(double* y, const float* x, const float* W, const float* bias,
                            const float* A_stack, const float* B_stack,
                            const int32_t* seg_indptr, const int32_t* adapter_ids,
                            int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                            int32_t H1, int32_t H2, int32_t r, double scale)
{
    if (H1 < 0 || H2 < 0 || r < 0) return -1;
    if (check_segments(seg_indptr, adapter_ids, num_segments, num_rows, num_adapters)) return -1;
    for (int64_t i = 0; i < num_rows; ++i) {
        const float* xr = x + i * (int64_t)H1;
        for (int64_t j = 0; j < H2; ++j) {
            const float* wr = W + j * (int64_t)H1;
            double acc = 0.0;
            for (int64_t h = 0; h < H1; ++h)
                acc += (double)xr[h] * (double)wr[h];
            y[i * H2 + j] = bias ? acc + (double)bias[j] : acc;
        }
    }
    double* v = (double*)calloc((size_t)num_rows * (size_t)(r > 0 ? r : 1), sizeof(double));
    if (!v) return -1;
    int rc = sgmv_oracle_shrink(v, x, A_stack, seg_indptr, adapter_ids, num_segments,
                                num_rows, num_adapters, H1, r);
    if (!rc)
        rc = sgmv_oracle_expand(y, v, B_stack, seg_indptr, adapter_ids, num_segments,
                                num_rows, num_adapters, r, H2, scale);
    free(v);
    return rc;
}
