/*
 * moe_oracle.c -- plain, slow CPU reference for the MoE dispatch-permute ->
 * grouped SwiGLU MLP -> combine-unpermute path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; floating point is evaluated
 * in double precision except where a float decides an integer (fp8 scale and
 * code selection), which is taken in float as the GPU kernels take it.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and expert
 *        output buffers"
 *   [P2] DeepEP PR #716 "perf: reuse HybridEP routing allgather buffer"
 *   [P3] NeMo-Automodel PR #3931 "perf(moe): sync-free HybridEP dispatch
 *        (capacity mode, equal token counts)"
 *   [P4] Megatron-LM PR #4632 "moe: add DeepEP V2 ElasticBuffer support to MoE
 *        flex dispatcher"
 *   [P5] TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels"
 *
 * The pages state the interface of the operation, not its arithmetic, so each
 * function below is the plain definition of what that interface returns.
 * Where the pages leave a choice open the reading taken is written next to
 * the code that applies it.
 *
 * Pins: every function here is checked by the CPU tests against something
 * other than itself (brute force, invariants, numpy/torch library routines,
 * page-printed values).  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FLAG_CAPACITY   1  /* some expert received more copies than its capacity   */
#define ORC_FLAG_OUT_ROWS   2  /* padded segments need more rows than the output holds */
#define ORC_FLAG_BAD_EXPERT 4  /* a dense entry outside [-1, E)                        */
#define ORC_FLAG_DUPLICATE  8  /* repeated expert in a dense row / too many in a sparse row */

enum { ORC_DENSE_I16 = 0, ORC_DENSE_I32 = 1, ORC_SPARSE_U8 = 2 };

/* ------------------------------------------------------------------------ */
/* threads                                                                   */
/* ------------------------------------------------------------------------ */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* number formats, from their definitions                                     */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.  Round a double
 * to the nearest bfloat16 value, ties to even, overflow to infinity. */
uint16_t orc_bf16_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex);                    /* a in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    if (e < -126) e = -126;           /* subnormals share the lowest binade's spacing */
    double q = ldexp(1.0, e - 7);     /* spacing of representable values here */
    double n = nearbyint(a / q);      /* exact quotient; default mode = ties-to-even */
    double r = n * q;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)r;               /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

double orc_bf16_to_double(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* OCP fp8 e4m3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite 448; subnormals m/8 * 2^-6. */
double orc_e4m3_to_double(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest e4m3 value, ties to even, magnitudes beyond 448 saturate to 448. */
uint8_t orc_e4m3_from_double_sat(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -6) e = -6;
    double q = ldexp(1.0, e - 3);
    double r = nearbyint(a / q) * q;  /* <= 448 because 448 is representable */
    if (r == 0.0) return sign;
    frexp(r, &ex);
    e = ex - 1;
    uint8_t code;
    if (e >= -6) {
        double frac = r / ldexp(1.0, e) - 1.0;          /* in [0, 1) in steps of 1/8 */
        code = (uint8_t)(((e + 7) << 3) | (int)(frac * 8.0));
    } else {
        code = (uint8_t)(r / ldexp(1.0, -9));           /* subnormal: multiple of 2^-9 */
    }
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* host helpers whose values the pages print                                 */
/* ------------------------------------------------------------------------ */

/* Size of one rank's routing payload: a Boolean map holds one byte per
 * (token, expert); dense top-k indices hold one int16 per (token, slot).
 * [P2] section "Memory impact". */
int64_t orc_routing_bytes(int64_t tokens, int64_t experts, int64_t topk, int32_t fmt) {
    if (fmt == ORC_SPARSE_U8) return tokens * experts;
    if (fmt == ORC_DENSE_I16) return tokens * topk * 2;
    return tokens * topk * 4;
}

/* Static output bound from a calibrated row count: rows x factor rounded up,
 * then up to a multiple of 4.  [P3] section "What does this PR do ?" and the
 * calibration figure under "Validation". */
int64_t orc_capacity_from_rows(int64_t rows, double factor) {
    double c = ceil((double)rows * factor);
    int64_t ci = (int64_t)c;
    return (ci + 3) / 4 * 4;
}

/* Largest row count the padded segments can need: every expert's segment is
 * at most roundup(capacity, p) rows, and padding adds at most p-1 rows to each
 * of the E segments on top of the T*K copies. */
int64_t orc_out_rows_bound(int32_t T, int32_t E, int32_t K, int32_t pad, int32_t cap) {
    int64_t by_copies = (int64_t)T * K + (int64_t)E * (pad - 1);
    if (cap < 0) return by_copies;
    int64_t per = ((int64_t)cap + pad - 1) / pad * pad;
    int64_t by_cap = per * E;
    return by_cap < by_copies ? by_cap : by_copies;
}

/* ------------------------------------------------------------------------ */
/* routing metadata: counts, capacity, padding, offsets, row map, flag       */
/* ------------------------------------------------------------------------ */
/*
 * Inputs: T tokens (only t < T_live are routed), E experts, K slots, routing
 * as dense indices [T,K] (int16 or int32, -1 = empty slot) or a Boolean map
 * [T,E]; optional probabilities with the routing's shape; padding multiple
 * pad >= 1; per-expert capacity cap (< 0 = none); R rows in the output.
 *   [P2] "Memory impact" / "Implementation": the two routing formats.
 *   [P2] "Output and gradient regression": per-expert counts, handle metadata,
 *        optional probabilities.
 *   [P2] "Full HybridEP reference validation": padding multiple.
 *   [P3] "What does this PR do ?", "Validation": static output bound, device
 *        counts, overflow flag, silent truncation.
 *   [P4] "Motivation": the layout is inferred from the top-k indices.
 *
 * Readings where the pages are silent:
 *   - copies are taken in canonical order: token ascending, then dense slot
 *     ascending, or for the Boolean map expert ascending (slot j = rank of the
 *     expert among the row's routed experts);
 *   - dense entries outside [-1,E) and repeated experts in a row are skipped and
 *     flagged; a Boolean row with more than K experts keeps the K lowest ids;
 *   - counts are raw (before capacity and padding);
 *   - an expert keeps its first min(count, cap) copies in canonical order;
 *     count == cap is not an overflow;
 *   - a segment is the kept copies padded up to a multiple of pad; segments
 *     follow each other in expert order; rows inside a segment follow token
 *     order; copies whose row would fall at or beyond R are dropped;
 *   - rows that hold no copy have src_row = -1 and perm_prob = 0.
 * Outputs: counts[E], seg_off[E+1], row_id[T*K], copy_prob[T*K],
 * copy_expert[T*K] (expert of each slot or -1), src_row[R], perm_prob[R],
 * *rows_needed, *flag.
 */
int orc_route(int32_t T, int32_t E, int32_t K, int32_t fmt, const void* routing,
              const float* probs, int32_t pad, int32_t cap, int64_t R, int32_t T_live,
              int32_t* counts, int64_t* seg_off, int32_t* row_id, float* copy_prob,
              int32_t* copy_expert, int32_t* src_row, float* perm_prob,
              int64_t* rows_needed, int32_t* flag) {
    if (T < 0 || E < 1 || K < 1 || pad < 1 || R < 0) return -1;
    if (T_live < 0 || T_live > T) T_live = T;
    int32_t f = 0;
    uint8_t* seen = (uint8_t*)calloc((size_t)E, 1);
    int64_t* next = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int32_t* kept = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!seen || !next || !kept) { free(seen); free(next); free(kept); return -2; }

    /* 1. canonical copies */
    for (int64_t i = 0; i < (int64_t)T * K; i++) { copy_expert[i] = -1; copy_prob[i] = 0.0f; }
    for (int32_t t = 0; t < T_live; t++) {
        if (fmt == ORC_SPARSE_U8) {
            const uint8_t* map = (const uint8_t*)routing + (int64_t)t * E;
            int32_t j = 0;
            for (int32_t e = 0; e < E; e++) {
                if (!map[e]) continue;
                if (j >= K) { f |= ORC_FLAG_DUPLICATE; continue; }
                copy_expert[(int64_t)t * K + j] = e;
                copy_prob[(int64_t)t * K + j] = probs ? probs[(int64_t)t * E + e] : 1.0f;
                j++;
            }
        } else {
            memset(seen, 0, (size_t)E);
            for (int32_t j = 0; j < K; j++) {
                int64_t at = (int64_t)t * K + j;
                int32_t e = (fmt == ORC_DENSE_I16) ? ((const int16_t*)routing)[at]
                                                   : ((const int32_t*)routing)[at];
                if (e == -1) continue;
                if (e < -1 || e >= E) { f |= ORC_FLAG_BAD_EXPERT; continue; }
                if (seen[e]) { f |= ORC_FLAG_DUPLICATE; continue; }
                seen[e] = 1;
                copy_expert[at] = e;
                copy_prob[at] = probs ? probs[at] : 1.0f;
            }
        }
    }

    /* 2. raw counts */
    for (int32_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * K; i++)
        if (copy_expert[i] >= 0) counts[copy_expert[i]]++;

    /* 3. capacity */
    for (int32_t e = 0; e < E; e++) {
        kept[e] = counts[e];
        if (cap >= 0 && counts[e] > cap) { kept[e] = cap; f |= ORC_FLAG_CAPACITY; }
    }

    /* 4. padding and exclusive scan over experts */
    seg_off[0] = 0;
    for (int32_t e = 0; e < E; e++) {
        int64_t padded = ((int64_t)kept[e] + pad - 1) / pad * pad;
        seg_off[e + 1] = seg_off[e] + padded;
    }
    *rows_needed = seg_off[E];
    if (seg_off[E] > R) f |= ORC_FLAG_OUT_ROWS;

    /* 5. row assignment */
    for (int64_t r = 0; r < R; r++) { src_row[r] = -1; perm_prob[r] = 0.0f; }
    for (int32_t t = 0; t < T; t++) {
        for (int32_t j = 0; j < K; j++) {
            int64_t at = (int64_t)t * K + j;
            int32_t e = copy_expert[at];
            row_id[at] = -1;
            if (e < 0) continue;
            int64_t rank = next[e]++;
            int64_t row = seg_off[e] + rank;
            if (rank < kept[e] && row < R) {
                row_id[at] = (int32_t)row;
                src_row[row] = t;
                perm_prob[row] = copy_prob[at];
            } else {
                copy_prob[at] = 0.0f;
            }
        }
    }
    *flag = f;
    free(seen); free(next); free(kept);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* permute: copy each kept token row to its destination row                  */
/* [P1] "Summary"/"Configuration": dispatch writes permuted tokens into a      */
/* caller-provided output; [P2] "Full HybridEP reference validation":         */
/* dispatch with permutation, BF16 and FP8 payloads.                          */
/* Rows are opaque byte strings (a bf16 row, an fp8 row, or its scale row).   */
/* ------------------------------------------------------------------------ */
void orc_permute_rows(int32_t T, int32_t K, int64_t row_bytes, const uint8_t* x,
                      const int32_t* row_id, uint8_t* out) {
    for (int32_t t = 0; t < T; t++)
        for (int32_t j = 0; j < K; j++) {
            int32_t r = row_id[(int64_t)t * K + j];
            if (r >= 0) memcpy(out + (int64_t)r * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);
        }
}

/* ------------------------------------------------------------------------ */
/* combine: probability-weighted sum of each token's surviving copies         */
/* [P1] "Summary"/"Motivation": combine with unpermute is the final read of   */
/* the expert output; [P5] review-fix commit: the top-k reduction of a token  */
/* set that may be empty.  Sum in double, one rounding to bf16; a token with  */
/* no surviving copy yields 0.                                               */
/* ------------------------------------------------------------------------ */
void orc_combine_bf16(int32_t T, int32_t K, int32_t H, const int32_t* row_id,
                      const float* copy_prob, int32_t apply_probs, const uint16_t* Y,
                      uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        for (int32_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int32_t j = 0; j < K; j++) {
                int32_t r = row_id[(int64_t)t * K + j];
                if (r < 0) continue;
                double w = apply_probs ? (double)copy_prob[(int64_t)t * K + j] : 1.0;
                acc += w * orc_bf16_to_double(Y[(int64_t)r * H + h]);
            }
            y[(int64_t)t * H + h] = orc_bf16_from_double(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* combine from fp8 expert outputs                                           */
/* The fp8 combine format: expert-output rows are e4m3 codes with one fp32    */
/* scale per 128 columns ([P2] "Full HybridEP reference validation": FP8      */
/* token payloads; [P1] "Configuration": FP8 expert GEMMs).  Each copy's row  */
/* is dequantised exactly (code value * scale, in double), then combined as   */
/* in orc_combine_bf16: weighted sum in double, one rounding to bf16.         */
/* ------------------------------------------------------------------------ */
void orc_combine_fp8(int32_t T, int32_t K, int32_t H, const int32_t* row_id,
                     const float* copy_prob, int32_t apply_probs, const uint8_t* Yq,
                     const float* Ys, uint16_t* y) {
    const int32_t nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        for (int32_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int32_t j = 0; j < K; j++) {
                int32_t r = row_id[(int64_t)t * K + j];
                if (r < 0) continue;
                double w = apply_probs ? (double)copy_prob[(int64_t)t * K + j] : 1.0;
                double v = orc_e4m3_to_double(Yq[(int64_t)r * H + h]) * (double)Ys[(int64_t)r * nb + h / 128];
                acc += w * v;
            }
            y[(int64_t)t * H + h] = orc_bf16_from_double(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* backward of dispatch                                                      */
/* [P2] "Full HybridEP reference validation": hidden-state and probability    */
/* gradients of the backward-of-dispatch communication.  Dispatch copies      */
/* token t's row (and the copy's probability) to row row_id[t,j] for every    */
/* kept copy, so the gradient of token t is the sum of its kept copies' row   */
/* gradients (double, one rounding to bf16; 0 with no kept copy), and the     */
/* gradient of probability (t, j) is the probability gradient of its row.     */
/* grad_probs has the routing's shape: dense [T,K] by slot, sparse [T,E] by   */
/* expert (copy_expert), 0 wherever no copy was kept.                         */
/* ------------------------------------------------------------------------ */
void orc_dispatch_backward(int32_t T, int32_t K, int32_t E, int32_t H, int32_t sparse,
                           const int32_t* row_id, const int32_t* copy_expert,
                           const uint16_t* grad_out, const float* grad_out_probs,
                           uint16_t* grad_x, float* grad_probs) {
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        for (int32_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int32_t j = 0; j < K; j++) {
                int32_t r = row_id[(int64_t)t * K + j];
                if (r >= 0) acc += orc_bf16_to_double(grad_out[(int64_t)r * H + h]);
            }
            grad_x[(int64_t)t * H + h] = orc_bf16_from_double(acc);
        }
    }
    if (!grad_probs || !grad_out_probs) return;
    const int64_t width = sparse ? E : K;
    for (int64_t i = 0; i < (int64_t)T * width; i++) grad_probs[i] = 0.0f;
    for (int32_t t = 0; t < T; t++)
        for (int32_t j = 0; j < K; j++) {
            int32_t r = row_id[(int64_t)t * K + j];
            if (r < 0) continue;
            int64_t col = sparse ? copy_expert[(int64_t)t * K + j] : j;
            grad_probs[(int64_t)t * width + col] = grad_out_probs[r];
        }
}

/* ------------------------------------------------------------------------ */
/* backward of combine                                                       */
/* [P2] "Full HybridEP reference validation": hidden-state and probability    */
/* gradients of the backward-of-combine communication.  With                  */
/* y[t] = sum_j w_tj * Y[row_id[t,j]], w = the copy probability when          */
/* probabilities are applied, else 1:                                         */
/*   dL/dY[row_id[t,j]] = w_tj * dL/dy[t]  (product in double, one rounding   */
/*   to bf16; rows holding no kept copy are not written), and                 */
/*   dL/dp_tj = sum_h dL/dy[t,h] * Y[row_id[t,j],h]  (double, then float)     */
/*   when probabilities are applied, 0 otherwise and for dropped copies.      */
/* grad_probs has the routing's shape as in the dispatch backward.            */
/* ------------------------------------------------------------------------ */
void orc_combine_backward(int32_t T, int32_t K, int32_t E, int32_t H, int32_t sparse,
                          const int32_t* row_id, const int32_t* copy_expert,
                          const float* copy_prob, int32_t apply_probs, const uint16_t* grad_y,
                          const uint16_t* Y, uint16_t* grad_Y, float* grad_probs) {
    const int64_t width = sparse ? E : K;
    if (grad_probs)
        for (int64_t i = 0; i < (int64_t)T * width; i++) grad_probs[i] = 0.0f;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        for (int32_t j = 0; j < K; j++) {
            int32_t r = row_id[(int64_t)t * K + j];
            if (r < 0) continue;
            double w = apply_probs ? (double)copy_prob[(int64_t)t * K + j] : 1.0;
            double dot = 0.0;
            for (int32_t h = 0; h < H; h++) {
                double g = orc_bf16_to_double(grad_y[(int64_t)t * H + h]);
                grad_Y[(int64_t)r * H + h] = orc_bf16_from_double(w * g);
                if (grad_probs && apply_probs) dot += g * orc_bf16_to_double(Y[(int64_t)r * H + h]);
            }
            if (grad_probs) {
                int64_t col = sparse ? copy_expert[(int64_t)t * K + j] : j;
                grad_probs[(int64_t)t * width + col] = apply_probs ? (float)dot : 0.0f;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* expert MLP (bf16 weights)                                                 */
/* [P1] "Summary"/"Configuration": a grouped FC1 -> activation -> FC2 MLP     */
/* writing FC2 into a caller-owned buffer; [P5] streaming-load commit: FC1    */
/* weight is the concatenated w3_w1 matrix.                                  */
/* Reading: W1 is [2F, H] with rows [0,F) the gate (SiLU) half and [F,2F) the  */
/* up half; W2 is [H, F]; a = bf16(silu(g) * u); y = bf16(W2 a); sums and     */
/* silu in double; silu(z) = z / (1 + exp(-z)).                              */
/* ------------------------------------------------------------------------ */
static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* y32 (nullable [n,H]): the FC2 sums rounded once to float, the value an    */
/* fp8 output format quantises (below, combine in the fp8 format).            */
/* Every output value is one sequential sum in ascending index order; the     */
/* threads only split the independent (row, feature) and (row, output) pairs. */
void orc_expert_mlp_bf16(int32_t n, int32_t H, int32_t F, const uint16_t* x,
                         const uint16_t* w1, const uint16_t* w2, uint16_t* y,
                         uint16_t* a_out /* nullable [n,F] */, float* y32) {
    uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * (size_t)F);
    /* FC1 + SwiGLU: a[r,i] = bf16(silu(g) * u) */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t ri = 0; ri < (int64_t)n * F; ri++) {
        const int32_t r = (int32_t)(ri / F), i = (int32_t)(ri % F);
        const uint16_t* xr = x + (int64_t)r * H;
        const uint16_t* wg = w1 + (int64_t)i * H;
        const uint16_t* wu = w1 + (int64_t)(F + i) * H;
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; h++) {
            double xv = orc_bf16_to_double(xr[h]);
            g += xv * orc_bf16_to_double(wg[h]);
            u += xv * orc_bf16_to_double(wu[h]);
        }
        a[ri] = orc_bf16_from_double(orc_silu(g) * u);
    }
    if (a_out) memcpy(a_out, a, sizeof(uint16_t) * (size_t)n * (size_t)F);
    /* FC2: y[r,o] = bf16(sum_i a[r,i] * W2[o,i]) */
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t ro = 0; ro < (int64_t)n * H; ro++) {
        const int32_t r = (int32_t)(ro / H), o = (int32_t)(ro % H);
        const uint16_t* ar = a + (int64_t)r * F;
        const uint16_t* w = w2 + (int64_t)o * F;
        double acc = 0.0;
        for (int32_t i = 0; i < F; i++)
            acc += orc_bf16_to_double(ar[i]) * orc_bf16_to_double(w[i]);
        y[ro] = orc_bf16_from_double(acc);
        if (y32) y32[ro] = (float)acc;
    }
    free(a);
}

/* ------------------------------------------------------------------------ */
/* fp8 block quantisation of activation rows                                 */
/* [P2] "Full HybridEP reference validation" and [P1] "Configuration": FP8    */
/* payloads and FP8 expert GEMMs.  The pages do not fix the scaling; reading: */
/* one fp32 scale per (row, 128 columns), scale = block amax / 448 (1 for an  */
/* all-zero block), code = e4m3(x / scale) saturating.  Scale and quotient    */
/* are float operations (they decide the integer code).                       */
/* ------------------------------------------------------------------------ */
void orc_quant_rows_e4m3_f32(int32_t n, int32_t cols, const float* x, uint8_t* q, float* scales) {
    int32_t nb = cols / 128;
    for (int32_t r = 0; r < n; r++)
        for (int32_t b = 0; b < nb; b++) {
            const float* xb = x + (int64_t)r * cols + (int64_t)b * 128;
            float amax = 0.0f;
            for (int32_t i = 0; i < 128; i++) {
                float v = fabsf(xb[i]);
                if (v > amax) amax = v;
            }
            float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[(int64_t)r * nb + b] = s;
            for (int32_t i = 0; i < 128; i++) {
                float v = xb[i] / s;
                q[(int64_t)r * cols + (int64_t)b * 128 + i] = orc_e4m3_from_double_sat((double)v);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* expert MLP with fp8 weights (W8A8)                                        */
/* [P5] first and streaming-load commits: low-precision expert weights with   */
/* block scales.  Readings: weights are e4m3 codes with one fp32 scale per    */
/* 128x128 block; the bf16 input row is quantised per 1x128 block (above);     */
/* products use dequantised values (code * scale, exact in double); a =       */
/* silu(g)*u is re-quantised per 1x128 block (decision in float) before FC2;  */
/* FC2 output is bf16.                                                        */
/* ------------------------------------------------------------------------ */
void orc_expert_mlp_fp8(int32_t n, int32_t H, int32_t F, const uint16_t* x,
                        const uint8_t* w1q, const float* w1s, const uint8_t* w2q,
                        const float* w2s, uint16_t* y) {
    int32_t hb = H / 128, fb = F / 128;
    /* the value of every e4m3 code, from the definition above (read back per weight) */
    double code_val[256];
    for (int c = 0; c < 256; c++) code_val[c] = orc_e4m3_to_double((uint8_t)c);
    double* xd = (double*)malloc(sizeof(double) * (size_t)n * (size_t)H);   /* dequantised input rows */
    float* af = (float*)malloc(sizeof(float) * (size_t)n * (size_t)F);     /* silu(g) * u, in float  */
    double* ad = (double*)malloc(sizeof(double) * (size_t)n * (size_t)F);  /* dequantised a          */
    /* quantise each input row per 1x128 block, keep its dequantised values */
#pragma omp parallel
    {
        float* xf = (float*)malloc(sizeof(float) * (size_t)H);
        uint8_t* xq = (uint8_t*)malloc((size_t)H);
        float* xs = (float*)malloc(sizeof(float) * (size_t)hb);
#pragma omp for schedule(static)
        for (int32_t r = 0; r < n; r++) {
            for (int32_t h = 0; h < H; h++) xf[h] = (float)orc_bf16_to_double(x[(int64_t)r * H + h]);
            orc_quant_rows_e4m3_f32(1, H, xf, xq, xs);
            for (int32_t h = 0; h < H; h++) xd[(int64_t)r * H + h] = orc_e4m3_to_double(xq[h]) * (double)xs[h / 128];
        }
        free(xf); free(xq); free(xs);
    }
    /* FC1 + SwiGLU over every (row, feature) pair; each sum in ascending h */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t ri = 0; ri < (int64_t)n * F; ri++) {
        const int32_t r = (int32_t)(ri / F), i = (int32_t)(ri % F);
        const double* xr = xd + (int64_t)r * H;
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; h++) {
            double wg = code_val[w1q[(int64_t)i * H + h]] * (double)w1s[(int64_t)(i / 128) * hb + h / 128];
            double wu = code_val[w1q[(int64_t)(F + i) * H + h]] * (double)w1s[(int64_t)((F + i) / 128) * hb + h / 128];
            g += xr[h] * wg;
            u += xr[h] * wu;
        }
        af[ri] = (float)(orc_silu(g) * u);
    }
    /* re-quantise a per 1x128 block */
#pragma omp parallel
    {
        uint8_t* aq = (uint8_t*)malloc((size_t)F);
        float* as = (float*)malloc(sizeof(float) * (size_t)fb);
#pragma omp for schedule(static)
        for (int32_t r = 0; r < n; r++) {
            orc_quant_rows_e4m3_f32(1, F, af + (int64_t)r * F, aq, as);
            for (int32_t i = 0; i < F; i++) ad[(int64_t)r * F + i] = orc_e4m3_to_double(aq[i]) * (double)as[i / 128];
        }
        free(aq); free(as);
    }
    /* FC2 over every (row, output) pair; each sum in ascending i */
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t ro = 0; ro < (int64_t)n * H; ro++) {
        const int32_t r = (int32_t)(ro / H), o = (int32_t)(ro % H);
        const double* ar = ad + (int64_t)r * F;
        double acc = 0.0;
        for (int32_t i = 0; i < F; i++)
            acc += ar[i] * code_val[w2q[(int64_t)o * F + i]] * (double)w2s[(int64_t)(o / 128) * fb + i / 128];
        y[ro] = orc_bf16_from_double(acc);
    }
    free(xd); free(af); free(ad);
}
