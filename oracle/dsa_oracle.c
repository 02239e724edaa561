/*
 * dsa_oracle.c -- plain, slow CPU reference for one DeepSeek Sparse Attention (DSA)
 * layer step.  TEST INFRASTRUCTURE ONLY: it is loaded by the test-suite, by the
 * smoke check and by the benchmark's CPU-baseline leg, never by the GPU product
 * path.  It shares no code, header, table or constant with the HIP library.
 *
 * Everything is computed in double precision straight from the definitions on the
 * pages; the only stored-precision step is the fp32 index score, which is what the
 * method itself ranks (the score tensor is fp32 on the pages).
 *
 * Sources (web pages, cited by title and section):
 *   [IDX]  "DeepSeek-V3.2-Exp - Split indexer heads", Indexer.forward excerpt: FP8
 *          queries and keys with per-block scales; the projected head weights (scaled
 *          by the inverse square root of the head count) are multiplied by the query
 *          scales and the indexer softmax scale; the score call is masked additively
 *          and the best index_topk positions are kept, never more than are visible.
 *   [DIAG] "dsa-indexer.excalidraw" (one DSA decode step in one layer, V3.2 sizes):
 *          the score of key s is the head-weighted sum of per-head ReLU(q . k_s); the
 *          top-k selector keeps 2048; the selected latent rows are gathered and all
 *          query heads attend to them (MQA), each row serving as key and value; the
 *          per-token cost box.
 *   [MASK] "DeepSeek-V3.2-Exp - Causal mask", Transformer.forward excerpt: additive
 *          -inf mask strictly above the diagonal when more than one row is processed,
 *          no mask for single-row decode.
 *   [MLA]  same page, MLA init and prefill excerpts: the softmax scale is the inverse
 *          square root of the qk head width; the MHA prefill form scales dense scores,
 *          adds an index mask (0 at the selected positions, -inf elsewhere) and the
 *          causal mask, takes a softmax and mixes the value rows.
 *   [V4]   "visualize_attention_masks.py" (DeepSeek-V4 mask visualiser): -1 marks
 *          unused top-k slots; in the compressed-sparse layers the indexer ranks
 *          compressed entries, entry e being available to the query at position p iff
 *          e < (p + 1) / compress_rate.
 *
 * Conventions (where the pages leave a point open, the plainest reading is taken):
 *   len[b]        valid keys of sequence b;  T query rows are the LAST T positions,
 *                 pos(b,t) = len[b] - T + t  (the excerpt's end position of a chunk is
 *                 its start position plus its length, [IDX]);
 *   key s is visible to row (b,t) iff 0 <= s <= pos(b,t)   ([MASK]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "dsa_oracle.h"

/* ------------------------------------------------------------------ element codecs */

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * exponent field 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
 * there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double orc_e4m3fn_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* p, int dtype, size_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return orc_bf16_value(((const uint16_t*)p)[i]);
    default: return ((const double*)p)[i];
    }
}

/* FP8 storage form of one latent cache row ([DIAG]: the latent cache holds FP8 latents
 * with bf16 rope parts, 656 bytes per token).  Reading taken for the byte order, which
 * the diagram does not draw: the 512 e4m3fn codes of the latent part, then its four
 * fp32 scales (one per 128 columns, the block size of the FP8 indexer keys, [IDX]),
 * then the 64 rope values as bf16; 512 + 4*4 + 64*2 = 656.  Column d < 512 is
 * code[d] * scale[d / 128]; column 512 + r is the bf16 rope value r. */
double orc_latent_fp8_value(const uint8_t* row, int d)
{
    if (d < ORC_FP8_LATENT_DV) {
        float scale;
        memcpy(&scale, row + ORC_FP8_LATENT_DV + 4 * (d / ORC_FP8_LATENT_BLOCK), sizeof scale);
        return orc_e4m3fn_value(row[d]) * (double)scale;
    }
    uint16_t bits;
    memcpy(&bits, row + ORC_FP8_LATENT_DV + 4 * (ORC_FP8_LATENT_DV / ORC_FP8_LATENT_BLOCK) +
                      2 * (d - ORC_FP8_LATENT_DV), sizeof bits);
    return orc_bf16_value(bits);
}

/* Element d of latent row `row` (of Dq columns) in storage type `dtype`. */
static double latent_elem(const void* latent, int dtype, size_t row, int Dq, int d)
{
    if (dtype == ORC_FP8_LATENT)
        return orc_latent_fp8_value((const uint8_t*)latent + row * ORC_FP8_LATENT_ROW_BYTES, d);
    return load_elem(latent, dtype, row * (size_t)Dq + d);
}

/* ------------------------------------------------------------------ visibility */

/* Cache rows visible to query row t of a call with T rows over a sequence of len
 * positions.  m = 1: every position is a cache row and row t sits at position
 * pos = len - T + t, so rows 0 .. pos are visible ([MASK]).  m > 1: the cache holds
 * compressed entries, each standing for m consecutive positions, and entry e is
 * available to the query at position pos iff e < (pos + 1) / m (integer division; the
 * causal threshold of the compressed-sparse layers in [V4]), so the first m - 1
 * positions see no entry at all. */
static int visible_rows(int len, int T, int t, int m)
{
    return (len - T + t + 1) / m;
}

/* T <= len[b] and every visible row exists in the cache (len[b] / m <= Lmax) */
static int check_rows(const int32_t* len, int B, int T, int Lmax, int m)
{
    if (m < 1) return ORC_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        if (len[b] < T || visible_rows(len[b], T, T - 1, m) > Lmax) return ORC_ERR_SHAPE;
    return ORC_OK;
}

/* ------------------------------------------------------------------ O2: index scores */

/* For every row (b,t) and cache position s:
 *   w'_h   = w[b,t,h] * q_scale[b,t,h] * sm_scale            (weight fold, [IDX])
 *   D_h    = sum_d deq(q[b,t,h,d]) * deq(k[b,s,d])            (FP8 query-key product)
 *   I      = k_scale[b,s] * sum_h w'_h * max(D_h, 0)          ([DIAG] score with ReLU)
 * and -inf where s is not visible ([MASK]; the additive mask of [IDX]).
 * The e4m3 products are exact in double and their 128-term sums stay far below 2^53
 * units of 2^-18, so D_h is exact; the head sum is one double rounding per term. */
int orc_index_scores(const uint8_t* q, const float* q_scale, const float* w,
                     const uint8_t* k, const float* k_scale, const int32_t* len,
                     int B, int T, int H, int D, int Lmax, double sm_scale, int m, float* scores)
{
    double table[256];
    int b;
    for (int c = 0; c < 256; ++c) table[c] = orc_e4m3fn_value((uint8_t)c);
    if (check_rows(len, B, T, Lmax, m) != ORC_OK) return ORC_ERR_SHAPE;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const int n = visible_rows(len[b], T, t, m);
            const size_t row = (size_t)b * T + t;
            float* out = scores + row * (size_t)Lmax;
            for (int s = 0; s < Lmax; ++s) {
                if (s >= n) { out[s] = -INFINITY; continue; }
                const uint8_t* ks = k + ((size_t)b * Lmax + s) * D;
                double acc = 0.0;
                for (int h = 0; h < H; ++h) {
                    const uint8_t* qh = q + (row * H + h) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += table[qh[d]] * table[ks[d]];
                    double wf = (double)w[row * H + h] * (double)q_scale[row * H + h] * sm_scale;
                    acc += wf * (dot > 0.0 ? dot : 0.0);
                }
                out[s] = (float)(acc * (double)k_scale[(size_t)b * Lmax + s]);
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ O3: top-k */

typedef struct { float score; int32_t pos; } scored_pos;

/* larger score first; equal scores by smaller position first */
static int by_score_desc(const void* a, const void* b)
{
    const scored_pos* x = (const scored_pos*)a;
    const scored_pos* y = (const scored_pos*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int by_pos_asc(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Per row: the min(k, n) visible rows with the largest scores (n = visible_rows; a full
 * sort, ties by smaller position), written in ascending position order and padded with
 * -1 up to k slots ([IDX] top-k capped at the visible count; [V4] -1 sentinel). */
int orc_topk(const float* scores, const int32_t* len, int B, int T, int Lmax, int k, int m,
             int32_t* idx)
{
    int b;
    if (k <= 0) return ORC_ERR_SHAPE;
    if (check_rows(len, B, T, Lmax, m) != ORC_OK) return ORC_ERR_SHAPE;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)b * T + t;
            const int n = visible_rows(len[b], T, t, m);
            const int kk = n < k ? n : k;
            const float* sc = scores + row * (size_t)Lmax;
            int32_t* out = idx + row * (size_t)k;
            scored_pos* v = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)n);
            for (int s = 0; s < n; ++s) { v[s].score = sc[s]; v[s].pos = s; }
            qsort(v, (size_t)n, sizeof *v, by_score_desc);
            for (int j = 0; j < kk; ++j) out[j] = v[j].pos;
            qsort(out, (size_t)kk, sizeof *out, by_pos_asc);
            for (int j = kk; j < k; ++j) out[j] = -1;
            free(v);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ O4: sparse latent attention */

/* Absorbed (MQA) form of the diagram's core attention: every query head h of row
 * (b,t) attends over the selected latent rows C[b, s] (s = idx[b,t,j] >= 0 and
 * visible), each row serving as key (all Dv+Dr columns) and value (first Dv columns):
 *   l_j = sm_scale * sum_{d < Dv+Dr} q[b,t,h,d] * C[b,s_j,d]
 *   p   = softmax(l),  out[b,t,h,:] = sum_j p_j C[b,s_j,0:Dv],  lse = log sum_j e^{l_j}
 * A row with no usable index gets out = 0 and lse = -inf.  With dtype ORC_FP8_LATENT
 * the rows are in the FP8 storage form and C[b,s,d] is their decoded value
 * (orc_latent_fp8_value), the queries bf16. */
int orc_sparse_mla_decode(const void* q, const void* latent, const int32_t* idx,
                          const int32_t* len, int dtype, int B, int T, int H, int Dv, int Dr,
                          int Lmax, int k, double sm_scale, int m, double* out, double* lse)
{
    const int Dq = Dv + Dr;
    /* FP8 latent rows pair with bf16 queries, at the storage form's fixed widths */
    const int qdt = dtype == ORC_FP8_LATENT ? ORC_BF16 : dtype;
    int b;
    if (dtype == ORC_FP8_LATENT && (Dv != ORC_FP8_LATENT_DV || Dr != ORC_FP8_LATENT_DR))
        return ORC_ERR_SHAPE;
    if (check_rows(len, B, T, Lmax, m) != ORC_OK) return ORC_ERR_SHAPE;
    for (size_t i = 0; i < (size_t)B * T * k; ++i)
        if (idx[i] < -1 || idx[i] >= Lmax) return ORC_ERR_INDEX;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)b * T + t;
            const int nvis = visible_rows(len[b], T, t, m);
            const int32_t* sel = idx + row * (size_t)k;
            double* logit = (double*)malloc(sizeof(double) * (size_t)k);
            int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
            int n = 0;
            for (int j = 0; j < k; ++j)
                if (sel[j] >= 0 && sel[j] < nvis) keys[n++] = sel[j];
            /* the selected rows' values, decoded once for all heads: C[j][c] = C[b, s_j, c] */
            double* C = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * Dq);
            for (int j = 0; j < n; ++j)
                for (int c = 0; c < Dq; ++c)
                    C[(size_t)j * Dq + c] = latent_elem(latent, dtype, (size_t)b * Lmax + keys[j], Dq, c);
            for (int h = 0; h < H; ++h) {
                const size_t qoff = (row * H + h) * (size_t)Dq;
                double* o = out + (row * H + h) * (size_t)Dv;
                double m = -INFINITY, sum = 0.0;
                for (int j = 0; j < n; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < Dq; ++d)
                        dot += load_elem(q, qdt, qoff + d) * C[(size_t)j * Dq + d];
                    logit[j] = sm_scale * dot;
                    if (logit[j] > m) m = logit[j];
                }
                for (int d = 0; d < Dv; ++d) o[d] = 0.0;
                if (n == 0) { if (lse) lse[row * H + h] = -INFINITY; continue; }
                for (int j = 0; j < n; ++j) sum += exp(logit[j] - m);
                for (int j = 0; j < n; ++j) {
                    const double p = exp(logit[j] - m) / sum;
                    for (int d = 0; d < Dv; ++d) o[d] += p * C[(size_t)j * Dq + d];
                }
                if (lse) lse[row * H + h] = m + log(sum);
            }
            free(C);
            free(logit);
            free(keys);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ O5: sparse MHA prefill */

/* MHA prefill form ([MLA] prefill excerpt) over a chunk that starts at position 0:
 * keys and values are the chunk's own T positions, per head.  Row t attends over
 * the selected positions that are also causally visible (s <= t):
 *   l_s = sm_scale * q[b,t,h,:] . k[b,s,h,:],  out = sum_s softmax(l)_s v[b,s,h,:].
 * Gather form: loop over the selected list only.  One query row (b,t), all heads;
 * out points at that row's [H,Dv] block, lse at its [H] block (may be NULL). */
static void mha_row(const void* q, const void* kk, const void* v, const int32_t* idx, int dtype,
                    int b, int t, int T, int H, int Dqk, int Dv, int k, double sm_scale,
                    double* out_row, double* lse_row)
{
    const size_t row = (size_t)b * T + t;
    const int32_t* sel = idx + row * (size_t)k;
    double* logit = (double*)malloc(sizeof(double) * (size_t)k);
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int n = 0;
    for (int j = 0; j < k; ++j)
        if (sel[j] >= 0 && sel[j] <= t) keys[n++] = sel[j];
    for (int h = 0; h < H; ++h) {
        const size_t qoff = (row * H + h) * (size_t)Dqk;
        double* o = out_row + (size_t)h * Dv;
        double m = -INFINITY, sum = 0.0;
        for (int j = 0; j < n; ++j) {
            const size_t koff = (((size_t)b * T + keys[j]) * H + h) * (size_t)Dqk;
            double dot = 0.0;
            for (int d = 0; d < Dqk; ++d)
                dot += load_elem(q, dtype, qoff + d) * load_elem(kk, dtype, koff + d);
            logit[j] = sm_scale * dot;
            if (logit[j] > m) m = logit[j];
        }
        for (int d = 0; d < Dv; ++d) o[d] = 0.0;
        if (n == 0) { if (lse_row) lse_row[h] = -INFINITY; continue; }
        for (int j = 0; j < n; ++j) sum += exp(logit[j] - m);
        for (int j = 0; j < n; ++j) {
            const double p = exp(logit[j] - m) / sum;
            const size_t voff = (((size_t)b * T + keys[j]) * H + h) * (size_t)Dv;
            for (int d = 0; d < Dv; ++d) o[d] += p * load_elem(v, dtype, voff + d);
        }
        if (lse_row) lse_row[h] = m + log(sum);
    }
    free(logit);
    free(keys);
}

int orc_sparse_mha_prefill(const void* q, const void* kk, const void* v, const int32_t* idx,
                           int dtype, int B, int T, int H, int Dqk, int Dv, int k,
                           double sm_scale, double* out, double* lse)
{
    int b;
    for (size_t i = 0; i < (size_t)B * T * k; ++i)
        if (idx[i] < -1 || idx[i] >= T) return ORC_ERR_INDEX;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)b * T + t;
            mha_row(q, kk, v, idx, dtype, b, t, T, H, Dqk, Dv, k, sm_scale,
                    out + row * H * (size_t)Dv, lse ? lse + row * H : NULL);
        }
    }
    return ORC_OK;
}

/* The same gather form for a list of query rows (b, t) = (rows_b[r], rows_t[r]) only;
 * out [n_rows,H,Dv], lse [n_rows,H].  Lets large chunks be checked on sampled rows. */
int orc_sparse_mha_prefill_rows(const void* q, const void* kk, const void* v, const int32_t* idx,
                                int dtype, int B, int T, int H, int Dqk, int Dv, int k,
                                double sm_scale, const int32_t* rows_b, const int32_t* rows_t,
                                int n_rows, double* out, double* lse)
{
    int r;
    for (r = 0; r < n_rows; ++r)
        if (rows_b[r] < 0 || rows_b[r] >= B || rows_t[r] < 0 || rows_t[r] >= T) return ORC_ERR_SHAPE;
    for (r = 0; r < n_rows; ++r) {
        const int32_t* sel = idx + ((size_t)rows_b[r] * T + rows_t[r]) * k;
        for (int j = 0; j < k; ++j)
            if (sel[j] < -1 || sel[j] >= T) return ORC_ERR_INDEX;
    }
#pragma omp parallel for schedule(dynamic)
    for (r = 0; r < n_rows; ++r)
        mha_row(q, kk, v, idx, dtype, rows_b[r], rows_t[r], T, H, Dqk, Dv, k, sm_scale,
                out + (size_t)r * H * Dv, lse ? lse + (size_t)r * H : NULL);
    return ORC_OK;
}

/* The same attention computed the way the MLA prefill excerpt writes it: dense scores
 * over all T keys, plus an additive index mask that is -inf everywhere except 0 at the
 * selected positions, plus the causal mask, then a softmax over all T keys and a mix
 * of all values.  Kept as a second, independently structured form for cross-checks. */
int orc_sparse_mha_prefill_dense(const void* q, const void* kk, const void* v,
                                 const int32_t* idx, int dtype, int B, int T, int H, int Dqk,
                                 int Dv, int k, double sm_scale, double* out, double* lse)
{
    int b;
    for (size_t i = 0; i < (size_t)B * T * k; ++i)
        if (idx[i] < -1 || idx[i] >= T) return ORC_ERR_INDEX;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)b * T + t;
            double* mask = (double*)malloc(sizeof(double) * (size_t)T);
            double* sc = (double*)malloc(sizeof(double) * (size_t)T);
            for (int s = 0; s < T; ++s) mask[s] = -INFINITY;           /* full(-inf)      */
            for (int j = 0; j < k; ++j)
                if (idx[row * k + j] >= 0) mask[idx[row * k + j]] = 0.0; /* scatter_(.., 0) */
            for (int s = t + 1; s < T; ++s) mask[s] += -INFINITY;       /* += causal mask  */
            for (int h = 0; h < H; ++h) {
                const size_t qoff = (row * H + h) * (size_t)Dqk;
                double* o = out + (row * H + h) * (size_t)Dv;
                double m = -INFINITY, sum = 0.0;
                for (int s = 0; s < T; ++s) {
                    const size_t koff = (((size_t)b * T + s) * H + h) * (size_t)Dqk;
                    double dot = 0.0;
                    for (int d = 0; d < Dqk; ++d)
                        dot += load_elem(q, dtype, qoff + d) * load_elem(kk, dtype, koff + d);
                    sc[s] = dot * sm_scale + mask[s];
                    if (sc[s] > m) m = sc[s];
                }
                for (int d = 0; d < Dv; ++d) o[d] = 0.0;
                if (m == -INFINITY) { if (lse) lse[row * H + h] = -INFINITY; continue; }
                for (int s = 0; s < T; ++s) sum += exp(sc[s] - m);
                for (int s = 0; s < T; ++s) {
                    const double p = exp(sc[s] - m) / sum;
                    if (p == 0.0) continue;
                    const size_t voff = (((size_t)b * T + s) * H + h) * (size_t)Dv;
                    for (int d = 0; d < Dv; ++d) o[d] += p * load_elem(v, dtype, voff + d);
                }
                if (lse) lse[row * H + h] = m + log(sum);
            }
            free(mask);
            free(sc);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ O6: layer step */

/* Index scores -> top-k -> sparse latent attention ([DIAG], one layer).  Scores and
 * indices are optionally returned (NULL to discard). */
int orc_layer_step_latent(const uint8_t* q_i, const float* q_scale, const float* w,
                          const uint8_t* k_i, const float* k_scale, const int32_t* len,
                          int B, int T, int H_I, int D_I, int Lmax, double sm_scale_i, int k,
                          const void* q, const void* latent, int dtype, int H, int Dv, int Dr,
                          double sm_scale, int m, double* out, double* lse, float* scores_out,
                          int32_t* idx_out)
{
    float* scores = scores_out ? scores_out
                               : (float*)malloc(sizeof(float) * (size_t)B * T * Lmax);
    int32_t* idx = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)B * T * k);
    int rc = orc_index_scores(q_i, q_scale, w, k_i, k_scale, len, B, T, H_I, D_I, Lmax,
                              sm_scale_i, m, scores);
    if (rc == ORC_OK) rc = orc_topk(scores, len, B, T, Lmax, k, m, idx);
    if (rc == ORC_OK)
        rc = orc_sparse_mla_decode(q, latent, idx, len, dtype, B, T, H, Dv, Dr, Lmax, k,
                                   sm_scale, m, out, lse);
    if (!scores_out) free(scores);
    if (!idx_out) free(idx);
    return rc;
}

/* Index scores -> top-k -> sparse MHA prefill ([IDX] + [MLA] prefill), chunk from 0. */
int orc_layer_step_mha(const uint8_t* q_i, const float* q_scale, const float* w,
                       const uint8_t* k_i, const float* k_scale, int B, int T, int H_I, int D_I,
                       double sm_scale_i, int k, const void* q, const void* kk, const void* v,
                       int dtype, int H, int Dqk, int Dv, double sm_scale, double* out,
                       double* lse, float* scores_out, int32_t* idx_out)
{
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    float* scores = scores_out ? scores_out
                               : (float*)malloc(sizeof(float) * (size_t)B * T * T);
    int32_t* idx = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)B * T * k);
    int rc;
    for (int b = 0; b < B; ++b) len[b] = T;
    rc = orc_index_scores(q_i, q_scale, w, k_i, k_scale, len, B, T, H_I, D_I, T, sm_scale_i, 1,
                          scores);
    if (rc == ORC_OK) rc = orc_topk(scores, len, B, T, T, k, 1, idx);
    if (rc == ORC_OK)
        rc = orc_sparse_mha_prefill(q, kk, v, idx, dtype, B, T, H, Dqk, Dv, k, sm_scale, out,
                                    lse);
    if (!scores_out) free(scores);
    if (!idx_out) free(idx);
    free(len);
    return rc;
}

/* ------------------------------------------------------------------ O7: indexer preparation */

/* [IDX] Indexer.forward, the steps between the projections and the scores: the query
 * heads and the normalised key are split into a rope part (the first R columns) and the
 * rest; rope is applied "not interleaved"; both go through rotate_activation; act_quant
 * turns them into FP8 codes with one scale per block, and the keys are written into the
 * key cache at the new positions.  Readings taken where the pages name a step without
 * its body:
 *   - non-interleaved rope pairs column j with column j + R/2 (j < R/2) and rotates the
 *     pair by the angle of frequency j at the token's position: (a, b) ->
 *     (a cos - b sin, a sin + b cos), with the angles' cos and sin given per position;
 *   - rotate_activation is the orthonormal Walsh-Hadamard rotation of each D-wide row
 *     (Sylvester order): v'_i = D^-1/2 sum_j (-1)^popcount(i & j) v_j.  The pages give
 *     only the name, so this reading is not pinned by them;
 *   - act_quant with block_size = D (one block per head row / key row) and a plain fp32
 *     scale: scale = max(amax, 1e-12) / 448, code = e4m3fn(clamp(x / scale, +-448)),
 *     nearest value, ties to the even code. */

/* OCP e4m3fn code of a value in [-448, 448]: nearest representable magnitude, ties to
 * the even code (the even mantissa); the sign bit is y's sign bit. */
uint8_t orc_e4m3fn_encode(double y)
{
    const int neg = signbit(y) ? 1 : 0;
    const double a = fabs(y);
    int mag;
    if (a < ldexp(1.0, -6)) {
        mag = (int)nearbyint(ldexp(a, 9));           /* subnormal step 2^-9; 8 = 2^-6 */
    } else {
        int e;
        const double m = 2.0 * frexp(a, &e);         /* a = m 2^(e-1), m in [1, 2) */
        const int mant = (int)nearbyint((m - 1.0) * 8.0);   /* 8 carries into the exponent */
        mag = ((e - 1 + 7) << 3) + mant;
    }
    return (uint8_t)((neg << 7) | mag);
}

/* act_quant of one D-wide row: returns the scale, writes the codes and (if y) x / scale. */
static double quant_row(const double* x, int D, uint8_t* codes, double* y)
{
    double amax = 0.0;
    for (int d = 0; d < D; ++d) amax = fmax(amax, fabs(x[d]));
    const double scale = fmax(amax, 1e-12) / 448.0;
    for (int d = 0; d < D; ++d) {
        double v = x[d] / scale;
        if (y) y[d] = v;
        v = fmin(fmax(v, -448.0), 448.0);
        codes[d] = orc_e4m3fn_encode(v);
    }
    return scale;
}

/* rope (non-interleaved) on the first R columns, then the Walsh-Hadamard rotation */
static void prep_row(const void* src, int dtype, size_t off, int D, int R, const float* cs,
                     const float* sn, double* out)
{
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    for (int d = 0; d < D; ++d) v[d] = load_elem(src, dtype, off + d);
    for (int j = 0; j < R / 2; ++j) {
        const double a = v[j], b = v[j + R / 2];
        v[j] = a * (double)cs[j] - b * (double)sn[j];
        v[j + R / 2] = a * (double)sn[j] + b * (double)cs[j];
    }
    const double norm = 1.0 / sqrt((double)D);
    for (int i = 0; i < D; ++i) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -v[j] : v[j];
        out[i] = acc * norm;
    }
    free(v);
}

/* q [B,T,H,D], k [B,T,D] (dtype), cos/sin [P,R/2] f32, start [B]: token t of sequence b
 * sits at position start[b] + t.  Outputs: q codes [B,T,H,D] and scales [B,T,H]; the key
 * codes and scales go to k_cache [B,Lmax,D] / k_scale [B,Lmax] at that position (other
 * rows untouched); q_y [B,T,H,D] and k_y [B,T,D] (may be NULL) get x / scale before
 * rounding; q_scale64 [B,T,H] and k_scale64 [B,T] the scales in double. */
int orc_indexer_prep(const void* q, const void* k, int dtype, const float* cosT, const float* sinT,
                     int P, const int32_t* start, int B, int T, int H, int D, int R, int Lmax,
                     uint8_t* q_fp8, double* q_scale64, uint8_t* k_cache, float* k_scale,
                     double* k_scale64, double* q_y, double* k_y)
{
    if (D < 2 || (D & (D - 1)) || R < 0 || R > D || (R & 1)) return ORC_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        if (start[b] < 0 || start[b] + T > Lmax || start[b] + T > P) return ORC_ERR_SHAPE;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            const int pos = start[b] + t;
            const float* cs = cosT + (size_t)pos * (R / 2);
            const float* sn = sinT + (size_t)pos * (R / 2);
            const size_t row = (size_t)b * T + t;
            double* x = (double*)malloc(sizeof(double) * (size_t)D);
            for (int h = 0; h < H; ++h) {
                const size_t qr = row * H + h;
                prep_row(q, dtype, qr * D, D, R, cs, sn, x);
                q_scale64[qr] = quant_row(x, D, q_fp8 + qr * D, q_y ? q_y + qr * D : NULL);
            }
            prep_row(k, dtype, row * D, D, R, cs, sn, x);
            const size_t kr = (size_t)b * Lmax + pos;
            const double ks = quant_row(x, D, k_cache + kr * D, k_y ? k_y + row * D : NULL);
            k_scale[kr] = (float)ks;
            k_scale64[row] = ks;
            free(x);
        }
    }
    return ORC_OK;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following parallel loops (n >= 1); for timing the oracle on one core. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
