/*
 * oracle.c -- plain, slow CPU oracle for the gated fine-grained sparse attention
 * layer: indexer scoring -> Top-K selection -> exact softmax attention over the
 * selected keys/values -> elementwise sigmoid output gate.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU path never calls it,
 * shares no source, header, table or helper with it, and does not fall back to it.
 *
 * Each step is the plain definition written out, one query row at a time:
 *
 *   scoring  "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer +
 *            Top-K: How Fine-Grained Sparse Attention Works", step 1 (a light
 *            scorer over low-dimensional projections of every history position).
 *            The pages give no formula; the reading taken is
 *              S[s] = sum_h w_h * max(0, sum_j qI[h][j] * kI[s][j])
 *            over int8 inputs, accumulated exactly (int64 here), for every
 *            candidate s in 0..p (causal, own position included).
 *   Top-K    same section, step 2 and its pseudocode (keep the K best positions
 *            per query); "Optimizing LLM Long-Context Inference with Indexed
 *            Top-K Sparse Attention", section "Interface Design" (topk over the
 *            score row). Order: higher score first, lower position on equal
 *            scores. Output: the selected positions in ascending order, padded
 *            with -1 when fewer than K candidates exist.
 *            Block granularity (same steps: positions or blocks): a block of
 *            positions scores as its best position, and K blocks are kept under
 *            the same order; their causal positions form the index row.
 *   attention same page, step 3 (standard softmax attention over the selected
 *            positions only, scaled by 1/sqrt(d)), in fp64 from the exact values
 *            of the bf16 inputs; query head h reads KV head h / (Hq/Hkv).
 *   gate     same page, step 4, and "From Linear Attention to Gated Sparse
 *            Attention", section 2 pseudocode (the gate multiplies the attention
 *            output): y = o * sigmoid(G), elementwise per head and feature; or,
 *            mixed with the other branch's output x (step 4 and its pseudocode),
 *            y = sigmoid(G) * o + (1 - sigmoid(G)) * x.
 *   backward the gradients of attention and gate (orc_attn_bwd), by the chain
 *            rule on the definitions above.
 *   append   same page, section "Engineering and Evaluation Recommendations"
 *            (chunked prefill that reuses the cached scorer inputs): the new
 *            rows' keys, values and indexer keys go into the caches right after
 *            each sequence's history, so a later chunk or decode step scores
 *            against the cache instead of recomputing earlier rows.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_OVERFLOW 1

/* ---------------------------------------------------------------- scoring */

/* Scores of one query row against history rows 0..n-1.
 * qI [H_I][d_I], kI [n][d_I], w [H_I]; writes S[0..n-1].
 * Returns ORC_OVERFLOW if any score leaves the int32 range (S is then clamped). */
int orc_score_row(int H_I, int d_I, const int8_t *qI, const int8_t *kI, const int8_t *w,
                  int64_t n, int32_t *S)
{
    int rc = ORC_OK;
    for (int64_t s = 0; s < n; ++s) {
        int64_t acc = 0;
        for (int h = 0; h < H_I; ++h) {
            int64_t dot = 0;
            for (int j = 0; j < d_I; ++j)
                dot += (int64_t)qI[h * d_I + j] * (int64_t)kI[s * d_I + j];
            if (dot < 0) dot = 0;                 /* ReLU */
            acc += (int64_t)w[h] * dot;
        }
        if (acc > INT32_MAX) { acc = INT32_MAX; rc = ORC_OVERFLOW; }
        if (acc < INT32_MIN) { acc = INT32_MIN; rc = ORC_OVERFLOW; }
        S[s] = (int32_t)acc;
    }
    return rc;
}

/* ------------------------------------------------------------------ Top-K */

typedef struct { int32_t score; int32_t pos; } orc_pair;

/* a before b  <=>  a.score > b.score, or equal scores and a.pos < b.pos */
static int orc_cmp_rank(const void *pa, const void *pb)
{
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    if (a->score != b->score) return a->score > b->score ? -1 : 1;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

static int orc_cmp_pos(const void *pa, const void *pb)
{
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

/* The min(K, n) best of S[0..n-1]; idx[0..K-1] ascending, -1 padded; sel (nullable)
 * holds the score of each selected position, INT32_MIN in the padding. */
void orc_topk_row(const int32_t *S, int64_t n, int K, int32_t *idx, int32_t *sel)
{
    int64_t m = n < K ? n : K;
    orc_pair *pr = (orc_pair *)malloc((size_t)(n > 0 ? n : 1) * sizeof(orc_pair));
    for (int64_t s = 0; s < n; ++s) { pr[s].score = S[s]; pr[s].pos = (int32_t)s; }
    qsort(pr, (size_t)n, sizeof(orc_pair), orc_cmp_rank);   /* full sort: rank order */
    qsort(pr, (size_t)m, sizeof(orc_pair), orc_cmp_pos);    /* the first m, by position */
    for (int64_t j = 0; j < K; ++j) {
        idx[j] = j < m ? pr[j].pos : -1;
        if (sel) sel[j] = j < m ? pr[j].score : INT32_MIN;
    }
    free(pr);
}

/* -------------------------------------------------------------- attention */

static double orc_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* The gate on one attention output o: y = s*o with s = sigmoid(G), or, with
 * the output x of another branch to mix with, y = s*o + (1 - s)*x: the gate
 * weighs the sparse branch against the linear or compressed one ("Hybrid
 * Sparse Attention for Long-Context LLMs", section "Indexer + Top-K: How
 * Fine-Grained Sparse Attention Works", step 4 and its pseudocode; "How
 * Fine-Grained Sparse Attention Reshapes Long-Context Architecture in Large
 * Models", section "How Indexer + Top-K Works at Runtime", its pseudocode). */
static double orc_gate(double o, double G, const uint16_t *mix, int64_t j)
{
    double s = 1.0 / (1.0 + exp(-G));
    return s * o + (mix ? (1.0 - s) * orc_bf16(mix[j]) : 0.0);
}

/* Gated attention of one query row over the listed positions.
 * q, gate, mix [Hq][d]; k, v [kv_rows][Hkv][d] (one sequence); idx [sets][K]:
 * sets divides Hq, and query head h reads set h / (Hq/sets): one set shared by
 * every head (sets = 1), one per key/value head (sets = Hkv), one per query
 * head (sets = Hq).
 * Entries outside 0..kv_len-1 (the -1 padding) are skipped. gate may be NULL
 * (ungated; then mix is ignored), mix may be NULL (no mixing). out [Hq][d],
 * lse [Hq] (natural log of the softmax denominator, including the running
 * max); a row with no valid entry has o = 0 (so out = 0 without mixing) and
 * lse = -inf. */
/* Element i of a bf16 or an fp32 array, widened exactly to double. */
typedef double (*orc_load)(const void *p, int64_t i);
static double orc_ld_bf16(const void *p, int64_t i) { return orc_bf16(((const uint16_t *)p)[i]); }
static double orc_ld_f32(const void *p, int64_t i) { return (double)((const float *)p)[i]; }

/* The row's attention with q, k, v and gate read through ld (bf16 or fp32
 * elements; mix is always bf16). */
static void orc_attn_row_ld(int Hq, int Hkv, int d, const void *q, const void *k, const void *v,
                            int64_t kv_len, const int32_t *idx, int K, int sets, const void *gate,
                            const uint16_t *mix, double scale, double *out, double *lse,
                            orc_load ld)
{
    int G = Hq / Hkv;
    int hps = Hq / (sets > 1 ? sets : 1);   /* query heads per index set */
    double *logit = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (int h = 0; h < Hq; ++h) {
        int g = h / G;
        const int32_t *ih = idx + (int64_t)(h / hps) * K;   /* this head's index set */
        double m = -INFINITY;
        for (int t = 0; t < K; ++t) {
            int64_t s = ih[t];
            if (s < 0 || s >= kv_len) { logit[t] = -INFINITY; continue; }
            double dot = 0.0;
            for (int j = 0; j < d; ++j)
                dot += ld(q, (int64_t)h * d + j) * ld(k, (s * Hkv + g) * d + j);
            logit[t] = scale * dot;
            if (logit[t] > m) m = logit[t];
        }
        double *o = out + (size_t)h * d;
        for (int j = 0; j < d; ++j) o[j] = 0.0;
        if (m == -INFINITY) {
            if (lse) lse[h] = -INFINITY;
        } else {
            double Z = 0.0;
            for (int t = 0; t < K; ++t) {
                int64_t s = ih[t];
                if (s < 0 || s >= kv_len) continue;
                double e = exp(logit[t] - m);
                Z += e;
                for (int j = 0; j < d; ++j) o[j] += e * ld(v, (s * Hkv + g) * d + j);
            }
            for (int j = 0; j < d; ++j) o[j] /= Z;
            if (lse) lse[h] = m + log(Z);
        }
        if (gate)
            for (int j = 0; j < d; ++j)
                o[j] = orc_gate(o[j], ld(gate, (int64_t)h * d + j), mix ? mix + (size_t)h * d : NULL, j);
    }
    free(logit);
}

void orc_attn_row(int Hq, int Hkv, int d, const uint16_t *q, const uint16_t *k,
                  const uint16_t *v, int64_t kv_len, const int32_t *idx, int K, int sets,
                  const uint16_t *gate, const uint16_t *mix, double scale, double *out,
                  double *lse)
{
    orc_attn_row_ld(Hq, Hkv, d, q, k, v, kv_len, idx, K, sets, gate, mix, scale, out, lse,
                    orc_ld_bf16);
}

/* ----------------------------------------------------------- whole rows */

/* Scores for a list of (sequence, query row) pairs; rows [nrows][Tk], only
 * positions 0..p written (p = q_offset[b] + i). Returns ORC_OVERFLOW if any
 * score overflowed int32; invalid rows (p outside 0..kv_len-1) are left untouched. */
int orc_scores_rows(int Tq, int Tk, int H_I, int d_I, const int32_t *q_offset,
                    const int32_t *kv_len, const int8_t *q_idx, const int8_t *k_idx,
                    const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                    int64_t nrows, const int32_t *row_b, const int32_t *row_i, int32_t *S)
{
    int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (int64_t r = 0; r < nrows; ++r) {
        int b = row_b[r], i = row_i[r];
        int64_t p = (int64_t)q_offset[b] + i;
        if (p < 0 || p >= kv_len[b] || kv_len[b] > Tk) continue;
        const int8_t *qI = q_idx + ((int64_t)b * Tq + i) * H_I * d_I;
        const int8_t *kI = k_idx + (int64_t)b * Tk * d_I;
        const int8_t *wr = w + b * w_stride_b + (int64_t)i * w_stride_q;
        rc |= orc_score_row(H_I, d_I, qI, kI, wr, p + 1, S + r * (int64_t)Tk);
    }
    return rc;
}

/* Block-granular Top-K: the scorer and the selection work on blocks of
 * positions instead of single positions ("Hybrid Sparse Attention for
 * Long-Context LLMs", section "Indexer + Top-K: How Fine-Grained Sparse Attention
 * Works", steps 1-2: scores against positions or blocks, the top K positions or
 * blocks kept). The pages do not say how a block is scored; the reading taken:
 * block j holds positions j*block .. j*block + block - 1, and its score is the
 * largest score among its candidates (positions below n), so a block is as
 * relevant as its best position. The min(K, nb) best of the nb = ceil(n / block)
 * blocks are kept under the order of single positions (higher score first,
 * lower block index on equal scores).
 * idx [K*block]: the kept blocks' candidate positions, ascending, -1 padded;
 * blk (nullable) [K]: the kept blocks, ascending, -1 padded; bsel (nullable) [K]:
 * their scores, INT32_MIN in the padding. block = 1 is orc_topk_row. */
void orc_block_topk_row(const int32_t *S, int64_t n, int block, int K, int32_t *idx,
                        int32_t *blk, int32_t *bsel)
{
    int64_t nb = n > 0 ? (n + block - 1) / block : 0;
    int32_t *bs = (int32_t *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(int32_t));
    for (int64_t j = 0; j < nb; ++j) {
        int32_t m = INT32_MIN;
        for (int64_t s = j * block; s < (j + 1) * block && s < n; ++s)
            if (S[s] > m) m = S[s];
        bs[j] = m;
    }
    int32_t *bi = (int32_t *)malloc((size_t)K * sizeof(int32_t));
    int32_t *bv = (int32_t *)malloc((size_t)K * sizeof(int32_t));
    orc_topk_row(bs, nb, K, bi, bv);
    for (int kk = 0; kk < K; ++kk) {
        for (int t = 0; t < block; ++t) {
            int64_t s = bi[kk] < 0 ? -1 : (int64_t)bi[kk] * block + t;
            idx[(int64_t)kk * block + t] = (s >= 0 && s < n) ? (int32_t)s : -1;
        }
        if (blk) blk[kk] = bi[kk];
        if (bsel) bsel[kk] = bv[kk];
    }
    free(bv);
    free(bi);
    free(bs);
}

/* Block-granular Top-K over given score rows (as orc_topk_rows): idx
 * [nrows][K*block], blk and bsel [nrows][K], both nullable. */
void orc_block_topk_rows(int64_t nrows, const int32_t *S, int64_t stride, const int64_t *n,
                         int block, int K, int32_t *idx, int32_t *blk, int32_t *bsel)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r)
        orc_block_topk_row(S + r * stride, n[r] > 0 ? n[r] : 0, block, K,
                           idx + r * (int64_t)K * block, blk ? blk + r * (int64_t)K : NULL,
                           bsel ? bsel + r * (int64_t)K : NULL);
}

/* Top-K over given score rows: row r has n[r] candidates (positions 0..n[r]-1)
 * stored at S + r*stride. n[r] <= 0 gives an all -1 row. */
void orc_topk_rows(int64_t nrows, const int32_t *S, int64_t stride, const int64_t *n, int K,
                   int32_t *idx, int32_t *sel)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r)
        orc_topk_row(S + r * stride, n[r] > 0 ? n[r] : 0, K, idx + r * (int64_t)K,
                     sel ? sel + r * (int64_t)K : NULL);
}

/* Attention + gate for a list of rows with the given index rows idx
 * [nrows][sets][K] (sets as in orc_attn_row). */
void orc_attn_rows(int Tq, int Tk, int Hq, int Hkv, int d, int K, int sets, const int32_t *kv_len,
                   const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const uint16_t *gate, const uint16_t *mix, double scale, int64_t nrows,
                   const int32_t *row_b,
                   const int32_t *row_i, const int32_t *idx, double *out, double *lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int b = row_b[r], i = row_i[r];
        int64_t qrow = (int64_t)b * Tq + i;
        /* a history longer than its allocation is not a valid one: no entry is read */
        int64_t kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
        orc_attn_row(Hq, Hkv, d, q + qrow * Hq * d, k + (int64_t)b * Tk * Hkv * d,
                     v + (int64_t)b * Tk * Hkv * d, kvl, idx + r * (int64_t)sets * K, K, sets,
                     gate ? gate + qrow * Hq * d : NULL, mix ? mix + qrow * Hq * d : NULL, scale,
                     out + r * (int64_t)Hq * d, lse ? lse + r * (int64_t)Hq : NULL);
    }
}

/* orc_attn_rows with fp32 q, k, v and gate (sources drawn in fp32, such as the
 * Tiny configuration's), no mix; the same arithmetic in fp64. */
void orc_attn_rows_f32(int Tq, int Tk, int Hq, int Hkv, int d, int K, int sets,
                       const int32_t *kv_len, const float *q, const float *k, const float *v,
                       const float *gate, double scale, int64_t nrows, const int32_t *row_b,
                       const int32_t *row_i, const int32_t *idx, double *out, double *lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int b = row_b[r], i = row_i[r];
        int64_t qrow = (int64_t)b * Tq + i;
        int64_t kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
        orc_attn_row_ld(Hq, Hkv, d, q + qrow * Hq * d, k + (int64_t)b * Tk * Hkv * d,
                        v + (int64_t)b * Tk * Hkv * d, kvl, idx + r * (int64_t)sets * K, K, sets,
                        gate ? gate + qrow * Hq * d : NULL, NULL, scale,
                        out + r * (int64_t)Hq * d, lse ? lse + r * (int64_t)Hq : NULL,
                        orc_ld_f32);
    }
}

/* The whole layer for a list of rows: score -> Top-K -> attention -> gate.
 * With block > 1 the selection keeps K blocks of that many positions
 * (orc_block_topk_row): index rows of K*block positions, sel the K kept
 * blocks' scores; with block <= 1 single positions (K of each).
 * Index sets: sets divides Hq and H_I; sets = 1, one set per query row shared
 * by every head; sets = Hkv, one per key/value head; sets = Hq, one per query
 * head ("Hybrid Sparse Attention for Long-Context LLMs", the pseudocode of the
 * Indexer + Top-K section keeps indices per head; "How Fine-Grained Sparse
 * Attention Reshapes ...", the runtime section's pseudocode likewise). Query
 * head h attends over set h / (Hq/sets). Reading taken for the per-set scorer:
 * the H_I indexer heads are split into sets consecutive groups of H_I/sets
 * heads, and set g is scored by group g alone (its heads and their weights).
 * idx [nrows][sets][K or K*block], sel [nrows][sets][K], out [nrows][Hq][d],
 * lse [nrows][Hq]. Invalid rows give
 * idx = -1, sel = INT32_MIN, an attention output of 0 (out = 0 unless mixed)
 * and lse = -inf. Returns ORC_OVERFLOW if a score overflowed int32. */
int orc_layer_rows(int Tq, int Tk, int Hq, int Hkv, int d, int H_I, int d_I, int K,
                   int block, int sets, const int32_t *q_offset, const int32_t *kv_len, const int8_t *q_idx,
                   const int8_t *k_idx, const int8_t *w, int64_t w_stride_b,
                   int64_t w_stride_q, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, const uint16_t *gate, const uint16_t *mix, double scale,
                   int64_t nrows, const int32_t *row_b, const int32_t *row_i, int32_t *idx,
                   int32_t *sel, double *out, double *lse)
{
    int rc = ORC_OK;
    const int bl = block > 1 ? block : 1;
    const int KI = K * bl;   /* positions per index row */
    const int ns = sets > 1 ? sets : 1;
    const int Hg = H_I / ns; /* indexer heads per index set */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (int64_t r = 0; r < nrows; ++r) {
        int b = row_b[r], i = row_i[r];
        int64_t p = (int64_t)q_offset[b] + i;
        int32_t *irow = idx + r * (int64_t)ns * KI;
        int32_t *srow = sel ? sel + r * (int64_t)ns * K : NULL;
        double *orow = out + r * (int64_t)Hq * d;
        double *lrow = lse ? lse + r * (int64_t)Hq : NULL;
        if (p < 0 || p >= kv_len[b] || kv_len[b] > Tk) {
            int64_t qrow = (int64_t)b * Tq + i;
            for (int j = 0; j < ns * KI; ++j) irow[j] = -1;
            for (int j = 0; j < ns * K; ++j) if (srow) srow[j] = INT32_MIN;
            for (int64_t j = 0; j < (int64_t)Hq * d; ++j)
                orow[j] = gate ? orc_gate(0.0, orc_bf16(gate[qrow * Hq * d + j]),
                                          mix ? mix + qrow * Hq * d : NULL, j)
                               : 0.0;
            if (lrow) for (int h = 0; h < Hq; ++h) lrow[h] = -INFINITY;
            continue;
        }
        int32_t *S = (int32_t *)malloc((size_t)(p + 1) * sizeof(int32_t));
        const int8_t *kI = k_idx + (int64_t)b * Tk * d_I;
        const int8_t *wr = w + b * w_stride_b + (int64_t)i * w_stride_q;
        for (int gs = 0; gs < ns; ++gs) {
            /* index set gs: scored by indexer heads gs*Hg .. gs*Hg + Hg - 1 */
            const int8_t *qI = q_idx + (((int64_t)b * Tq + i) * H_I + (int64_t)gs * Hg) * d_I;
            int32_t *ir = irow + (int64_t)gs * KI;
            int32_t *sr = srow ? srow + (int64_t)gs * K : NULL;
            rc |= orc_score_row(Hg, d_I, qI, kI, wr + gs * Hg, p + 1, S);
            if (bl > 1)
                orc_block_topk_row(S, p + 1, bl, K, ir, NULL, sr);
            else
                orc_topk_row(S, p + 1, K, ir, sr);
        }
        free(S);
        int64_t qrow = (int64_t)b * Tq + i;
        orc_attn_row(Hq, Hkv, d, q + qrow * Hq * d, k + (int64_t)b * Tk * Hkv * d,
                     v + (int64_t)b * Tk * Hkv * d, kv_len[b], irow, KI, ns,
                     gate ? gate + qrow * Hq * d : NULL, mix ? mix + qrow * Hq * d : NULL, scale,
                     orow, lrow);
    }
    return rc;
}

/* Append new rows to a per-sequence cache (the "append" step above).
 * src [B][Tn][row_bytes], cache [B][Tk][row_bytes]; kv_len [B] the current
 * history lengths, n_new [B] the rows to append (NULL: Tn for every sequence).
 * A length outside 0..Tk is taken as the nearest end of that range and a count
 * outside 0..Tn likewise. Row t of sequence b goes to cache row kv_len[b] + t
 * for t < n_new[b]; rows that would land at or past Tk are dropped. Writes, when
 * non-NULL, q_offset_out[b] = the old length (the position of the first new row)
 * and kv_len_out[b] = the new length, min(old + n, Tk). */
void orc_kv_append(int B, int Tn, int Tk, int64_t row_bytes, const uint8_t *src,
                   uint8_t *cache, const int32_t *kv_len, const int32_t *n_new,
                   int32_t *q_offset_out, int32_t *kv_len_out)
{
    for (int b = 0; b < B; ++b) {
        int64_t old = kv_len[b] < 0 ? 0 : (kv_len[b] > Tk ? Tk : kv_len[b]);
        int64_t n = n_new ? n_new[b] : Tn;
        if (n < 0) n = 0;
        if (n > Tn) n = Tn;
        for (int64_t t = 0; t < n; ++t) {
            int64_t dst = old + t;
            if (dst >= Tk) break;
            memcpy(cache + ((int64_t)b * Tk + dst) * row_bytes,
                   src + ((int64_t)b * Tn + t) * row_bytes, (size_t)row_bytes);
        }
        if (q_offset_out) q_offset_out[b] = (int32_t)old;
        if (kv_len_out) kv_len_out[b] = (int32_t)(old + n < Tk ? old + n : Tk);
    }
}

/* Gradients of the gated sparse attention (the training direction of the
 * layer: "Hybrid Sparse Attention for Long-Context LLMs", section "Engineering
 * and Evaluation Recommendations", training side; the scorer, trained by
 * distillation, is not differentiated here). For the forward of orc_attn_row
 * (one index set) and an output gradient dy, by the chain rule on
 *   l_t = scale q.k[s_t],  P = softmax(l),  o = sum_t P_t v[s_t],
 *   y = s*o + (1 - s)*x,   s = sigmoid(G)   (s = 1 and no x when ungated):
 *   do = s*dy;  dG = dy*(o - x)*s*(1 - s);  dx = (1 - s)*dy;
 *   dP_t = do.v[s_t];  dl_t = P_t*(dP_t - sum_u P_u dP_u);
 *   dq = scale * sum_t dl_t k[s_t];  dk[s_t] += scale*dl_t*q;  dv[s_t] += P_t*do,
 * summed over the query heads that share a key/value head and over every
 * occurrence of a position in an index row. Rows B x Tq with idx
 * [B][Tq][sets][K] (sets as in orc_attn_row: query head h reads set
 * h / (Hq/sets)); entries outside 0..kv_len-1 are skipped. All outputs are overwritten (fp64):
 * dq, dgate, dmix [B][Tq][Hq][d] (dgate, dmix nullable; used only with gate /
 * mix), dk, dv [B][Tk][Hkv][d]. */
void orc_attn_bwd(int B, int Tq, int Tk, int Hq, int Hkv, int d, int K, int sets,
                  const int32_t *kv_len,
                  const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *gate,
                  const uint16_t *mix, const int32_t *idx, const uint16_t *dy, double scale,
                  double *dq, double *dk, double *dv, double *dgate, double *dmix)
{
    int G = Hq / Hkv;
    int ns = sets > 1 ? sets : 1;
    int hps = Hq / ns;   /* query heads per index set */
    memset(dk, 0, (size_t)B * Tk * Hkv * d * sizeof(double));
    memset(dv, 0, (size_t)B * Tk * Hkv * d * sizeof(double));
    double *P = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    double *dP = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    double *o = (double *)malloc((size_t)d * sizeof(double));
    double *dO = (double *)malloc((size_t)d * sizeof(double));
    for (int b = 0; b < B; ++b) {
        /* a history longer than its allocation is not a valid one: no entry is read */
        int64_t kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
        const uint16_t *kb = k + (int64_t)b * Tk * Hkv * d, *vb = v + (int64_t)b * Tk * Hkv * d;
        for (int i = 0; i < Tq; ++i) {
            int64_t row = (int64_t)b * Tq + i;
            for (int h = 0; h < Hq; ++h) {
                int g = h / G;
                const int32_t *ir = idx + (row * ns + h / hps) * K;   /* this head's index set */
                int64_t hb = (row * Hq + h) * d;
                /* softmax weights over the valid entries */
                double m = -INFINITY;
                for (int t = 0; t < K; ++t) {
                    int64_t st = ir[t];
                    if (st < 0 || st >= kvl) { P[t] = -INFINITY; continue; }
                    double dot = 0.0;
                    for (int j = 0; j < d; ++j)
                        dot += orc_bf16(q[hb + j]) * orc_bf16(kb[(st * Hkv + g) * d + j]);
                    P[t] = scale * dot;
                    if (P[t] > m) m = P[t];
                }
                double Z = 0.0;
                for (int t = 0; t < K; ++t) {
                    P[t] = (m == -INFINITY || P[t] == -INFINITY) ? 0.0 : exp(P[t] - m);
                    Z += P[t];
                }
                for (int t = 0; t < K; ++t) if (Z > 0.0) P[t] /= Z;
                for (int j = 0; j < d; ++j) o[j] = 0.0;
                for (int t = 0; t < K; ++t) {
                    if (P[t] == 0.0) continue;
                    int64_t st = ir[t];
                    for (int j = 0; j < d; ++j) o[j] += P[t] * orc_bf16(vb[(st * Hkv + g) * d + j]);
                }
                /* the gate */
                for (int j = 0; j < d; ++j) {
                    double gy = orc_bf16(dy[hb + j]);
                    if (gate) {
                        double sg = 1.0 / (1.0 + exp(-orc_bf16(gate[hb + j])));
                        double x = mix ? orc_bf16(mix[hb + j]) : 0.0;
                        dO[j] = sg * gy;
                        if (dgate) dgate[hb + j] = gy * (o[j] - x) * sg * (1.0 - sg);
                        if (dmix && mix) dmix[hb + j] = (1.0 - sg) * gy;
                    } else {
                        dO[j] = gy;
                    }
                }
                /* the softmax */
                double delta = 0.0;
                for (int t = 0; t < K; ++t) {
                    dP[t] = 0.0;
                    int64_t st = ir[t];
                    if (st < 0 || st >= kvl) continue;
                    for (int j = 0; j < d; ++j) dP[t] += dO[j] * orc_bf16(vb[(st * Hkv + g) * d + j]);
                    delta += P[t] * dP[t];
                }
                for (int j = 0; j < d; ++j) dq[hb + j] = 0.0;
                for (int t = 0; t < K; ++t) {
                    int64_t st = ir[t];
                    if (st < 0 || st >= kvl) continue;
                    double dl = P[t] * (dP[t] - delta);
                    double *dkr = dk + (((int64_t)b * Tk + st) * Hkv + g) * d;
                    double *dvr = dv + (((int64_t)b * Tk + st) * Hkv + g) * d;
                    for (int j = 0; j < d; ++j) {
                        dq[hb + j] += scale * dl * orc_bf16(kb[(st * Hkv + g) * d + j]);
                        dkr[j] += scale * dl * orc_bf16(q[hb + j]);
                        dvr[j] += P[t] * dO[j];
                    }
                }
            }
        }
    }
    free(dO);
    free(o);
    free(dP);
    free(P);
}

/* Gradients of the indexer's distillation loss (the training of the scorer:
 * "How Fine-Grained Sparse Attention Reshapes Long-Context Architecture in
 * Large Models", section "How Indexer + Top-K Works at Runtime" -- the
 * indexer's selection distribution is distilled from a full-attention teacher;
 * "Hybrid Sparse Attention for Long-Context LLMs", section "Engineering and
 * Evaluation Recommendations", training side -- the scorer is trained jointly).
 * The pages give no loss; the reading taken: for query row i with index row
 * idx[i][0..K) (entries outside 0..p or past the history are skipped), the
 * scorer's distribution is the softmax over the entries of z_t = tau * S_t,
 *   S_t = sum_h w_h max(0, d_ht),  d_ht = qI[i,h] . kI[idx_t],
 * the teacher's weights T_t (>= 0) are given per entry, and the loss is
 *   L_i = sum_t T_t (log T_t - log p_t)   (0 log 0 = 0),
 * the Kullback-Leibler divergence when T sums to 1. With q, k and w taken as
 * real numbers (their int8 values) and the ReLU's derivative 0 at 0:
 *   g_t = dL/dS_t = tau (p_t sum_u T_u - T_t),
 *   dw[i,h] = sum_t g_t max(0, d_ht),
 *   dq[i,h,:] = w_h sum_t g_t [d_ht > 0] kI[idx_t],
 *   dk[idx_t,:] += g_t sum_h w_h [d_ht > 0] qI[i,h]   (over every row and entry).
 * With sets > 1 index sets (a divisor of H_I; the reading of the forward's
 * per-head sets carried over) set g is the scorer of indexer heads
 * g*H_I/sets .. (g+1)*H_I/sets - 1 (their weights included) over its own index
 * rows and teacher: each set's loss is the one above with H_I/sets heads, dq
 * and dw of a head come from its set alone, and dk sums over every set.
 * q_idx [B][Tq][H_I][d_I], k_idx [B][Tk][d_I], w at b*w_stride_b + i*w_stride_q
 * (+h), idx and T [B][sets][Tq][K]. Outputs (fp64, overwritten): loss
 * [B][sets][Tq] (NULL allowed), dq [B][Tq][H_I][d_I], dk [B][Tk][d_I], dw
 * [B][Tq][H_I]. Invalid rows (p outside 0..kv_len-1, or kv_len > Tk) and rows
 * without a valid entry give zeros. */
void orc_indexer_bwd(int B, int Tq, int Tk, int H_I, int d_I, int K, int sets,
                     const int32_t *q_offset, const int32_t *kv_len, const int8_t *q_idx,
                     const int8_t *k_idx, const int8_t *w, int64_t w_stride_b,
                     int64_t w_stride_q, const int32_t *idx, const double *T, double tau,
                     double *loss, double *dq, double *dk, double *dw)
{
    int ns = sets > 1 ? sets : 1;
    int Hs = H_I / ns;  /* indexer heads of one set */
    memset(dk, 0, (size_t)B * Tk * d_I * sizeof(double));
    double *z = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    int64_t *dd = (int64_t *)malloc((size_t)(K > 0 ? K : 1) * H_I * sizeof(int64_t));
    for (int b = 0; b < B; ++b) {
        for (int gs = 0; gs < ns; ++gs)
        for (int i = 0; i < Tq; ++i) {
            int64_t row = (int64_t)b * Tq + i;
            int64_t srow = ((int64_t)b * ns + gs) * Tq + i;  /* the set's index row */
            int64_t p = (int64_t)q_offset[b] + i;
            const int8_t *qI = q_idx + (row * H_I + (int64_t)gs * Hs) * d_I;
            const int8_t *wr = w + b * w_stride_b + (int64_t)i * w_stride_q + gs * Hs;
            const int32_t *ir = idx + srow * K;
            const double *Tr = T + srow * K;
            double *dqr = dq + (row * H_I + (int64_t)gs * Hs) * d_I;
            double *dwr = dw + row * H_I + gs * Hs;
            for (int j = 0; j < Hs * d_I; ++j) dqr[j] = 0.0;
            for (int h = 0; h < Hs; ++h) dwr[h] = 0.0;
            if (loss) loss[srow] = 0.0;
            int valid_row = p >= 0 && p < kv_len[b] && kv_len[b] <= Tk;
            if (!valid_row) continue;
            /* scores of the entries (exact, int64) and the softmax of tau*S */
            double m = -INFINITY;
            for (int t = 0; t < K; ++t) {
                int64_t s = ir[t];
                if (s < 0 || s > p) { z[t] = -INFINITY; continue; }
                int64_t S = 0;
                for (int h = 0; h < Hs; ++h) {
                    int64_t d = 0;
                    for (int j = 0; j < d_I; ++j)
                        d += (int64_t)qI[h * d_I + j] * (int64_t)k_idx[((int64_t)b * Tk + s) * d_I + j];
                    dd[(int64_t)t * Hs + h] = d;
                    S += (int64_t)wr[h] * (d > 0 ? d : 0);
                }
                z[t] = tau * (double)S;
                if (z[t] > m) m = z[t];
            }
            if (m == -INFINITY) continue;   /* no valid entry */
            double Z = 0.0, Tsum = 0.0;
            for (int t = 0; t < K; ++t) {
                if (z[t] == -INFINITY) continue;
                Z += exp(z[t] - m);
                Tsum += Tr[t];
            }
            double logZ = m + log(Z);
            double L = 0.0;
            for (int t = 0; t < K; ++t) {
                if (z[t] == -INFINITY) continue;
                double logp = z[t] - logZ;
                double pt = exp(logp);
                if (Tr[t] > 0.0) L += Tr[t] * (log(Tr[t]) - logp);
                double g = tau * (pt * Tsum - Tr[t]);
                int64_t s = ir[t];
                const int8_t *kr = k_idx + ((int64_t)b * Tk + s) * d_I;
                double *dkr = dk + ((int64_t)b * Tk + s) * d_I;
                for (int h = 0; h < Hs; ++h) {
                    int64_t d = dd[(int64_t)t * Hs + h];
                    dwr[h] += g * (double)(d > 0 ? d : 0);
                    if (d <= 0) continue;
                    for (int j = 0; j < d_I; ++j) {
                        dqr[h * d_I + j] += g * (double)wr[h] * (double)kr[j];
                        dkr[j] += g * (double)wr[h] * (double)qI[h * d_I + j];
                    }
                }
            }
            if (loss) loss[srow] = L;
        }
    }
    free(dd);
    free(z);
}

int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
