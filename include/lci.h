/*
 * lci.h -- C ABI of the MI355X (gfx950) gated fine-grained sparse attention library.
 *
 * The layer, as the pages describe it ("Hybrid Sparse Attention for Long-Context
 * LLMs", section "Indexer + Top-K: How Fine-Grained Sparse Attention Works",
 * steps 1-4; "Optimizing LLM Long-Context Inference with Indexed Top-K Sparse
 * Attention", section "Interface Design for Practical Implementation"; "From
 * Linear Attention to Gated Sparse Attention", section 2):
 *   1. a light indexer scores every causal history position for each query,
 *   2. Top-K keeps the K best positions,
 *   3. exact softmax attention runs over those K keys/values only,
 *   4. a sigmoid gate multiplies the output elementwise, or weighs it against
 *      the output of the layer's other (linear or compressed) branch.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. Tensors are
 *     dense and row-major in the shapes written next to each argument; the
 *     library never frees, keeps or retains them after the call returns.
 *   - Inputs are never written. Outputs are fully overwritten over their whole
 *     documented extent (scores: see lci_idx_score).
 *   - Every call is asynchronous: it validates its arguments on the host,
 *     enqueues kernels on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and returns. There is no host synchronisation, no device
 *     memory allocation and no global mutable state except the per-thread last
 *     HIP error (and the kernel timing log, while timing is switched on). Calls are reentrant; calls that share output or workspace
 *     buffers must be ordered by the caller.
 *   - An invalid argument returns an error code synchronously and enqueues
 *     nothing. The contents of device arrays (q_offset, kv_len, idx) cannot be
 *     checked on the host; the kernels treat out-of-range values as documented
 *     below and never read or write outside the buffers described here.
 *   - bf16 tensors hold bfloat16 bit patterns (lci_bf16 = uint16_t storage).
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bit-identical outputs (no floating-point atomics anywhere).
 *
 * Positions. Query row i of sequence b sits at absolute position
 * p = q_offset[b] + i. Its candidate set is every history position 0..p, its
 * own position included (the key/value cache is kept whole so any past
 * position can be selected: "Hybrid Sparse Attention ...", section "Why Keep
 * Linear Attention ...", item 3). A row is VALID when 0 <= p < kv_len[b] <= Tk;
 * an invalid row produces idx = -1, out = 0 and lse = -inf.
 *
 * Indexer arithmetic (the pages give no formula; reading taken):
 *   S[b,i,s] = sum_{h < H_I} w[b,i,h] * max(0, sum_{j < d_I} qI[b,i,h,j] * kI[b,s,j])
 * with int8 qI, kI, w and exact int32 accumulation. |S| <= H_I*d_I*128*128*128,
 * which fits int32 whenever H_I*d_I <= 1024 (checked: LCI_ERR_OVERFLOW_RISK).
 *
 * Top-K order: higher score first; on equal scores the lower position wins.
 * The selected positions are written in ascending position order, followed by
 * -1 padding when the row has fewer than K candidates (then all are selected,
 * and the layer equals dense causal attention for that row).
 *
 * Supported shapes: d in {64, 128}; Hkv in {1, 2, 4, 8}; G = Hq/Hkv in
 * {1, 2, 4, 8, 16}; H_I in {1, 2, 4, 8, 16}; d_I in {32, 64, 128} with
 * H_I*d_I <= 1024; 1 <= K <= 4096; B, Tq, Tk >= 1; Tk < 2^31 / max(4, d_I).
 */
#ifndef LCI_H
#define LCI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCI_ABI_VERSION 5

typedef uint16_t lci_bf16;

typedef enum lci_status {
    LCI_OK = 0,
    LCI_ERR_NULL = -1,          /* a required pointer is NULL                           */
    LCI_ERR_SHAPE = -2,         /* a size is out of range or sizes are inconsistent     */
    LCI_ERR_UNSUPPORTED = -3,   /* a valid shape that no kernel here implements         */
    LCI_ERR_OVERFLOW_RISK = -4, /* H_I*d_I > 1024: an int32 score could overflow        */
    LCI_ERR_WORKSPACE = -5,     /* workspace NULL or smaller than lci_workspace_bytes() */
    LCI_ERR_HIP = -6,           /* a HIP call failed; see lci_last_hip_error()          */
    LCI_ERR_ALIGN = -7,         /* a pointer is not 16-byte aligned                     */
    LCI_ERR_SCRATCH = -8        /* lci_decode_fwd_noalloc: the call needs more workspace */
                                /* than the static scratch array holds                  */
} lci_status;

/* Geometry shared by every entry point. */
typedef struct lci_geom {
    int32_t B;                 /* sequences                                              */
    int32_t Tq;                /* query rows per sequence                                */
    int32_t Tk;                /* history rows allocated per sequence (row stride)       */
    int32_t Hq, Hkv, d;        /* query heads, key/value heads, head dim                 */
    int32_t H_I, d_I;          /* indexer heads, indexer dim                             */
    int32_t K;                 /* positions kept per query row                           */
    const int32_t *q_offset;   /* device [B]: position of query row 0 of each sequence   */
    const int32_t *kv_len;     /* device [B]: valid history rows of each sequence        */
    int32_t block;             /* selection granularity: 0 or 1 = single positions; a    */
                               /* power of two 2..256 = blocks of that many positions,   */
                               /* K then counts blocks (see lci_topk_select)             */
    int32_t sets;              /* index sets per query row: 0 or 1 = one set shared by   */
                               /* every head; S > 1 = S sets, query head h reading set   */
                               /* h / (Hq/S): Hkv = one per key/value head, Hq = one per */
                               /* query head (see below)                                 */
} lci_geom;

/* Entry ids for lci_workspace_bytes. */
enum {
    LCI_ENTRY_IDX_SCORE = 0,
    LCI_ENTRY_TOPK_SELECT = 1,
    LCI_ENTRY_SPARSE_ATTN = 2,
    LCI_ENTRY_PREFILL = 3,
    LCI_ENTRY_DECODE = 4,
    LCI_ENTRY_SPARSE_ATTN_BWD = 5,
    LCI_ENTRY_INDEXER_BWD = 6
};

/* Indexer scoring (step 1). "Hybrid Sparse Attention ...", section "Indexer +
 * Top-K ...", step 1 and the scoring step of its pseudocode; "Optimizing ...",
 * section "Two Engineering Considerations", item 1 (the scorer must stay cheap:
 * few heads of low dimension).
 *   q_idx  int8 [B, Tq, H_I, d_I]
 *   k_idx  int8 [B, Tk, d_I]
 *   w      int8, element (b, i, h) at w[b*w_stride_b + i*w_stride_q + h];
 *          strides in elements, 0 broadcasts (a [H_I] vector uses 0, 0)
 *   scores int32 [B, Tq, Tk] out: S[b,i,s] for s <= p of every valid row; all
 *          other elements are left unwritten. With g->sets = S > 1 (S must
 *          divide H_I, else SHAPE) set j is scored by indexer heads j*H_I/S ..
 *          (j+1)*H_I/S - 1 alone and scores is int32 [B, S, Tq, Tk].
 * Errors: NULL, SHAPE, UNSUPPORTED, OVERFLOW_RISK, HIP. Workspace: none. */
lci_status lci_idx_score(const lci_geom *g, const int8_t *q_idx, const int8_t *k_idx,
                         const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                         int32_t *scores, void *stream);

/* Top-K selection (step 2). "Hybrid Sparse Attention ...", step 2 and the
 * selection step of its pseudocode; "Optimizing ...", section "Interface
 * Design" (Top-K over the last, position axis of each score row).
 *   scores     int32 [B, Tq, Tk]: only s <= p of each row is read
 *   idx        int32 [B, Tq, K] out: selected positions ascending, -1 padded
 *   sel_scores int32 [B, Tq, K] out, nullable: the score of each idx entry,
 *              INT32_MIN in the padding
 * With g->sets = S > 1 every array gains a set axis after B (scores
 * [B, S, Tq, Tk], idx [B, S, Tq, ...], sel_scores [B, S, Tq, K]) and each
 * set's rows are selected like those of one set.
 * Block-granular selection (g->block = b > 1; same steps: the scorer rates
 * positions or blocks and the top K positions or blocks are kept): block j
 * holds positions j*b .. j*b + b - 1 and rates as its best causal position;
 * the K best blocks are kept (higher score, then lower block index). idx is
 * then int32 [B, Tq, K*b]: the kept blocks' causal positions ascending, -1
 * padded; sel_scores [B, Tq, K] the kept blocks' scores. Requires K*b <= 4096
 * (SHAPE) and ceil(Tk / b) <= 8192 (UNSUPPORTED).
 *   workspace  device scratch of at least lci_workspace_bytes(LCI_ENTRY_TOPK_SELECT)
 * Errors: NULL, SHAPE, WORKSPACE, HIP. */
lci_status lci_topk_select(const lci_geom *g, const int32_t *scores, int32_t *idx,
                           int32_t *sel_scores, void *workspace, size_t ws_bytes,
                           void *stream);

/* Sparse exact attention + sigmoid gate (steps 3-4). "Hybrid Sparse Attention
 * ...", steps 3-4 and the attention and gating steps of its pseudocode (softmax
 * of the 1/sqrt(d)-scaled dot products with the selected keys, weighting the
 * selected values; the gate multiplies the result, or mixes it with the linear
 * branch's output); "From Linear Attention ...", section 2 (a query-dependent
 * gate multiplies the attention output); "How Fine-Grained Sparse Attention
 * Reshapes ...", section "How Indexer + Top-K Works at Runtime" (the gate
 * mixes the exact result with a compressed global summary).
 *   q, gate  bf16 [B, Tq, Hq, d]; gate nullable (ungated)
 *   mix      bf16 [B, Tq, Hq, d], nullable: the other branch's output x to mix
 *            with; requires gate (NULL error otherwise)
 *   k, v     bf16 [B, Tk, Hkv, d]; query head h reads key/value head h / (Hq/Hkv)
 *   idx      int32 [B, Tq, K*max(1, g->block)]: positions to attend; entries
 *            outside 0..kv_len[b]-1 (the -1 padding) are skipped; duplicates count
 *            once each; order is free
 *   out      bf16 [B, Tq, Hq, d] out: s*o, or s*o + (1-s)*x with mix, where
 *            s = sigmoid(gate) (1 ungated) and o = softmax(scale*q.k) v (0 for
 *            a row without entries); fp32 arithmetic, rounded to nearest even
 *   lse      fp32 [B, Tq, Hq] out, nullable: natural log of the softmax
 *            denominator of scale*q.k (-inf for a row without entries)
 *   softmax_scale  positive and finite (1/sqrt(d) in the pages), else SHAPE
 *   workspace scratch of at least lci_workspace_bytes(LCI_ENTRY_SPARSE_ATTN)
 * Errors: NULL, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN, HIP. */
lci_status lci_sparse_attn_fwd(const lci_geom *g, const lci_bf16 *q, const lci_bf16 *k,
                               const lci_bf16 *v, const int32_t *idx, const lci_bf16 *gate,
                               const lci_bf16 *mix, float softmax_scale, lci_bf16 *out,
                               float *lse, void *workspace, size_t ws_bytes, void *stream);

/* Index sets (g->sets = S > 1). The pages' pseudocode keeps one index row per
 * head ("Hybrid Sparse Attention ...", the pseudocode of the Indexer + Top-K
 * section, index shape [B, H, Lq, top_k]; "How Fine-Grained Sparse Attention
 * Reshapes ...", section "How Indexer + Top-K Works at Runtime", index shape
 * [B, Hq, K]). Query head h attends over set h / (Hq/S): S = Hkv gives one set
 * per key/value head, S = Hq one per query head (S must divide Hq, else SHAPE).
 * The H_I indexer heads split into S consecutive groups of H_I/S heads (S must
 * divide H_I, else SHAPE); set j is scored by group j alone, with its heads'
 * weights, and selected like a shared set. Index rows are then int32 [B, S,
 * Tq, K*max(1, block)] (idx_out of the fused entries, idx of
 * lci_sparse_attn_fwd, lci_sparse_attn_bwd); lci_idx_score, lci_topk_select and
 * lci_indexer_bwd take the same set axis. */

/* Fused prefill: steps 1-4 for many query rows per sequence in one call
 * ("Hybrid Sparse Attention ...", section "Engineering and Evaluation
 * Recommendations": Top-K and gather need fused kernels; chunked long prefill).
 * Arguments as in the three calls above; idx_out (int32 [B, Tq, K*max(1,
 * g->block)]) and lse are nullable. Results equal lci_idx_score ->
 * lci_topk_select -> lci_sparse_attn_fwd on the same inputs (idx bit-exact),
 * with single positions or blocks as g->block says.
 * Errors: NULL, SHAPE, UNSUPPORTED, OVERFLOW_RISK, WORKSPACE, ALIGN, HIP. */
lci_status lci_prefill_fwd(const lci_geom *g, const int8_t *q_idx, const int8_t *k_idx,
                           const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                           const lci_bf16 *q, const lci_bf16 *k, const lci_bf16 *v,
                           const lci_bf16 *gate, const lci_bf16 *mix, float softmax_scale,
                           lci_bf16 *out, float *lse, int32_t *idx_out, void *workspace,
                           size_t ws_bytes, void *stream);

/* Fused decode: one query row per sequence (Tq == 1) over a long history, with
 * the history split across workgroups for scoring, an exact Top-K taken from
 * the list of positions at or above a threshold estimated from every 32nd
 * score (a whole-row selection where that list falls short of K or overflows),
 * and split-K attention combined in a fixed order ("How Fine-Grained Sparse
 * Attention Reshapes ...", section "Engineering Practices": per-step decode
 * work decoupled from context length). Same arguments and results as
 * lci_prefill_fwd. With block-granular selection (g->block > 1) the one row
 * runs the prefill path (scores of the whole row, then the block selection).
 * Errors: NULL, SHAPE (Tq != 1 included), UNSUPPORTED, OVERFLOW_RISK,
 * WORKSPACE, ALIGN, HIP. */
lci_status lci_decode_fwd(const lci_geom *g, const int8_t *q_idx, const int8_t *k_idx,
                          const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                          const lci_bf16 *q, const lci_bf16 *k, const lci_bf16 *v,
                          const lci_bf16 *gate, const lci_bf16 *mix, float softmax_scale,
                          lci_bf16 *out, float *lse, int32_t *idx_out, void *workspace,
                          size_t ws_bytes, void *stream);

/* Allocation-free fused decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results and errors as lci_decode_fwd, without
 * the workspace: the call carves its workspace out of a static device array of
 * LCI_NOALLOC_SCRATCH_MIB MiB (lci_noalloc_scratch_bytes()) that the library's
 * code object holds; each GPU the library runs on keeps its own copy until the
 * process ends. The call allocates and frees nothing; its first call on a
 * device looks up that device's copy (hipGetSymbolAddress). A geometry whose
 * lci_workspace_bytes(LCI_ENTRY_DECODE) exceeds the array returns
 * LCI_ERR_SCRATCH and enqueues nothing (Decode 128K, 64 x 131072 positions,
 * and Decode 1M, 8 x 1048576, both fit: about 13 B per history position, the
 * split-K partials included). Every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller. The array keeps the last call's contents; the decode kernels
 * read no workspace byte they have not written in the same call. */
#define LCI_NOALLOC_SCRATCH_MIB 128
size_t lci_noalloc_scratch_bytes(void);
lci_status lci_decode_fwd_noalloc(const lci_geom *g, const int8_t *q_idx, const int8_t *k_idx,
                                  const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                                  const lci_bf16 *q, const lci_bf16 *k, const lci_bf16 *v,
                                  const lci_bf16 *gate, const lci_bf16 *mix,
                                  float softmax_scale, lci_bf16 *out, float *lse,
                                  int32_t *idx_out, void *stream);

/* Append new rows to the key, value and indexer-key caches ("Hybrid Sparse
 * Attention ...", section "Engineering and Evaluation Recommendations": long
 * prompts are prefilled in chunks that reuse the cached scorer inputs). The
 * caches are the k, v and k_idx arguments of the calls above; after an append,
 * a prefill or decode call with q_offset = q_offset_out and kv_len = kv_len_out
 * takes the appended rows as its query rows and scores and attends against the
 * whole cached history, earlier rows included, without recomputing them.
 *   g        B (at most 65535); Tq = Tn, rows per sequence of the new tensors; Tk, the cache
 *            capacity (row stride); Hkv, d, d_I; g->kv_len (device [B]) the
 *            current history lengths. Hq, H_I, K and q_offset are not used
 *            (q_offset may be NULL).
 *   k_new, v_new  bf16 [B, Tn, Hkv, d]; kI_new int8 [B, Tn, d_I]
 *   n_new    int32 device [B], nullable: rows of sequence b to append (NULL:
 *            all Tn); values outside 0..Tn are taken at the nearest end
 *   k_cache, v_cache  bf16 [B, Tk, Hkv, d]; kI_cache int8 [B, Tk, d_I]:
 *            row t < n of sequence b is written at position kv_len[b] + t;
 *            rows that would land at or past Tk are not written (a length
 *            outside 0..Tk is taken at the nearest end); nothing else changes
 *   q_offset_out  int32 device [B] out, nullable: the old length, i.e. the
 *            position of the first appended row
 *   kv_len_out    int32 device [B] out, nullable: min(old + n, Tk). It may be
 *            g->kv_len itself (the lengths are updated after every row is
 *            copied); q_offset_out and kv_len_out must differ (else SHAPE).
 * Hkv*d must be a multiple of 8 and d_I of 16 (16-byte rows), else
 * UNSUPPORTED. Two kernel launches, no workspace.
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, HIP. */
lci_status lci_kv_append(const lci_geom *g, const lci_bf16 *k_new, const lci_bf16 *v_new,
                         const int8_t *kI_new, const int32_t *n_new, lci_bf16 *k_cache,
                         lci_bf16 *v_cache, int8_t *kI_cache, int32_t *q_offset_out,
                         int32_t *kv_len_out, void *stream);

/* Gradients of sparse attention + gate (the training direction of steps 3-4;
 * "Hybrid Sparse Attention ...", section "Engineering and Evaluation
 * Recommendations", training side). For the forward of lci_sparse_attn_fwd
 * on the same inputs and an output gradient dy, by the chain rule:
 *   do = s*dy, dgate = dy*(o - x)*s*(1 - s), dmix = (1 - s)*dy (s = sigmoid(gate),
 *   s = 1 ungated), dP_t = do.v_t, delta = do.o, dl_t = P_t (dP_t - delta),
 *   dq = scale sum_t dl_t k_t, dk_t += scale dl_t q, dv_t += P_t do,
 * summed over the query heads of a key/value head and over every occurrence of
 * a position in an index row. The scorer (indexer) gets no gradient here.
 *   q, k, v, idx, gate, mix, softmax_scale: as in lci_sparse_attn_fwd, index
 *            sets included (g->sets > 1: idx [B, sets, Tq, K*max(1, block)])
 *   dy       bf16 [B, Tq, Hq, d]: gradient of out
 *   dq       fp32 [B, Tq, Hq, d] out
 *   dk, dv   fp32 [B, Tk, Hkv, d] out: 0 for positions no row selected; sums in
 *            32.32 fixed point, so they do not depend on the summation order
 *            (deterministic); each element's sum must stay below 2^31 in size
 *   dgate    fp32 [B, Tq, Hq, d] out, nullable (only with gate)
 *   dmix     fp32 [B, Tq, Hq, d] out, nullable (only with mix)
 *   workspace at least lci_workspace_bytes(LCI_ENTRY_SPARSE_ATTN_BWD): the
 *            recomputed forward output and lse, do, delta and the transpose of
 *            the index rows. B*sets*Tq*K*max(1, block) < 2^31 (SHAPE).
 * Errors: NULL, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN, HIP. */
lci_status lci_sparse_attn_bwd(const lci_geom *g, const lci_bf16 *q, const lci_bf16 *k,
                               const lci_bf16 *v, const int32_t *idx, const lci_bf16 *gate,
                               const lci_bf16 *mix, const lci_bf16 *dy, float softmax_scale,
                               float *dq, float *dk, float *dv, float *dgate, float *dmix,
                               void *workspace, size_t ws_bytes, void *stream);

/* Gradients of the scorer's distillation loss (the training of the indexer:
 * "How Fine-Grained Sparse Attention Reshapes ...", section "How Indexer + Top-K
 * Works at Runtime" -- the indexer's selection distribution is distilled from a
 * full-attention teacher; "Hybrid Sparse Attention ...", section "Engineering
 * and Evaluation Recommendations", training side). The pages give no loss; the
 * reading taken: for query row i with index row idx[i] (entries outside 0..p
 * skipped; each entry counts, a repeated position twice), the scorer's
 * distribution is p_t = softmax_t(tau * S_t) over the entries, with S the
 * indexer score of lci_idx_score, and the loss is
 *   L_i = sum_t T_t (log T_t - log p_t)      (0 log 0 = 0; KL when T sums to 1).
 * With q_idx, k_idx and w taken as real numbers (their int8 values) and the
 * ReLU's derivative 0 at 0, g_t = tau (p_t sum_u T_u - T_t) and
 *   dw[i,h] = sum_t g_t max(0, d_ht),  dq[i,h,:] = w_h sum_t g_t [d_ht > 0] k_idx[idx_t],
 *   dk[s,:] = sum over entries with idx_t = s of g_t sum_h w_h [d_ht > 0] q_idx[i,h],
 * d_ht = q_idx[i,h] . k_idx[idx_t]. With S = g->sets > 1 index sets (S divides
 * H_I, else SHAPE), set j is the scorer of indexer heads j*H_I/S ..
 * (j+1)*H_I/S - 1 (their weights included) over its own index rows and teacher:
 * each set has the loss above on its heads, dq and dw of a head come from its
 * set, and dk sums over the sets.
 *   q_idx, k_idx, w, strides: as in lci_idx_score
 *   idx      int32 [B, S, Tq, K*max(1, block)] (S = 1 without sets): the entries
 *            (the index rows of the forward, or any positions)
 *   teacher  fp32 [B, S, Tq, K*max(1, block)]: the teacher's weights, >= 0,
 *            aligned with idx (they need not sum to 1)
 *   tau      the score scale of the scorer's softmax (finite, else SHAPE)
 *   loss     fp32 [B, S, Tq] out, nullable
 *   dq_idx   fp32 [B, Tq, H_I, d_I] out;  dk_idx fp32 [B, Tk, d_I] out (0 where no
 *            entry points); dw fp32 [B, Tq, H_I] out (per row: for weights shared
 *            by every row, their gradient is the sum over rows)
 *   workspace at least lci_workspace_bytes(LCI_ENTRY_INDEXER_BWD): g and the
 *            heads' ReLU masks per entry, the entries of each position, and
 *            the query rows with each feature's heads side by side. dk
 *            sums its products as 64-bit integers with 32 fraction bits (the
 *            sum does not depend on the order: deterministic); each element's
 *            sum must stay below 2^31 in size. B*Tq*K < 2^31 (SHAPE). The sets
 *            run one after another and share the workspace (its size does
 *            not grow with S).
 * Invalid rows and rows without a valid entry give zeros. Floating-point work is
 * fp32 (the scores themselves are exact).
 * Errors: NULL, SHAPE, UNSUPPORTED, OVERFLOW_RISK, WORKSPACE, ALIGN, HIP. */
lci_status lci_indexer_bwd(const lci_geom *g, const int8_t *q_idx, const int8_t *k_idx,
                           const int8_t *w, int64_t w_stride_b, int64_t w_stride_q,
                           const int32_t *idx, const float *teacher, float tau, float *loss,
                           float *dq_idx, float *dk_idx, float *dw, void *workspace,
                           size_t ws_bytes, void *stream);

/* Workspace bytes an entry needs for this geometry (host only, reads no device
 * memory). Returns 0 for an invalid geometry or entry id. */
size_t lci_workspace_bytes(int entry, const lci_geom *g);

/* Query rows of an entry that take the dense-tile attention path (host only,
 * reads no device memory): a valid row at position p takes it when
 * p + 1 <= the returned limit, which is 0 when the entry runs no tile path for
 * this geometry (few rows: split-K; the one-row decode path). The two exact
 * formulations of the pages ("From Linear Attention to Gated Sparse
 * Attention", section 2: scores over all causal positions under a selection
 * mask; "Hybrid Sparse Attention ...", the Indexer + Top-K pseudocode: a
 * gather of the selected rows) give the same result up to fp32 summation
 * order; the limit only says which kernel does the work (for per-kernel
 * accounting). entry: LCI_ENTRY_PREFILL, LCI_ENTRY_SPARSE_ATTN or
 * LCI_ENTRY_DECODE; any other id, or an invalid geometry, gives 0. */
int lci_dense_row_limit(int entry, const lci_geom *g);

/* Static text for a status code. */
const char *lci_status_str(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int lci_last_hip_error(void);

/* LCI_ABI_VERSION of the loaded library. */
int lci_abi_version(void);

/* Kernel timing (instrumentation for profiling and roofline reports; not part
 * of the computation). While switched on, every kernel the library launches is
 * bracketed by two HIP events recorded on its launch stream, and the pairs are
 * kept in a process-wide log (the one piece of global mutable state besides the
 * per-thread last HIP error; it is guarded by a mutex). Off by default.
 *   lci_kernel_timing(1) clears the log and switches timing on; (0) switches it
 *     off and clears the log. Returns LCI_OK, or LCI_ERR_HIP.
 *   lci_kernel_timing_read(kernel, &total_ms, &launches) waits for the logged
 *     events of that kernel kind (host synchronisation on those events only)
 *     and returns the summed event-to-event time and the launch count since the
 *     log was cleared. Errors: NULL, SHAPE (unknown kernel id), HIP.
 *   lci_kernel_name(kernel) is the kernel kind's name, NULL for an unknown id.
 * Recording events costs a few microseconds per launch: use it for per-kernel
 * figures, not for the end-to-end latency of a call. */
enum {
  LCI_KERNEL_IDX_SCORE = 0,   /* indexer scores, prefill layout                     */
  LCI_KERNEL_TOPK = 1,        /* Top-K over materialised score rows                 */
  LCI_KERNEL_IDX_MASK = 2,    /* index rows -> position bit masks for dense tiles    */
  LCI_KERNEL_ATTN_DENSE = 3,  /* masked attention over contiguous key tiles          */
  LCI_KERNEL_ATTN_GATHER = 4, /* attention over gathered selected keys              */
  LCI_KERNEL_ATTN_COMBINE = 5,/* fixed-order merge of split-K partial results        */
  LCI_KERNEL_DEC_SAMPLE = 6,  /* decode: histogram of every 32nd position's score  */
  LCI_KERNEL_DEC_THRESH = 7,  /* decode: the candidate threshold from the histogram */
  LCI_KERNEL_DEC_SCORE = 8,   /* decode: every score; candidates at the threshold   */
  LCI_KERNEL_DEC_SELECT = 9,  /* decode: exact Top-K of the candidates (or the row) */
  LCI_KERNEL_KV_APPEND = 10,  /* new rows into the key/value/indexer-key caches     */
  LCI_KERNEL_KV_LENGTHS = 11, /* new cache lengths and first positions after append */
  LCI_KERNEL_BWD_PROLOGUE = 12, /* backward: output gradient through the gate, delta */
  LCI_KERNEL_BWD_DQ = 13,     /* backward: query gradients                           */
  LCI_KERNEL_BWD_TRANSPOSE = 14, /* backward: the rows that selected each position  */
  LCI_KERNEL_BWD_DKDV = 15,   /* backward: key and value gradients                   */
  LCI_KERNEL_SEL_SCAN = 16,   /* long prefill: scores, sampled threshold, candidates */
  LCI_KERNEL_SEL_ROWS = 17,   /* long prefill: exact Top-K of each row's candidates  */
  LCI_KERNEL_SEL_FALLBACK = 18, /* long prefill: rows whose candidates fell short    */
  LCI_KERNEL_IBWD = 19,       /* scorer's distillation loss: rows (loss, g, dq, dw)  */
  LCI_KERNEL_IBWD_TRANSPOSE = 20, /* scorer's gradients: the entries of each position */
  LCI_KERNEL_IBWD_DK = 21,    /* scorer's gradients: indexer-key gradients           */
  LCI_KERNEL_COUNT = 22
};
int lci_kernel_timing(int enable);
int lci_kernel_timing_read(int kernel, double *total_ms, int64_t *launches);
const char *lci_kernel_name(int kernel);

/* Concurrent attention paths (a schedule, not part of the computation: the
 * results are bit-identical either way). When the rows of a call split between
 * the tile path and the gather path ("Hybrid Sparse Attention ...", section
 * "Indexer + Top-K", step 3, run two exact ways; see lci_dense_row_limit), the
 * two kernels can run at once on two library-owned streams whose compute-unit
 * masks split every XCD (the gather gets k of each XCD's 32 CUs, the tile
 * kernel t of them, a few possibly shared): the gather is bound by the rate rows arrive from the
 * last-level cache and saturates on part of the chip, the tile kernel by its
 * MFMA and softmax work. The caller's stream forks to them and joins back
 * through events, so the call stays ordered on that stream. The library
 * creates a pair of streams (default priority) and three events per device and
 * split used (four splits at most) on first use and keeps them until the
 * process ends; under graph capture, or on a device without 256 CUs, calls run
 * on the caller's stream alone. Calls from several host threads on one device
 * share the streams (their work is serialised there; the fork and join are
 * guarded by a mutex).
 *   LCI_OVERLAP_AUTO  (default) only for a whole prompt (Tq == Tk) when a cost
 *                     model of the two kernels (measured on Prefill 64K) picks
 *                     a split that beats running them one after the other
 *   LCI_OVERLAP_OFF   never
 *   LCI_OVERLAP_ON    for every call with gather rows possible (gather on 20
 *                     CUs of each XCD, tile kernel on 16: 4 shared)
 * lci_attn_overlap(mode) sets the process-wide mode: LCI_OK, or SHAPE for an
 * unknown mode. lci_attn_overlap_forks() counts the calls so far (process-wide)
 * that ran the two kernels on the library streams. */
enum { LCI_OVERLAP_AUTO = 0, LCI_OVERLAP_OFF = 1, LCI_OVERLAP_ON = 2 };
int lci_attn_overlap(int mode);
long long lci_attn_overlap_forks(void);

#ifdef __cplusplus
}
#endif

#endif /* LCI_H */
