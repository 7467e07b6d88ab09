// C ABI of the library: argument validation on the host, workspace carving and
// kernel dispatch on the caller's stream. See include/lci.h for the contract.
#include "../../include/lci.h"

#include <algorithm>

#include "decode.h"
#include "internal.h"

using lci::Geom;

namespace {

thread_local int g_last_hip_error = 0;

lci_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LCI_OK;
  g_last_hip_error = static_cast<int>(e);
  return LCI_ERR_HIP;
}

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int kMaxK = 4096;

// Positions per selected unit: 1, or the block size of block-granular selection.
int sel_block(const lci_geom* g) { return g->block > 1 ? g->block : 1; }

// Index sets per query row: 1 (shared by every head), or g->sets.
int sel_sets(const lci_geom* g) { return g->sets > 1 ? g->sets : 1; }

// Index sets: query head h reads set h / (Hq/sets), so with attention the sets
// divide Hq; with scoring the indexer heads split evenly into them.
lci_status check_sets(const lci_geom* g, bool indexer, bool attention) {
  if (g->sets < 0) return LCI_ERR_SHAPE;
  const int ns = sel_sets(g);
  if (ns == 1) return LCI_OK;
  if (attention && g->Hq % ns != 0) return LCI_ERR_SHAPE;
  if (indexer && g->H_I % ns != 0) return LCI_ERR_SHAPE;
  return LCI_OK;
}

// Sizes common to every entry.
lci_status check_base(const lci_geom* g) {
  if (!g) return LCI_ERR_NULL;
  if (!g->q_offset || !g->kv_len) return LCI_ERR_NULL;
  if (g->B < 1 || g->Tq < 1 || g->Tk < 1 || g->K < 1 || g->K > kMaxK) return LCI_ERR_SHAPE;
  if (g->block < 0) return LCI_ERR_SHAPE;
  const int bl = sel_block(g);
  if (bl > 1 && (bl > 256 || (bl & (bl - 1)) != 0)) return LCI_ERR_UNSUPPORTED;
  // index rows hold K*block positions
  if (static_cast<int64_t>(g->K) * bl > kMaxK) return LCI_ERR_SHAPE;
  // a row's blocks live in LDS
  if (bl > 1 && (static_cast<int64_t>(g->Tk) + bl - 1) / bl > lci::kBlockTopkMaxBlocks)
    return LCI_ERR_UNSUPPORTED;
  if (!aligned4(g->q_offset) || !aligned4(g->kv_len)) return LCI_ERR_ALIGN;
  return LCI_OK;
}

lci_status check_indexer(const lci_geom* g) {
  if (g->H_I < 1 || g->d_I < 1) return LCI_ERR_SHAPE;
  if (static_cast<int64_t>(g->H_I) * g->d_I > 1024) return LCI_ERR_OVERFLOW_RISK;
  if (!pow2_in(g->H_I, 1, 16) || !(g->d_I == 32 || g->d_I == 64 || g->d_I == 128))
    return LCI_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(g->Tk) * g->d_I >= (int64_t(1) << 31)) return LCI_ERR_SHAPE;
  return LCI_OK;
}

lci_status check_attention(const lci_geom* g) {
  if (g->Hq < 1 || g->Hkv < 1 || g->d < 1 || g->Hq % g->Hkv != 0) return LCI_ERR_SHAPE;
  if (!(g->d == 64 || g->d == 128) || !pow2_in(g->Hkv, 1, 8) || !pow2_in(g->Hq / g->Hkv, 1, 16))
    return LCI_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(g->Tk) * g->Hkv * g->d >= (int64_t(1) << 31)) return LCI_ERR_SHAPE;
  return LCI_OK;
}

// The kernels track running maxima of the raw dot products, which are the
// maxima of scale*q.k only for a positive scale.
bool scale_ok(float scale) { return scale > 0.f && scale < INFINITY; }

Geom to_geom(const lci_geom* g) {
  return Geom{g->B, g->Tq, g->Tk, g->Hq, g->Hkv, g->d, g->H_I, g->d_I, g->K, g->q_offset,
              g->kv_len, sel_block(g), sel_sets(g)};
}

// The attention kernels' view: index rows of K*block positions.
Geom attn_geom(const lci_geom* g) {
  Geom a = to_geom(g);
  a.K = g->K * a.block;
  return a;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Fused prefill: query rows are scored and selected in chunks whose int32 score
// block stays within kScoreBudget. Each chunk costs a scoring and a selection
// launch, whose ramp and tail dominate when chunks are small: on Prefill 64K,
// 4096-row chunks (1 GiB) beat 1024-row ones (256 MiB) by 14% (scoring) and
// 18% (selection); 256-row chunks that would stay in the 256 MiB last-level
// cache were slower still. At 8K the whole sequence is one chunk.
constexpr size_t kScoreBudget = size_t(1024) << 20;

int prefill_chunk_rows(const lci_geom* g) {
  const size_t per_row = static_cast<size_t>(g->B) * g->Tk * sizeof(int32_t);
  size_t rows = std::max<size_t>(1, kScoreBudget / per_row);
  if (rows >= 64) rows = rows / 64 * 64;
  return static_cast<int>(std::min<size_t>(rows, static_cast<size_t>(g->Tq)));
}

struct PrefillLayout {
  size_t idx_off, idx_bytes, score_off, score_bytes, attn_off, attn_bytes, qg_off, qg_bytes,
      sel_off, sel_bytes, total;
  int chunk_rows, splits;
  bool sel;  // scores and Top-K by the long-prefill kernels (no score block)
};

// The geometry of one index set's scoring and selection: H_I/sets indexer heads.
Geom set_geom(const lci_geom* g) {
  Geom gs = to_geom(g);
  gs.H_I = g->H_I / gs.sets;
  return gs;
}

PrefillLayout prefill_layout(const lci_geom* g, int64_t wsb = 0, int64_t wsq = 0) {
  PrefillLayout L{};
  const Geom gg = attn_geom(g);
  const Geom gs = set_geom(g);
  L.sel = lci::sel_supported(gs, wsb, wsq);
  L.chunk_rows = prefill_chunk_rows(g);
  L.splits = lci::sparse_attn_pick_splits(gg);
  L.idx_off = 0;
  L.idx_bytes =
      align_up(static_cast<size_t>(g->B) * sel_sets(g) * g->Tq * gg.K * sizeof(int32_t));
  L.score_off = L.idx_off + L.idx_bytes;
  L.score_bytes =
      L.sel ? 0
            : align_up(static_cast<size_t>(g->B) * L.chunk_rows * g->Tk * sizeof(int32_t));
  L.attn_off = L.score_off + L.score_bytes;
  L.attn_bytes = align_up(lci::sparse_attn_workspace(gg, L.splits));
  // the query rows regrouped by index set (for the long-prefill kernels; the
  // scoring kernel reads a set's heads in place)
  L.qg_off = L.attn_off + L.attn_bytes;
  L.qg_bytes = L.sel && sel_sets(g) > 1
                   ? align_up(static_cast<size_t>(g->B) * g->Tq * g->H_I * g->d_I)
                   : 0;
  L.sel_off = L.qg_off + L.qg_bytes;
  L.sel_bytes = L.sel ? align_up(lci::sel_layout(gs).total) : 0;
  L.total = L.sel_off + L.sel_bytes;
  return L;
}

}  // namespace

namespace lci {
int hip_error_status(hipError_t e) { return hip_status(e); }
}  // namespace lci

extern "C" {

int lci_abi_version(void) { return LCI_ABI_VERSION; }

int lci_last_hip_error(void) { return g_last_hip_error; }

const char* lci_status_str(int s) {
  switch (s) {
    case LCI_OK: return "LCI_OK";
    case LCI_ERR_NULL: return "LCI_ERR_NULL: a required pointer is NULL";
    case LCI_ERR_SHAPE: return "LCI_ERR_SHAPE: a size is out of range or inconsistent";
    case LCI_ERR_UNSUPPORTED: return "LCI_ERR_UNSUPPORTED: no kernel for this shape";
    case LCI_ERR_OVERFLOW_RISK: return "LCI_ERR_OVERFLOW_RISK: H_I*d_I > 1024 could overflow int32 scores";
    case LCI_ERR_WORKSPACE: return "LCI_ERR_WORKSPACE: workspace missing or too small";
    case LCI_ERR_HIP: return "LCI_ERR_HIP: a HIP call failed";
    case LCI_ERR_ALIGN: return "LCI_ERR_ALIGN: a pointer is not 16-byte aligned";
    case LCI_ERR_SCRATCH:
      return "LCI_ERR_SCRATCH: the call needs more workspace than the allocation-free entry's "
             "static scratch array holds";
    default: return "unknown lci status";
  }
}

size_t lci_workspace_bytes(int entry, const lci_geom* g) {
  if (check_base(g) != LCI_OK) return 0;
  switch (entry) {
    case LCI_ENTRY_IDX_SCORE:
    case LCI_ENTRY_TOPK_SELECT:
      return 0;
    case LCI_ENTRY_SPARSE_ATTN: {
      if (check_attention(g) != LCI_OK || check_sets(g, false, true) != LCI_OK) return 0;
      const Geom gg = attn_geom(g);
      return lci::sparse_attn_workspace(gg, lci::sparse_attn_pick_splits(gg));
    }
    case LCI_ENTRY_PREFILL:
      if (check_attention(g) != LCI_OK || check_indexer(g) != LCI_OK ||
          check_sets(g, true, true) != LCI_OK)
        return 0;
      // the weights' strides are not known here: enough for either scoring path
      return std::max(prefill_layout(g, 0, 0).total, prefill_layout(g, 1, 1).total);
    case LCI_ENTRY_SPARSE_ATTN_BWD: {
      if (check_attention(g) != LCI_OK || check_sets(g, false, true) != LCI_OK) return 0;
      return lci::bwd_layout(attn_geom(g)).total;
    }
    case LCI_ENTRY_INDEXER_BWD:
      if (check_indexer(g) != LCI_OK || check_sets(g, true, false) != LCI_OK) return 0;
      return lci::ibwd_workspace(attn_geom(g));  // index rows of K*block positions
    case LCI_ENTRY_DECODE:
      if (check_attention(g) != LCI_OK || check_indexer(g) != LCI_OK || g->Tq != 1 ||
          check_sets(g, true, true) != LCI_OK)
        return 0;
      // block-granular or per-head-set decode runs the prefill path on its one row
      if (sel_block(g) > 1 || sel_sets(g) > 1)
        return std::max(prefill_layout(g, 0, 0).total, prefill_layout(g, 1, 1).total);
      return lci::decode_layout(to_geom(g)).total;
    default:
      return 0;
  }
}

int lci_dense_row_limit(int entry, const lci_geom* g) {
  if (check_base(g) != LCI_OK || check_attention(g) != LCI_OK) return 0;
  if (entry != LCI_ENTRY_PREFILL && entry != LCI_ENTRY_SPARSE_ATTN &&
      entry != LCI_ENTRY_DECODE)
    return 0;
  // the one-row decode path never takes the tile kernel
  if (entry == LCI_ENTRY_DECODE && sel_block(g) == 1 && sel_sets(g) == 1) return 0;
  const Geom ga = attn_geom(g);
  if (lci::sparse_attn_pick_splits(ga) != 1) return 0;
  return lci::dense_row_limit(ga);
}

lci_status lci_idx_score(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                         const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                         int32_t* scores, void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_indexer(g)) != LCI_OK) return s;
  if ((s = check_sets(g, true, false)) != LCI_OK) return s;
  if (!q_idx || !k_idx || !w || !scores) return LCI_ERR_NULL;
  if (w_stride_b < 0 || w_stride_q < 0) return LCI_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned4(scores)) return LCI_ERR_ALIGN;
  // set g: indexer heads g*Hg .. g*Hg + Hg - 1 read in place from the query
  // rows, their weights, score rows [B][sets][Tq][Tk]
  const Geom gs = set_geom(g);
  const int ns = gs.sets;
  for (int set = 0; set < ns; ++set) {
    hipError_t e = lci::launch_idx_score(
        gs, q_idx + static_cast<size_t>(set) * gs.H_I * g->d_I, g->H_I, k_idx,
        w + set * gs.H_I, w_stride_b, w_stride_q, scores + static_cast<size_t>(set) * g->Tq * g->Tk,
        g->Tk, static_cast<int64_t>(ns) * g->Tq, 0, g->Tq, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e);
  }
  return LCI_OK;
}

lci_status lci_topk_select(const lci_geom* g, const int32_t* scores, int32_t* idx,
                           int32_t* sel_scores, void* workspace, size_t ws_bytes,
                           void* stream) {
  (void)workspace;
  (void)ws_bytes;
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_sets(g, false, false)) != LCI_OK) return s;
  if (!scores || !idx) return LCI_ERR_NULL;
  if (!aligned4(scores) || !aligned4(idx) || (sel_scores && !aligned4(sel_scores)))
    return LCI_ERR_ALIGN;
  // rows [B][sets][Tq]: the kernels address index rows as b*Tq' + row with
  // Tq' = sets*Tq, and set g's rows start g*Tq rows in
  const int ns = sel_sets(g);
  Geom gsel = to_geom(g);
  gsel.Tq = g->Tq * ns;
  const int KI = g->K * gsel.block;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int set = 0; set < ns; ++set) {
    const size_t r0 = static_cast<size_t>(set) * g->Tq;
    const int32_t* sc = scores + r0 * g->Tk;
    int32_t* is = idx + r0 * KI;
    int32_t* ss = sel_scores ? sel_scores + r0 * g->K : nullptr;
    const int64_t brows = static_cast<int64_t>(ns) * g->Tq;
    hipError_t e = gsel.block > 1
                       ? lci::launch_block_topk(gsel, sc, g->Tk, brows, 0, g->Tq, is, ss, nullptr, st)
                       : lci::launch_topk_rows(gsel, sc, g->Tk, brows, 0, g->Tq, is, ss, nullptr, st);
    if (e != hipSuccess) return hip_status(e);
  }
  return LCI_OK;
}

lci_status lci_sparse_attn_fwd(const lci_geom* g, const lci_bf16* q, const lci_bf16* k,
                               const lci_bf16* v, const int32_t* idx, const lci_bf16* gate,
                               const lci_bf16* mix, float softmax_scale, lci_bf16* out,
                               float* lse, void* workspace, size_t ws_bytes, void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_attention(g)) != LCI_OK) return s;
  if ((s = check_sets(g, false, true)) != LCI_OK) return s;
  if (!q || !k || !v || !idx || !out || (mix && !gate)) return LCI_ERR_NULL;
  if (!scale_ok(softmax_scale)) return LCI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (gate && !aligned16(gate)) || (mix && !aligned16(mix)) || !aligned4(idx) ||
      (lse && !aligned4(lse)))
    return LCI_ERR_ALIGN;
  const Geom gg = attn_geom(g);
  const int splits = lci::sparse_attn_pick_splits(gg);
  const size_t need = lci::sparse_attn_workspace(gg, splits);
  if (need > 0 && (!workspace || ws_bytes < need)) return LCI_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return LCI_ERR_ALIGN;
  return hip_status(lci::launch_sparse_attn(gg, q, k, v, idx, gate, mix, softmax_scale, out,
                                            lse, splits, workspace, false,
                                            static_cast<hipStream_t>(stream)));
}

static lci_status fused_forward(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                                const int8_t* w, int64_t wsb, int64_t wsq, const lci_bf16* q,
                                const lci_bf16* k, const lci_bf16* v, const lci_bf16* gate,
                                const lci_bf16* mix, float scale, lci_bf16* out, float* lse,
                                int32_t* idx_out, void* workspace, size_t ws_bytes,
                                void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_indexer(g)) != LCI_OK) return s;
  if ((s = check_attention(g)) != LCI_OK) return s;
  if ((s = check_sets(g, true, true)) != LCI_OK) return s;
  if (!q_idx || !k_idx || !w || !q || !k || !v || !out || (mix && !gate)) return LCI_ERR_NULL;
  if (wsb < 0 || wsq < 0 || !scale_ok(scale)) return LCI_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || !aligned16(out) || (gate && !aligned16(gate)) ||
      (mix && !aligned16(mix)) || (lse && !aligned4(lse)) || (idx_out && !aligned4(idx_out)))
    return LCI_ERR_ALIGN;
  const PrefillLayout L = prefill_layout(g, wsb, wsq);
  if (!workspace || ws_bytes < L.total) return LCI_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LCI_ERR_ALIGN;
  const Geom gg = to_geom(g);
  const Geom ga = attn_geom(g);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx_off);
  int32_t* sc = reinterpret_cast<int32_t*>(ws + L.score_off);
  // with the dense-tile path on (one split), the selection kernel writes the
  // tile path's masks and flags: the block kernel always, the position kernel
  // for rows short enough for its one-wave form, the long-prefill selection
  // always
  const bool masks = L.splits == 1 && (gg.block > 1 || g->Tk <= lci::kWaveTopkMax || L.sel);
  const lci::DenseMasks dm = masks ? lci::dense_masks(ga, ws + L.attn_off) : lci::DenseMasks{};
  // index sets: set g is scored as an indexer of H_I/sets heads (heads
  // g*Hg .. g*Hg + Hg - 1 of the query rows, their weights) and its index rows
  // go to [B][sets][Tq][K*block] (the selection kernels address rows as
  // b*Tq' + row, so Tq' = sets*Tq and an offset of g*Tq rows place them)
  const Geom gs = set_geom(g);
  Geom gsel = gg;
  gsel.Tq = g->Tq * gg.sets;
  if (L.sel) {
    // long prefill: scores never leave the chip; its kernels take each set's
    // query heads as a contiguous array
    const int8_t* qsrc = q_idx;
    if (gg.sets > 1) {
      int8_t* qg = reinterpret_cast<int8_t*>(ws + L.qg_off);
      hipError_t e = lci::launch_regroup_q_idx(gg, q_idx, qg, st);
      if (e != hipSuccess) return hip_status(e);
      qsrc = qg;
    }
    const size_t qset = static_cast<size_t>(g->B) * g->Tq * gs.H_I * g->d_I;
    for (int set = 0; set < gg.sets; ++set) {
      int32_t* iset = idx + static_cast<size_t>(set) * g->Tq * ga.K;
      // this set's masks and flags: rows [B][sets][Tq] like the index rows
      lci::DenseMasks dms = dm;
      if (masks) {
        dms.mask += static_cast<size_t>(set) * g->Tq * dm.Wm;
        dms.flag += static_cast<size_t>(set) * g->Tq;
      }
      hipError_t e = lci::launch_sel(gs, qsrc + set * qset, k_idx, w + set * gs.H_I, iset,
                                     g->Tq * gg.sets, ws + L.sel_off, masks ? &dms : nullptr, st);
      if (e != hipSuccess) return hip_status(e);
    }
  }
  for (int r0 = 0; !L.sel && r0 < g->Tq; r0 += L.chunk_rows) {
    const int rc = std::min(L.chunk_rows, g->Tq - r0);
    for (int set = 0; set < gg.sets; ++set) {
      hipError_t e = lci::launch_idx_score(
          gs, q_idx + static_cast<size_t>(set) * gs.H_I * g->d_I, g->H_I, k_idx,
          w + set * gs.H_I, wsb, wsq, sc, g->Tk, rc, r0, rc, st);
      if (e != hipSuccess) return hip_status(e);
      int32_t* iset = idx + static_cast<size_t>(set) * g->Tq * ga.K;
      // this set's masks and flags: rows [B][sets][Tq] like the index rows
      lci::DenseMasks dms = dm;
      if (masks) {
        dms.mask += static_cast<size_t>(set) * g->Tq * dm.Wm;
        dms.flag += static_cast<size_t>(set) * g->Tq;
      }
      e = gg.block > 1
              ? lci::launch_block_topk(gsel, sc, g->Tk, rc, r0, rc, iset, nullptr,
                                       masks ? &dms : nullptr, st)
              : lci::launch_topk_rows(gsel, sc, g->Tk, rc, r0, rc, iset, nullptr,
                                      masks ? &dms : nullptr, st);
      if (e != hipSuccess) return hip_status(e);
    }
  }
  return hip_status(lci::launch_sparse_attn(ga, q, k, v, idx, gate, mix, scale, out, lse,
                                            L.splits, ws + L.attn_off, masks, st));
}

lci_status lci_prefill_fwd(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                           const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                           const lci_bf16* q, const lci_bf16* k, const lci_bf16* v,
                           const lci_bf16* gate, const lci_bf16* mix, float softmax_scale,
                           lci_bf16* out, float* lse, int32_t* idx_out, void* workspace,
                           size_t ws_bytes, void* stream) {
  return fused_forward(g, q_idx, k_idx, w, w_stride_b, w_stride_q, q, k, v, gate, mix,
                       softmax_scale, out, lse, idx_out, workspace, ws_bytes, stream);
}

lci_status lci_decode_fwd(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                          const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                          const lci_bf16* q, const lci_bf16* k, const lci_bf16* v,
                          const lci_bf16* gate, const lci_bf16* mix, float softmax_scale,
                          lci_bf16* out, float* lse, int32_t* idx_out, void* workspace,
                          size_t ws_bytes, void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if (g->Tq != 1) return LCI_ERR_SHAPE;
  // block-granular selection or several index sets: the prefill path
  // on the one row (block selection works on at most kBlockTopkMaxBlocks
  // blocks, which bounds the history)
  if (sel_block(g) > 1 || sel_sets(g) > 1)
    return fused_forward(g, q_idx, k_idx, w, w_stride_b, w_stride_q, q, k, v, gate, mix,
                         softmax_scale, out, lse, idx_out, workspace, ws_bytes, stream);
  if ((s = check_indexer(g)) != LCI_OK) return s;
  if ((s = check_attention(g)) != LCI_OK) return s;
  if (static_cast<int64_t>(g->Tk) > static_cast<int64_t>(lci::kDecChunk) * lci::kDecMaxChunks)
    return LCI_ERR_SHAPE;
  if (!q_idx || !k_idx || !w || !q || !k || !v || !out || (mix && !gate)) return LCI_ERR_NULL;
  if (w_stride_b < 0 || w_stride_q < 0) return LCI_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || !aligned16(out) || (gate && !aligned16(gate)) ||
      (mix && !aligned16(mix)) || (lse && !aligned4(lse)) || (idx_out && !aligned4(idx_out)))
    return LCI_ERR_ALIGN;
  const Geom gg = to_geom(g);
  const lci::DecLayout L = lci::decode_layout(gg);
  if (!workspace || ws_bytes < L.total) return LCI_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LCI_ERR_ALIGN;
  return hip_status(lci::launch_decode(gg, q_idx, k_idx, w, w_stride_b, q, k, v, gate, mix,
                                       softmax_scale, out, lse, idx_out, workspace,
                                       static_cast<hipStream_t>(stream)));
}

lci_status lci_sparse_attn_bwd(const lci_geom* g, const lci_bf16* q, const lci_bf16* k,
                               const lci_bf16* v, const int32_t* idx, const lci_bf16* gate,
                               const lci_bf16* mix, const lci_bf16* dy, float softmax_scale,
                               float* dq, float* dk, float* dv, float* dgate, float* dmix,
                               void* workspace, size_t ws_bytes, void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_attention(g)) != LCI_OK) return s;
  if ((s = check_sets(g, false, true)) != LCI_OK) return s;
  if (!q || !k || !v || !idx || !dy || !dq || !dk || !dv || (mix && !gate) ||
      (dgate && !gate) || (dmix && !mix))
    return LCI_ERR_NULL;
  if (!scale_ok(softmax_scale)) return LCI_ERR_SHAPE;
  const Geom ga = attn_geom(g);
  // the transpose of the index rows addresses entries with int32 offsets
  if (static_cast<int64_t>(g->B) * ga.sets * g->Tq * ga.K >= (int64_t(1) << 31) ||
      static_cast<int64_t>(g->B) * ga.sets * g->Tk >= (int64_t(1) << 31))
    return LCI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dy) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (gate && !aligned16(gate)) ||
      (mix && !aligned16(mix)) || (dgate && !aligned16(dgate)) || (dmix && !aligned16(dmix)) ||
      !aligned4(idx))
    return LCI_ERR_ALIGN;
  const lci::BwdLayout L = lci::bwd_layout(ga);
  if (!workspace || ws_bytes < L.total) return LCI_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LCI_ERR_ALIGN;
  return hip_status(lci::launch_sparse_attn_bwd(ga, q, k, v, idx, gate, mix, dy, softmax_scale,
                                                dq, dk, dv, dgate, dmix, workspace,
                                                static_cast<hipStream_t>(stream)));
}

lci_status lci_indexer_bwd(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                           const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                           const int32_t* idx, const float* teacher, float tau, float* loss,
                           float* dq_idx, float* dk_idx, float* dw, void* workspace,
                           size_t ws_bytes, void* stream) {
  lci_status s = check_base(g);
  if (s != LCI_OK) return s;
  if ((s = check_indexer(g)) != LCI_OK) return s;
  if ((s = check_sets(g, true, false)) != LCI_OK) return s;
  if (!q_idx || !k_idx || !w || !idx || !teacher || !dq_idx || !dk_idx || !dw)
    return LCI_ERR_NULL;
  if (w_stride_b < 0 || w_stride_q < 0 || !(tau == tau) || tau == INFINITY || tau == -INFINITY)
    return LCI_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(dq_idx) || !aligned4(idx) ||
      !aligned4(teacher) || !aligned4(dk_idx) || !aligned4(dw) || (loss && !aligned4(loss)))
    return LCI_ERR_ALIGN;
  Geom gg = to_geom(g);
  gg.K = g->K * gg.block;  // index rows of K*block positions
  // entries are numbered with int32
  if (static_cast<int64_t>(g->B) * g->Tq * gg.K >= (int64_t(1) << 31) ||
      static_cast<int64_t>(g->B) * g->Tk >= (int64_t(1) << 31))
    return LCI_ERR_SHAPE;
  const size_t need = lci::ibwd_workspace(gg);
  if (!workspace || ws_bytes < need) return LCI_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LCI_ERR_ALIGN;
  return hip_status(lci::launch_indexer_bwd(gg, q_idx, k_idx, w, w_stride_b, w_stride_q, idx,
                                            teacher, tau, loss, dq_idx, dk_idx, dw, workspace,
                                            static_cast<hipStream_t>(stream)));
}

lci_status lci_kv_append(const lci_geom* g, const lci_bf16* k_new, const lci_bf16* v_new,
                         const int8_t* kI_new, const int32_t* n_new, lci_bf16* k_cache,
                         lci_bf16* v_cache, int8_t* kI_cache, int32_t* q_offset_out,
                         int32_t* kv_len_out, void* stream) {
  if (!g || !g->kv_len) return LCI_ERR_NULL;
  if (!k_new || !v_new || !kI_new || !k_cache || !v_cache || !kI_cache) return LCI_ERR_NULL;
  // one workgroup row per sequence: B within the grid's y limit
  if (g->B < 1 || g->B > 65535 || g->Tq < 1 || g->Tk < 1 || g->Hkv < 1 || g->d < 1 ||
      g->d_I < 1)
    return LCI_ERR_SHAPE;
  if (q_offset_out && q_offset_out == kv_len_out) return LCI_ERR_SHAPE;
  if ((static_cast<int64_t>(g->Hkv) * g->d) % 8 != 0 || g->d_I % 16 != 0)
    return LCI_ERR_UNSUPPORTED;
  // int32 unit counts inside one workgroup, int64 row offsets
  if (static_cast<int64_t>(g->Hkv) * g->d > (int64_t(1) << 20) || g->d_I > (1 << 20))
    return LCI_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kI_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(kI_cache) || !aligned4(g->kv_len) ||
      (n_new && !aligned4(n_new)) || (q_offset_out && !aligned4(q_offset_out)) ||
      (kv_len_out && !aligned4(kv_len_out)))
    return LCI_ERR_ALIGN;
  return hip_status(lci::launch_kv_append(to_geom(g), k_new, v_new, kI_new, n_new, k_cache,
                                          v_cache, kI_cache, q_offset_out, kv_len_out,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
