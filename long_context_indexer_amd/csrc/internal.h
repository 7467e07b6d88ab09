// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lci {

// Brackets one kernel launch with timing events on its stream while kernel
// timing is on (lci_kernel_timing); does nothing otherwise.
class KernelTimer {
 public:
  KernelTimer(int kind, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int kind_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

struct Geom {
  int B, Tq, Tk, Hq, Hkv, d, H_I, d_I, K;
  const int32_t* q_offset;
  const int32_t* kv_len;
  int block;  // selection granularity: 1 = single positions, else blocks of this many
  int sets;   // index sets per query row: 1, or Hkv (index rows [B][sets][Tq][K])
};

// ---- indexer scoring
hipError_t launch_idx_score(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                            const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                            int32_t* scores, int64_t score_row_stride, int row_begin,
                            int row_count, hipStream_t stream);

// ---- Top-K over materialised score rows.
// Both launchers work on query rows [row_begin, row_begin+row_count) of every
// sequence; the score row of (b, row_begin + r) is at scores + (b*row_count + r)*stride.
// idx/sel are always the full [B, Tq, K] arrays.
// Rows of histories up to kWaveTopkMax positions (Tk <= kWaveTopkMax) run one
// wave per row with the row in registers; longer ones one workgroup per row.
constexpr int kWaveTopkMax = 8192;

// Row flags of the dense-tile attention path.
enum : uint8_t {
  kRowGather = 0,  // left to the gather kernel
  kRowMasked = 1,  // tile kernel, keys given by the row's bit mask
  kRowAll = 2,     // tile kernel, the row keeps every position 0..p
  kRowEmpty = 3,   // tile kernel writes the empty-row result (no valid position)
};

// Inputs of the dense-tile attention kernel, inside the sparse-attention
// workspace: per-row bit masks over positions (Wm words a row, written for
// every row on the tile path: the selected positions, all of 0..p for kRowAll
// rows, none for kRowEmpty rows), row flags (kRow*) and per-token-block "done
// by the tile kernel" bytes. Rows qualify when p + 1 <= lim.
struct DenseMasks {
  uint32_t* mask;
  uint8_t* flag;
  uint8_t* done;
  int Wm, lim;
};
DenseMasks dense_masks(const Geom& g, void* workspace);

// With dm (only when Tk <= kWaveTopkMax), the Top-K kernel also writes the
// dense-path flags and masks of its rows.
hipError_t launch_topk_rows(const Geom& g, const int32_t* scores, int64_t score_row_stride,
                            int row_begin, int row_count, int32_t* idx, int32_t* sel,
                            const DenseMasks* dm, hipStream_t stream);

// ---- sparse attention over index rows
size_t sparse_attn_workspace(const Geom& g, int splits);
int sparse_attn_pick_splits(const Geom& g);
// masks_ready: the dense-path masks and flags in the workspace were written by
// the Top-K kernel (valid index rows by construction), so the index rows are
// not scanned again.
hipError_t launch_sparse_attn(const Geom& g, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                              const uint16_t* mix,
                              float scale, uint16_t* out, float* lse, int splits,
                              void* workspace, bool masks_ready, hipStream_t stream);

// ---- block-granular Top-K: K blocks of g.block positions (a power of two,
// at least 2) per row, the row's blocks in LDS. idx rows hold K*block positions,
// sel (nullable) the K kept blocks' scores. With dm (masks of the attention
// geometry, K*block positions a row) it also writes the dense-path flags and
// masks of its rows.
constexpr int kBlockTopkMaxBlocks = 8192;  // ceil(Tk / block) at most
constexpr int kBlockTopkMaxKeep = 2048;    // K at most (K*block <= 4096, block >= 2)
hipError_t launch_block_topk(const Geom& g, const int32_t* scores, int64_t score_row_stride,
                             int row_begin, int row_count, int32_t* idx, int32_t* sel,
                             const DenseMasks* dm, hipStream_t stream);

// ---- index sets per key/value head: q_idx [B,Tq,H_I,d_I] regrouped into
// [sets][B][Tq][H_I/sets][d_I], so each set's indexer heads form a contiguous
// query array for the scoring kernels
hipError_t launch_regroup_q_idx(const Geom& g, const int8_t* q_idx, int8_t* out,
                                hipStream_t stream);

// ---- gradients of sparse attention + gate (g.K = index row length, one set)
struct BwdLayout {
  size_t fwd, o, lse, dO, delta, cnt, off, cursor, tiles, rows, part, total;
  int splits, ntiles;
  int nch;  // row chunks of the key-major tile kernel (partials summed in order)
};
BwdLayout bwd_layout(const Geom& g);
hipError_t launch_sparse_attn_bwd(const Geom& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                                  const uint16_t* mix, const uint16_t* dy, float scale, float* dq,
                                  float* dk, float* dv, float* dgate, float* dmix,
                                  void* workspace, hipStream_t stream);

// ---- appending rows to the key / value / indexer-key caches
// Sizes from g: B, Tq (= rows of the new tensors per sequence), Tk (capacity),
// Hkv, d, d_I; g.kv_len holds the current lengths.
hipError_t launch_kv_append(const Geom& g, const uint16_t* k_new, const uint16_t* v_new,
                            const int8_t* kI_new, const int32_t* n_new, uint16_t* k_cache,
                            uint16_t* v_cache, int8_t* kI_cache, int32_t* q_offset_out,
                            int32_t* kv_len_out, hipStream_t stream);

}  // namespace lci
