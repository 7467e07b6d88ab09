// Deterministic Top-K over materialised indexer score rows (gfx950).
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer + Top-K: How
// Fine-Grained Sparse Attention Works", step 2 (keep the K best positions per
// query); "Optimizing LLM Long-Context Inference with Indexed Top-K Sparse
// Attention", section "Interface Design" (topk over the last axis of the score
// row). Order: higher score first, lower position on equal scores. Output: the
// selected positions in ascending order, -1 padded when the row has fewer than
// K candidates (positions 0..p).
//
// One workgroup per query row:
//   1. min/max of the order-preserving uint32 keys fixes the varying low bits;
//   2. radix select, up to 11 bits per pass, with an LDS histogram (integer
//      atomics: order-independent, so the result is deterministic) finds the
//      exact K-th key v* and r = how many keys equal to v* are kept;
//   3. an ordered compaction in position order keeps every key > v* and the
//      first r keys == v*: one block-wide prefix scan per chunk of the packed
//      (count greater, count equal) pair gives each thread its output slot.
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"
#include "select_row.h"

namespace lci {

__global__ __launch_bounds__(TOPK_NT) void topk_rows_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ scores, int64_t stride,
    int row_begin, int row_count, int32_t* __restrict__ idx, int32_t* __restrict__ sel) {
  __shared__ SelectLds sm;
  const int rr = blockIdx.x;
  const int b = blockIdx.y;
  const int row = row_begin + rr;
  const int64_t orow = (static_cast<int64_t>(b) * Tq + row) * K;
  int32_t* out = idx + orow;
  int32_t* outs = sel ? sel + orow : nullptr;
  const int kvl = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + row;
  const bool valid = kvl <= Tk && p >= 0 && p < kvl;
  const int64_t n = valid ? p + 1 : 0;
  const int32_t* S = scores + (static_cast<int64_t>(b) * row_count + rr) * stride;

  if (n <= K) {  // every candidate is kept (dense-equivalent row) or the row is invalid
    for (int j = threadIdx.x; j < K; j += TOPK_NT) {
      out[j] = j < n ? j : -1;
      if (outs) outs[j] = j < n ? S[j] : INT32_MIN;
    }
    return;
  }
  select_row(S, n, K, out, outs, sm);
}

hipError_t launch_topk_rows(const Geom& g, const int32_t* scores, int64_t stride,
                            int row_begin, int row_count, int32_t* idx, int32_t* sel,
                            hipStream_t st) {
  dim3 grid(row_count, g.B);
  {
    KernelTimer timer(LCI_KERNEL_TOPK, st);
    hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TOPK_NT), 0, st, g.Tq, g.Tk, g.K,
                       g.q_offset, g.kv_len, scores, stride, row_begin, row_count, idx, sel);
  }
  return hipGetLastError();
}

}  // namespace lci
