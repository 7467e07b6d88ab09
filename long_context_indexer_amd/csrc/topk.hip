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
#include "internal.h"

namespace lci {

constexpr int TOPK_NT = 512;         // threads per row
constexpr int TOPK_BINS = 2048;      // 11-bit digits
constexpr int TOPK_E = 4;            // elements per thread per compaction chunk

__device__ __forceinline__ uint32_t low_mask(int bits) {
  return bits >= 32 ? 0xffffffffu : ((1u << bits) - 1u);
}

template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, 64)));
  }
  if (lane == 0) {
    red[2 * wid] = lo;
    red[2 * wid + 1] = hi;
  }
  __syncthreads();
  lo = red[0];
  hi = red[1];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    lo = min(lo, red[2 * w]);
    hi = max(hi, red[2 * w + 1]);
  }
  __syncthreads();
}

__global__ __launch_bounds__(TOPK_NT) void topk_rows_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ scores, int64_t stride,
    int row_begin, int row_count, int32_t* __restrict__ idx, int32_t* __restrict__ sel) {
  constexpr int NT = TOPK_NT;
  __shared__ uint32_t hist[TOPK_BINS];
  __shared__ uint32_t scratch[NT / 64 + 2];
  __shared__ uint32_t red[2 * (NT / 64)];
  __shared__ uint32_t found[2];

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
    for (int j = threadIdx.x; j < K; j += NT) {
      out[j] = j < n ? j : -1;
      if (outs) outs[j] = j < n ? S[j] : INT32_MIN;
    }
    return;
  }

  // 1. range of keys
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int64_t s = threadIdx.x; s < n; s += NT) {
    const uint32_t u = score_key(S[s]);
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_minmax<NT>(lo, hi, red);

  // 2. radix select of the K-th largest key
  uint32_t vstar, r;
  if (lo == hi) {
    vstar = lo;
    r = K;
  } else {
    const int top = 32 - __clz(lo ^ hi);  // bits [top-1:0] vary
    uint32_t mask = ~low_mask(top);
    uint32_t prefix = lo & mask;
    uint32_t krem = K;
    int shift = top;
    while (shift > 0) {
      const int nb = min(11, shift);
      shift -= nb;
      const uint32_t bmask = low_mask(nb);
      for (int j = threadIdx.x; j < TOPK_BINS; j += NT) hist[j] = 0;
      __syncthreads();
      for (int64_t s = threadIdx.x; s < n; s += NT) {
        const uint32_t u = score_key(S[s]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & bmask], 1u);
      }
      __syncthreads();
      // bins from the top: thread t owns bins top_bin - BPT*t - (0..BPT-1)
      constexpr int BPT = TOPK_BINS / NT;
      const int nbins = 1 << nb;
      uint32_t c[BPT];
      uint32_t sum = 0;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        const int bin = nbins - 1 - BPT * static_cast<int>(threadIdx.x) - e;
        c[e] = bin >= 0 ? hist[bin] : 0u;
        sum += c[e];
      }
      uint32_t tot;
      uint32_t above = block_excl_scan(sum, scratch, &tot);
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (above < krem && krem <= above + c[e]) {
          found[0] = static_cast<uint32_t>(nbins - 1 - BPT * static_cast<int>(threadIdx.x) - e);
          found[1] = above;
        }
        above += c[e];
      }
      __syncthreads();
      const uint32_t bin = found[0];
      krem -= found[1];
      prefix |= bin << shift;
      mask |= bmask << shift;
      __syncthreads();
    }
    vstar = prefix;
    r = krem;
  }

  // 3. ordered compaction
  uint32_t out_count = 0, eq_seen = 0;
  for (int64_t c0 = 0; c0 < n && out_count < static_cast<uint32_t>(K); c0 += NT * TOPK_E) {
    const int64_t base = c0 + static_cast<int64_t>(threadIdx.x) * TOPK_E;
    uint32_t u[TOPK_E];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < TOPK_E; ++e) {
      const int64_t s = base + e;
      u[e] = s < n ? score_key(S[s]) : 0u;
      const bool ok = s < n;
      gt += (ok && u[e] > vstar) ? 1u : 0u;
      eq += (ok && u[e] == vstar) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((gt << 16) | eq, scratch, &tot);
    const uint32_t gt_before = ex >> 16, eq_before = ex & 0xffffu;
    const uint32_t tot_gt = tot >> 16, tot_eq = tot & 0xffffu;
    uint32_t tie = eq_seen + eq_before;
    uint32_t pos = out_count + gt_before + (min(tie, r) - min(eq_seen, r));
#pragma unroll
    for (int e = 0; e < TOPK_E; ++e) {
      const int64_t s = base + e;
      if (s >= n) break;
      bool keep = u[e] > vstar;
      if (u[e] == vstar) {
        keep = tie < r;
        ++tie;
      }
      if (keep) {
        out[pos] = static_cast<int32_t>(s);
        if (outs) outs[pos] = key_score(u[e]);
        ++pos;
      }
    }
    out_count += tot_gt + (min(eq_seen + tot_eq, r) - min(eq_seen, r));
    eq_seen += tot_eq;
  }
}

hipError_t launch_topk_rows(const Geom& g, const int32_t* scores, int64_t stride,
                            int row_begin, int row_count, int32_t* idx, int32_t* sel,
                            hipStream_t st) {
  dim3 grid(row_count, g.B);
  hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TOPK_NT), 0, st, g.Tq, g.Tk, g.K,
                     g.q_offset, g.kv_len, scores, stride, row_begin, row_count, idx, sel);
  return hipGetLastError();
}

}  // namespace lci
