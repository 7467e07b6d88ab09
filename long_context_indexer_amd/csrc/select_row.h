// Exact Top-K of one score row by one workgroup (shared by the prefill Top-K
// kernel and the decode path's fallback).
//
// Order: higher score first, lower position on equal scores. The selected
// positions are written in ascending order. Steps:
//   1. min/max of the order-preserving uint32 keys fixes the varying low bits;
//   2. radix select, up to 11 bits per pass, with an LDS histogram (integer
//      atomics: order-independent, so the result is deterministic) finds the
//      exact K-th key v* and r = how many keys equal to v* are kept;
//   3. an ordered compaction in position order keeps every key > v* and the
//      first r keys == v*: one block-wide prefix scan per chunk of the packed
//      (count greater, count equal) pair gives each thread its output slot.
#pragma once

#include "common.h"

namespace lci {

constexpr int TOPK_NT = 512;         // threads per row
constexpr int TOPK_BINS = 2048;      // 11-bit digits
constexpr int TOPK_E = 4;            // elements per thread per compaction chunk

struct SelectLds {
  uint32_t hist[TOPK_BINS];
  uint32_t scratch[TOPK_NT / 64 + 2];
  uint32_t red[2 * (TOPK_NT / 64)];
  uint32_t found[2];
};

__device__ __forceinline__ uint32_t low_mask(int bits) {
  return bits >= 32 ? 0xffffffffu : ((1u << bits) - 1u);
}

__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* red) {
  constexpr int NT = TOPK_NT;
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

// Requires blockDim.x == TOPK_NT and n > K. Writes out[0..K-1] (and outs).
__device__ __forceinline__ void select_row(const int32_t* __restrict__ S, int64_t n, int K,
                                        int32_t* __restrict__ out, int32_t* __restrict__ outs,
                                        SelectLds& sm) {
  constexpr int NT = TOPK_NT;
  // 1. range of keys
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int64_t s = threadIdx.x; s < n; s += NT) {
    const uint32_t u = score_key(S[s]);
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_minmax(lo, hi, sm.red);

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
      for (int j = threadIdx.x; j < TOPK_BINS; j += NT) sm.hist[j] = 0;
      __syncthreads();
      for (int64_t s = threadIdx.x; s < n; s += NT) {
        const uint32_t u = score_key(S[s]);
        if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & bmask], 1u);
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
        c[e] = bin >= 0 ? sm.hist[bin] : 0u;
        sum += c[e];
      }
      uint32_t tot;
      uint32_t above = block_excl_scan(sum, sm.scratch, &tot);
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (above < krem && krem <= above + c[e]) {
          sm.found[0] = static_cast<uint32_t>(nbins - 1 - BPT * static_cast<int>(threadIdx.x) - e);
          sm.found[1] = above;
        }
        above += c[e];
      }
      __syncthreads();
      const uint32_t bin = sm.found[0];
      krem -= sm.found[1];
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
    const uint32_t ex = block_excl_scan((gt << 16) | eq, sm.scratch, &tot);
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

}  // namespace lci
