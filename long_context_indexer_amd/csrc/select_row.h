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

// Monotone map int32 -> [0, 2048) (2048 log-spaced bins): 1024 + f(s) for s >= 0, 1023 - f(~s) for s < 0,
// f(t) = 32*bitlength(t) + the 5 bits after the leading one (exact below 64).
__device__ __forceinline__ int score_bin(int32_t s) {
  const uint32_t t = s >= 0 ? static_cast<uint32_t>(s) : ~static_cast<uint32_t>(s);
  const int e = 32 - __clz(t);
  const uint32_t m = e > 5 ? (t >> (e - 6)) & 31u : (t << (6 - e)) & 31u;
  const int f = e * 32 + static_cast<int>(m);
  return s >= 0 ? 1024 + f : 1023 - f;
}

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

// ------------------------------------------------ two passes, mask in LDS
//
// Rows of at most kSel2MaxN positions (one workgroup, TOPK_NT threads):
//   1. pass over the row: histogram of score_bin (2048 log-spaced bins, LDS
//      integer atomics), then the bin b* that holds the K-th largest score and
//      the count of positions in higher bins;
//   2. pass over the row: positions in bins above b* set their bit of an LDS
//      keep mask, positions inside b* go to an LDS candidate list;
//   3. a candidate is kept when fewer than K - (count above b*) candidates
//      precede it under (score desc, position asc): its bit joins the mask;
//   4. ordered compaction of the mask: ascending positions.
// Two reads of the row instead of four or five for the radix select. Returns
// false (nothing written) when the candidates overflow their capacity.
// S must be 16-byte aligned.
constexpr int kSel2MaxN = 131072;
constexpr int kSel2Cap = 1024;
constexpr int kSel2U = 8;  // 16-byte loads in flight per thread

// f(position, score) over positions 0..n-1 of a 16-byte aligned row: thread t
// takes the 4-position groups t, t + NT, ..., kSel2U loads issued before any
// is used (a row pass is latency bound otherwise: one memory round trip per
// element).
template <typename F>
__device__ __forceinline__ void for_each_score4(const int32_t* __restrict__ S, int n, F f) {
  constexpr int NT = TOPK_NT;
  const int ng = (n + 3) / 4;
  const int4* S4 = reinterpret_cast<const int4*>(S);
  for (int g0 = 0; g0 < ng; g0 += NT * kSel2U) {
    int4 v[kSel2U];
#pragma unroll
    for (int u = 0; u < kSel2U; ++u) v[u] = S4[min(g0 + u * NT + static_cast<int>(threadIdx.x), ng - 1)];
#pragma unroll
    for (int u = 0; u < kSel2U; ++u) {
      const int p0 = 4 * (g0 + u * NT + static_cast<int>(threadIdx.x));
      if (p0 < n) f(p0, v[u].x);
      if (p0 + 1 < n) f(p0 + 1, v[u].y);
      if (p0 + 2 < n) f(p0 + 2, v[u].z);
      if (p0 + 3 < n) f(p0 + 3, v[u].w);
    }
  }
}

struct Select2Lds {
  uint32_t hist[TOPK_BINS];
  uint32_t keep[kSel2MaxN / 32];
  int2 cand[kSel2Cap + 16];
  uint32_t scratch[TOPK_NT / 64 + 2];
  uint32_t found[2];
  uint32_t ncand;
};

__device__ __forceinline__ bool select_row_2pass(const int32_t* __restrict__ S, int n, int K,
                                                 int32_t* __restrict__ out,
                                                 int32_t* __restrict__ outs, Select2Lds& sm) {
  constexpr int NT = TOPK_NT;
  const int t = threadIdx.x;
  const int nw = (n + 31) / 32;
  for (int j = t; j < TOPK_BINS; j += NT) sm.hist[j] = 0u;
  for (int j = t; j < nw; j += NT) sm.keep[j] = 0u;
  if (t == 0) sm.ncand = 0u;
  __syncthreads();
  // 1. histogram and threshold bin
  for_each_score4(S, n, [&](int, int32_t v) { atomicAdd(&sm.hist[score_bin(v)], 1u); });
  __syncthreads();
  constexpr int BPT = TOPK_BINS / NT;
  uint32_t c[BPT];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    c[e] = sm.hist[TOPK_BINS - 1 - BPT * t - e];
    sum += c[e];
  }
  uint32_t tot;
  uint32_t above = block_excl_scan(sum, sm.scratch, &tot);
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    if (above < static_cast<uint32_t>(K) && static_cast<uint32_t>(K) <= above + c[e]) {
      sm.found[0] = static_cast<uint32_t>(TOPK_BINS - 1 - BPT * t - e);
      sm.found[1] = above;
    }
    above += c[e];
  }
  __syncthreads();
  const int bstar = static_cast<int>(sm.found[0]);
  const uint32_t krem = static_cast<uint32_t>(K) - sm.found[1];
  // 2. keep mask above b*, candidates inside b*
  for_each_score4(S, n, [&](int s, int32_t v) {
    const int bin = score_bin(v);
    if (bin > bstar) {
      atomicOr(&sm.keep[s >> 5], 1u << (s & 31));
    } else if (bin == bstar) {
      const uint32_t slot = atomicAdd(&sm.ncand, 1u);
      if (slot < static_cast<uint32_t>(kSel2Cap)) sm.cand[slot] = make_int2(v, s);
    }
  });
  __syncthreads();
  const int nc = static_cast<int>(sm.ncand);
  if (nc > kSel2Cap) return false;  // uniform: read after the barrier
  // 3. rank of each candidate by direct count (broadcast LDS reads, 16 at a
  // time); entries past nc are padded with a pair that precedes nothing
  const int npad = (nc + 15) & ~15;
  for (int i = nc + t; i < npad; i += NT) sm.cand[i] = make_int2(INT32_MIN, INT32_MAX);
  __syncthreads();
  for (int i = t; i < nc; i += NT) {
    const int2 ci = sm.cand[i];
    uint32_t rank = 0;
    for (int j0 = 0; j0 < npad; j0 += 16) {
      int4 qv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) qv[u] = *reinterpret_cast<const int4*>(&sm.cand[j0 + 2 * u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        rank += (qv[u].x > ci.x || (qv[u].x == ci.x && qv[u].y < ci.y)) ? 1u : 0u;
        rank += (qv[u].z > ci.x || (qv[u].z == ci.x && qv[u].w < ci.y)) ? 1u : 0u;
      }
    }
    if (rank < krem) atomicOr(&sm.keep[ci.y >> 5], 1u << (ci.y & 31));
  }
  __syncthreads();
  // 4. ordered compaction: thread t takes the words [t * wpt, (t + 1) * wpt)
  constexpr int WMAX = kSel2MaxN / 32 / NT;
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = t * wpt;
  uint32_t wr[WMAX];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < WMAX; ++j) {
    wr[j] = (j < wpt && w0 + j < nw) ? sm.keep[w0 + j] : 0u;
    mine += static_cast<uint32_t>(__popc(wr[j]));
  }
  uint32_t total;
  uint32_t slot = block_excl_scan(mine, sm.scratch, &total);
#pragma unroll
  for (int j = 0; j < WMAX; ++j) {
    uint32_t word = wr[j];
    while (word != 0u) {
      const int bit = __ffs(static_cast<int>(word)) - 1;
      word &= word - 1u;
      const int pos = 32 * (w0 + j) + bit;
      if (slot < static_cast<uint32_t>(K)) {
        out[slot] = pos;
        if (outs) outs[slot] = S[pos];
      }
      ++slot;
    }
  }
  return true;
}

}  // namespace lci
