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
// Rows longer than 8192 positions, one workgroup per query row: two passes
// over the row with the keep mask in LDS (select_row_2pass: log-bin histogram
// and threshold bin, then keep bits above it and candidates inside it, exact
// rank among the candidates, ordered compaction of the mask). When the
// threshold bin holds too many candidates (heavy ties), the radix select:
//   1. min/max of the order-preserving uint32 keys fixes the varying low bits;
//   2. radix select, up to 11 bits per pass, with an LDS histogram (integer
//      atomics: order-independent, so the result is deterministic) finds the
//      exact K-th key v* and r = how many keys equal to v* are kept;
//   3. an ordered compaction in position order keeps every key > v* and the
//      first r keys == v*: one block-wide prefix scan per chunk of the packed
//      (count greater, count equal) pair gives each thread its output slot.
#include <type_traits>

#include "common.h"
#include "../../include/lci.h"
#include "internal.h"
#include "select_row.h"

namespace lci {

__global__ __launch_bounds__(TOPK_NT) void topk_rows_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ scores, int64_t stride,
    int64_t batch_rows, int row_begin, int row_count, int32_t* __restrict__ idx, int32_t* __restrict__ sel) {
  __shared__ union {
    SelectLds radix;
    Select2Lds mask2;
  } sm;
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
  const int32_t* S = scores + (static_cast<int64_t>(b) * batch_rows + rr) * stride;

  if (n <= K) {  // every candidate is kept (dense-equivalent row) or the row is invalid
    for (int j = threadIdx.x; j < K; j += TOPK_NT) {
      out[j] = j < n ? j : -1;
      if (outs) outs[j] = j < n ? S[j] : INT32_MIN;
    }
    return;
  }
  // two passes with the keep mask in LDS; the radix select when the row is
  // longer or the threshold bin holds too many candidates
  const bool vec = (reinterpret_cast<uintptr_t>(S) & 15) == 0;
  if (vec && n <= kSel2MaxN && select_row_2pass(S, static_cast<int>(n), K, out, outs, sm.mask2))
    return;
  __syncthreads();  // the radix select reuses the LDS
  select_row(S, n, K, out, outs, sm.radix);
}

// ---------------------------------------- four waves per row, row in registers
//
// Rows of at most kWaveTopkMax candidates. The row of n positions is cut into
// four segments of m = 256*ceil(n/1024) positions, one per wave; lane l of
// wave w holds chunk c at positions w*m + 256c + 4l .. +3, so the scores are
// read once (coalesced) and each wave's positions are contiguous. Steps:
//   1. min/max of the keys (positions >= n first hold copies of valid keys,
//      then the minimum key: they rank below every valid position, so with
//      more than K valid positions none is selected and no count above the
//      minimum changes; no step below tests validity);
//   2. radix passes, up to 11 bits each, with one LDS histogram per row; each
//      thread owns 8 bins from the top, a block prefix sum finds the bin of
//      the K-th largest key; updates that must not count go to a per-thread
//      dummy word (no branches, no bank conflicts);
//   3. ordered compaction: a count pass gives each wave the numbers of kept
//      and tied keys before its segment; then chunk by chunk, ballots of
//      (key > v*) and (key == v*) with lane-prefix popcounts give every kept
//      position its slot in an LDS copy of the output row, written out
//      coalesced at the end.
// With dense-path outputs, the kernel also writes the row flag of the
// dense-tile attention kernel (kRow* in internal.h) and, for masked rows, the
// bit mask of the kept positions.

namespace {

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}
// popcount of the bits of m held by lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}
// OR over each group of 8 lanes (DPP: swap pairs, swap pair-pairs, mirror 8)
__device__ __forceinline__ uint32_t or8(uint32_t v) {
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false));
  return v;
}

}  // namespace

constexpr int B4_CH = kWaveTopkMax / 1024;  // chunks per lane
constexpr int B4_NT = 256;
constexpr int B4_STAGE = 4096;              // output row staging (K <= 4096)

// Exclusive prefix sum over the four waves of a B4_NT-thread workgroup with a
// single barrier; *total receives the workgroup sum. `red` (4 words) must not
// be written again before a later barrier.
__device__ __forceinline__ uint32_t scan_b4(uint32_t v, int wv, uint32_t* red, uint32_t* total) {
  const uint32_t incl = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) red[wv] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = red[w];
    before += w < wv ? x : 0u;
    tot += x;
  }
  *total = tot;
  return before + incl - v;
}

// Six workgroups per CU (80 VGPRs, 26 KiB of LDS each): latency of the
// row's barriers and loads is hidden by the other rows on the CU.
__global__ __launch_bounds__(B4_NT, 6) void topk_b4_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ scores, int64_t stride,
    int64_t batch_rows, int row_begin, int row_count, int32_t* __restrict__ idx, int32_t* __restrict__ sel,
    uint32_t* __restrict__ dmask, uint8_t* __restrict__ dflag, int Wm, int lim) {
  // histogram (+ one dummy word per thread), staged output row (+ dummies)
  __shared__ __align__(16) uint32_t hist[TOPK_BINS + B4_NT];
  __shared__ __align__(16) uint32_t stage[B4_STAGE + B4_NT];
  __shared__ uint32_t red[8];
  __shared__ uint32_t segc[4];
  __shared__ uint32_t bc[2];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(t >> 6));
  const int rr = blockIdx.x;
  const int b = blockIdx.y;
  const int row = row_begin + rr;
  const int64_t grow = static_cast<int64_t>(b) * Tq + row;
  int32_t* out = idx + grow * K;
  int32_t* outs = sel ? sel + grow * K : nullptr;
  const int kvl = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + row;
  const bool valid = kvl <= Tk && p >= 0 && p < kvl;
  const int n = valid ? static_cast<int>(p + 1) : 0;  // n <= Tk <= kWaveTopkMax
  const int32_t* S = scores + (static_cast<int64_t>(b) * batch_rows + rr) * stride;

  if (n <= K) {  // every candidate is kept (dense-equivalent row) or the row is invalid
    for (int j = t; j < K; j += B4_NT) {
      out[j] = j < n ? j : -1;
      if (outs) outs[j] = j < n ? S[j] : INT32_MIN;
    }
    if (dflag && t == 0) dflag[grow] = valid ? kRowAll : kRowEmpty;
    if (dmask) {
      // the tile path's mask: all of 0..n-1
      for (int w = t; w < Wm; w += B4_NT) {
        const int nb = n - 32 * w;
        dmask[grow * Wm + w] = nb >= 32 ? 0xffffffffu : (nb <= 0 ? 0u : (1u << nb) - 1u);
      }
    }
    return;
  }
  const bool want_mask = dmask != nullptr && n <= lim;
  if (dflag && t == 0) dflag[grow] = want_mask ? kRowMasked : kRowGather;
  // the histogram starts at zero; each radix pass leaves it zero again
  for (int j = t; j < TOPK_BINS; j += B4_NT) hist[j] = 0u;
  const int m = 256 * ((n + 1023) >> 10);  // positions per wave segment
  const int nch = m >> 8;                   // chunks per lane, 1..B4_CH
  const int seg = wv * m;

  // 0. the row into registers: every load issued before any is used (one
  // memory round trip per row, not one per chunk); with 16-byte aligned rows,
  // 16-byte loads clamped to the last aligned group of the row
  const bool vec = (reinterpret_cast<uintptr_t>(S) & 15) == 0 && (stride & 3) == 0;
  uint32_t u[B4_CH][4];
  if (vec) {
    const int last4 = (n - 1) & ~3;
    int4 v4[B4_CH];
#pragma unroll
    for (int c = 0; c < B4_CH; ++c)
      v4[c] = *reinterpret_cast<const int4*>(S + min(seg + 256 * c + 4 * lane, last4));
#pragma unroll
    for (int c = 0; c < B4_CH; ++c) {
      u[c][0] = score_key(v4[c].x);
      u[c][1] = score_key(v4[c].y);
      u[c][2] = score_key(v4[c].z);
      u[c][3] = score_key(v4[c].w);
    }
  } else {
#pragma unroll
    for (int c = 0; c < B4_CH; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) u[c][e] = score_key(S[min(seg + 256 * c + 4 * lane + e, n - 1)]);
  }

  // 1. range of the keys, then positions >= n take the minimum
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int c = 0; c < B4_CH; ++c)
    if (c < nch)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo = min(lo, u[c][e]);
        hi = max(hi, u[c][e]);
      }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    red[2 * wv] = lo;
    red[2 * wv + 1] = hi;
  }
  __syncthreads();
  lo = min(min(red[0], red[2]), min(red[4], red[6]));
  hi = max(max(red[1], red[3]), max(red[5], red[7]));
#pragma unroll
  for (int c = 0; c < B4_CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) u[c][e] = seg + 256 * c + 4 * lane + e < n ? u[c][e] : lo;

  // 2. radix select of the K-th largest key v* and r = how many keys == v* are kept
  uint32_t vstar = lo, r = static_cast<uint32_t>(K);
  if (lo != hi) {
    const int top = 32 - __clz(lo ^ hi);  // bits [top-1:0] vary
    uint32_t mask = ~low_mask(top);
    uint32_t prefix = lo & mask;
    uint32_t krem = static_cast<uint32_t>(K);
    int shift = top;
    const int dummy = TOPK_BINS + t;
    while (shift > 0) {
      const int nb = min(11, shift);
      shift -= nb;
      const uint32_t bmask = low_mask(nb);
      const int nbins = 1 << nb;
#pragma unroll
      for (int c = 0; c < B4_CH; ++c)
        if (c < nch)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool hit = (u[c][e] & mask) == prefix;
            atomicAdd(&hist[hit ? static_cast<int>((u[c][e] >> shift) & bmask) : dummy], 1u);
          }
      __syncthreads();
      // thread t owns the 8 bins nbins-1-8t-7 .. nbins-1-8t (from the top); it
      // reads them and sets them back to zero for the next pass
      const int bhi = nbins - 1 - 8 * t;
      uint32_t cnt[8];
      uint32_t sum = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cnt[e] = 0u;
        if (bhi - e >= 0) {
          cnt[e] = hist[bhi - e];
          hist[bhi - e] = 0u;
        }
        sum += cnt[e];
      }
      uint32_t tot;
      uint32_t above = scan_b4(sum, wv, red, &tot);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (above < krem && krem <= above + cnt[e]) {
          bc[0] = static_cast<uint32_t>(bhi - e);
          bc[1] = above;
        }
        above += cnt[e];
      }
      __syncthreads();
      // bc is read before this thread's next barrier; it is rewritten only
      // after two more barriers
      const uint32_t bin = bc[0];
      krem -= bc[1];
      prefix |= bin << shift;
      mask |= bmask << shift;
    }
    vstar = prefix;
    r = krem;
  }

  // 3. ordered compaction. Counts of kept (> v*) and tied (== v*) keys per
  // segment give each wave its starting slot and tie rank.
  uint32_t ng = 0, nq = 0;
#pragma unroll
  for (int c = 0; c < B4_CH; ++c)
    if (c < nch)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ng += u[c][e] > vstar ? 1u : 0u;
        nq += u[c][e] == vstar ? 1u : 0u;
      }
  const uint32_t packed = wave_sum((ng << 16) | nq);  // both < 2^16 per wave
  if (lane == 0) segc[wv] = packed;
  __syncthreads();
  uint32_t gt_before = 0, eq_seen = 0;
  for (int w = 0; w < wv; ++w) {
    gt_before += segc[w] >> 16;
    eq_seen += segc[w] & 0xffffu;
  }
  // slots taken by earlier segments: their keys > v* plus their kept ties
  uint32_t out_count = gt_before + min(eq_seen, r);
  const int dummy_s = B4_STAGE + t;
  auto compact = [&](auto with_scores) {
    constexpr bool WS = decltype(with_scores)::value;
#pragma unroll
    for (int c = 0; c < B4_CH; ++c) {
      if (c < nch) {
        bool gt[4], eq[4];
        uint32_t gtb = 0, eqb = 0, tg = 0, tq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt[e] = u[c][e] > vstar;
          eq[e] = u[c][e] == vstar;
          const uint64_t G = __ballot(gt[e]);
          const uint64_t Q = __ballot(eq[e]);
          gtb += lanes_below(G);
          eqb += lanes_below(Q);
          tg += static_cast<uint32_t>(__builtin_popcountll(G));
          tq += static_cast<uint32_t>(__builtin_popcountll(Q));
        }
        uint32_t tie = eq_seen + eqb;
        uint32_t pos = out_count + gtb + (min(tie, r) - min(eq_seen, r));
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = gt[e] || (eq[e] && tie < r);
          tie += eq[e] ? 1u : 0u;
          const int spos = seg + 256 * c + 4 * lane + e;
          stage[keep ? static_cast<int>(pos) : dummy_s] = static_cast<uint32_t>(spos);
          if constexpr (WS) {
            if (keep) outs[pos] = key_score(u[c][e]);
          }
          pos += keep ? 1u : 0u;
          nib |= keep ? (1u << e) : 0u;
        }
        out_count += tg + (min(eq_seen + tq, r) - min(eq_seen, r));
        eq_seen += tq;
        if (want_mask) {
          const uint32_t word = or8(nib << (4 * (lane & 7)));
          const int wi = (seg >> 5) + 8 * c + (lane >> 3);
          if ((lane & 7) == 0 && wi < Wm) dmask[grow * Wm + wi] = word;
        }
      }
    }
  };
  if (outs)
    compact(std::true_type{});
  else
    compact(std::false_type{});
  if (want_mask)  // words past the four segments
    for (int wi = (4 * m >> 5) + t; wi < Wm; wi += B4_NT) dmask[grow * Wm + wi] = 0u;
  __syncthreads();
  if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    for (int j = 4 * t; j < K; j += 4 * B4_NT)
      *reinterpret_cast<uint4*>(out + j) = *reinterpret_cast<const uint4*>(stage + j);
  } else {
    for (int j = t; j < K; j += B4_NT) out[j] = static_cast<int32_t>(stage[j]);
  }
}

hipError_t launch_topk_rows(const Geom& g, const int32_t* scores, int64_t stride,
                            int64_t batch_rows, int row_begin, int row_count, int32_t* idx,
                            int32_t* sel,
                            const DenseMasks* dm, hipStream_t st) {
  if (g.Tk <= kWaveTopkMax) {
    dim3 grid(row_count, g.B);
    KernelTimer timer(LCI_KERNEL_TOPK, st);
    hipLaunchKernelGGL(topk_b4_kernel, grid, dim3(B4_NT), 0, st, g.Tq, g.Tk, g.K, g.q_offset,
                       g.kv_len, scores, stride, batch_rows, row_begin, row_count, idx, sel,
                       dm ? dm->mask : nullptr, dm ? dm->flag : nullptr, dm ? dm->Wm : 0,
                       dm ? dm->lim : 0);
    return hipGetLastError();
  }
  if (dm) return hipErrorInvalidValue;  // dense masks come from the wave kernel only
  dim3 grid(row_count, g.B);
  {
    KernelTimer timer(LCI_KERNEL_TOPK, st);
    hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TOPK_NT), 0, st, g.Tq, g.Tk, g.K,
                       g.q_offset, g.kv_len, scores, stride, batch_rows, row_begin, row_count, idx, sel);
  }
  return hipGetLastError();
}

}  // namespace lci
