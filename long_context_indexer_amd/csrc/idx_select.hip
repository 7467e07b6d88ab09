// Long-prefill scoring and Top-K without materialised score rows (gfx950).
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer + Top-K:
// How Fine-Grained Sparse Attention Works", steps 1-2 (score every causal
// position, keep the K best), and its section "Engineering and Evaluation
// Recommendations" (Top-K needs fused kernels); "From Linear Attention to Gated
// Sparse Attention", section 4 (whether the sorting overhead can be fused into
// kernels). A score row of a 64K-token prefill is 256 KiB; written out and read
// back twice for every row it is 17 GB of traffic. Here the scores stay in
// registers:
//
//   sel_scan_kernel   one wave per 16 consecutive query rows of a sequence. For
//                     rows with more than `cap` candidates, two sampled passes
//                     set a per-row threshold t: every 32nd position fills a
//                     64-bin histogram (sign and bit length of the score), which
//                     names the coarse bin holding the estimated K-th score;
//                     every 8th position then fills 256 linear sub-bins of that
//                     bin. t is the lowest score of the sub-bin where the count
//                     of sampled scores at or above it first reaches
//                     K*f + 4*sqrt(K*f) + 2 (f: the sampled fraction of the row),
//                     so that about K + 4 standard deviations of the row's
//                     positions score at least t. One full pass then scores every
//                     causal position (int8 MFMA 16x16x64, positions as MFMA rows,
//                     one indexer head per MFMA, as in the scoring kernel) and
//                     appends each (score, position) with score >= t to the row's
//                     candidate list (LDS counters, at most cap stored). Rows
//                     with at most cap candidates take every position.
//   sel_rows_kernel   one workgroup per row. When the list holds every position
//                     whose score is >= t and at least K of them (count in
//                     [K, cap]), the row's Top-K is the Top-K of the list: an
//                     exact radix select of the K-th key under (score desc,
//                     position asc) over the list in LDS, the kept positions set
//                     in an LDS bit map of the row (ties at the K-th score: the
//                     lowest positions), and an ordered compaction of the map
//                     writes the ascending index row. Any other count (the
//                     threshold missed: too few or too many scores >= t) puts the
//                     row on the fallback list.
//   sel_fallback_kernel  the listed rows, exactly as the materialised path does
//                     them: the row's scores into a scratch row, then the same
//                     one-workgroup selection (select_row_2pass, or the radix
//                     select) as the Top-K kernel over score rows.
// The result is exact whatever the threshold: a row is only finished from its
// list when the list provably contains its Top-K.
#include <math.h>

#include "common.h"
#include "../../include/lci.h"
#include "internal.h"
#include "select_row.h"

namespace lci {

constexpr int SEL_SS1 = 32;    // stride of the coarse sample
constexpr int SEL_SS2 = 8;     // stride of the fine sample
constexpr int SEL_CB = 64;     // coarse bins
constexpr int SEL_FB = 256;    // fine bins inside one coarse bin
constexpr int SEL_NT = 256;    // threads of the per-row selection
constexpr int SEL_FB_GRID = 64;  // workgroups of the fallback kernel

// Candidate list capacity for K: the expected count plus seven standard
// deviations of the sampled estimate, and a margin for the sub-bin width.
int sel_cap(int K) {
  const double kf = static_cast<double>(K);
  const double expect = kf + 4.0 * sqrt(kf * SEL_SS2) + 2.0 * SEL_SS2;
  const double c = expect + 7.0 * sqrt(SEL_SS2 * expect) + 64.0;
  return (static_cast<int>(c) + 255) / 256 * 256;
}

// Coarse bin of a score: monotone, 64 bins by sign and bit length
// (s >= 0: 32 + bitlength(s); s < 0: 31 - bitlength(~s)).
__device__ __forceinline__ int sel_cbin(int32_t s) {
  const uint32_t t = s >= 0 ? static_cast<uint32_t>(s) : ~static_cast<uint32_t>(s);
  const int e = 32 - __clz(t);
  return s >= 0 ? 32 + e : 31 - e;
}

// Key range [ulo, uhi] (score_key order) of coarse bin cb.
__device__ __forceinline__ void sel_cbin_range(int cb, uint32_t& ulo, uint32_t& uhi) {
  int64_t slo, shi;
  if (cb >= 33) {
    const int e = cb - 32;
    slo = int64_t(1) << (e - 1);
    shi = (int64_t(1) << e) - 1;
  } else if (cb == 32) {
    slo = shi = 0;
  } else {
    const int e = 31 - cb;
    if (e == 0) {
      slo = shi = -1;
    } else {
      slo = -(int64_t(1) << e);
      shi = -(int64_t(1) << (e - 1)) - 1;
    }
  }
  ulo = score_key(static_cast<int32_t>(slo));
  uhi = score_key(static_cast<int32_t>(shi));
}

// Shift that maps a key range of width uhi - ulo onto at most 256 sub-bins.
__device__ __forceinline__ int sel_fshift(uint32_t ulo, uint32_t uhi) {
  const uint32_t wdt = uhi - ulo;
  const int bl = 32 - __clz(wdt);
  return bl > 8 ? bl - 8 : 0;
}

// Sampled scores a row needs to see at or above its threshold: f = ns / n of
// the row is sampled, so K*f are expected among the K best; four standard
// deviations and two more keep the full count at or above K but for rare rows.
__device__ __forceinline__ int sel_target(int K, int ns, int n) {
  const float kf = static_cast<float>(K) * static_cast<float>(ns) / static_cast<float>(n);
  return static_cast<int>(ceilf(kf + 4.f * sqrtf(kf) + 2.f));
}

// Histogram counters are 16-bit, two to a word (bin j in half j & 1 of word
// j >> 1): a row samples at most kSelMaxTk / SEL_SS2 = 16384 positions, so no
// count carries into its neighbour.
static_assert(kSelMaxTk / SEL_SS2 < 65536, "16-bit histogram counters");
struct SelScanLds {
  uint32_t hist[16][SEL_FB / 2];   // coarse (first SEL_CB / 2 words of a row), fine, then
                                   // the candidates' histogram
  uint32_t cnt[16];                // candidates of each row
  int32_t thr[16];                 // threshold of each row
  int32_t cb[16];                  // coarse bin of each row
  uint32_t hb[16];                 // key at the bottom of the candidates' histogram
  int32_t hsh[16];                 // its bin width, log2
};

// Per-row summary the scan leaves for the row kernel: the candidates'
// histogram is 256 bins of width 2^hsh over keys from hb up (keys below hb in
// bin 0, keys past the top in bin 255); kbin is the bin holding the K-th
// largest listed key and above the count of listed keys in higher bins.
struct SelMeta {
  uint32_t hb;
  int32_t hsh, kbin;
  uint32_t above;
};

__device__ __forceinline__ uint32_t sel_hbin(uint32_t key, uint32_t hb, int hsh) {
  return key < hb ? 0u : min((key - hb) >> hsh, static_cast<uint32_t>(SEL_FB - 1));
}

// a * b + c for 24-bit signed a, b (one v_mad_i32_i24: the compiler would
// otherwise pair the products into v_add3, three operations per two terms)
__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm volatile("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt left at their maxima)
constexpr int kWaitVm0 = 0x0F70;

// One wave: 16 query rows rb*16 .. rb*16+15 of sequence b (a set's rows).
// q_idx [B, Tq, H_I, D_I] (this set's heads), k_idx [B, Tk, D_I], w [H_I]
// shared by every row. cand [B*Tq][cap] int2 (score, position), cnt [B*Tq]
// (the true count, possibly above cap), meta [B*Tq]. nfb: the fallback list's
// length, zeroed here for the row kernel that follows.
template <int H_I, int D_I>
__global__ __launch_bounds__(64, 3) void sel_scan_kernel(
    int Tq, int Tk, int K, int cap, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const int8_t* __restrict__ w, int2* __restrict__ cand,
    uint32_t* __restrict__ cnt, SelMeta* __restrict__ meta, uint32_t* __restrict__ nfb) {
  constexpr int NCH = D_I / 64;  // 64-deep MFMA steps over d_I
  constexpr int U = 2;           // 16-position tiles per step
  __shared__ SelScanLds sm;
  const int lane = threadIdx.x;
  const int nrb = (Tq + 15) / 16;
  const int rb = nrb - 1 - static_cast<int>(blockIdx.x);  // longest rows first
  const int b = blockIdx.y;
  if (blockIdx.x == 0 && blockIdx.y == 0 && lane == 0) *nfb = 0u;
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int i = rb * 16 + r;
  const int kvl0 = kv_len[b];
  const int kvl = kvl0 <= Tk ? kvl0 : 0;
  const int64_t p64 = static_cast<int64_t>(q_offset[b]) + i;
  const bool rok = i < Tq && p64 >= 0 && p64 < kvl;
  const int p = rok ? static_cast<int>(p64) : -1;   // causal limit of this lane's row
  const int n = p + 1;                              // candidates of the row
  // a row that keeps everything (n <= K) needs no list; the others sample a
  // threshold (rows with at most cap positions may end up listing all)
  const bool listed = n > K;
  if (lane < 16) {
    sm.cnt[r] = 0u;
    sm.thr[r] = INT32_MIN;
  }
  for (int j = lane; j < 16 * (SEL_CB / 2); j += 64) sm.hist[j / (SEL_CB / 2)][j % (SEL_CB / 2)] = 0u;
  int pmax = p;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) pmax = max(pmax, __shfl_xor(pmax, off, 64));
  pmax = __builtin_amdgcn_readfirstlane(pmax);
  if (pmax < 0) return;  // no valid row: the row kernel writes the -1 rows
  const bool any_listed = __any(listed);
  if (!any_listed) return;  // every row keeps all of 0..p

  // B operands: query row i of every head (rows past the end read row rb*16, zeroed)
  v4i bq[H_I][NCH];
  {
    const int ic = i < Tq ? i : rb * 16;
    const int8_t* src = q_idx + (static_cast<int64_t>(b) * Tq + ic) * H_I * D_I + 16 * g4;
#pragma unroll
    for (int h = 0; h < H_I; ++h)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const v4i t = *reinterpret_cast<const v4i*>(src + h * D_I + 64 * c);
        const v4i z = {0, 0, 0, 0};
        bq[h][c] = i < Tq ? t : z;
      }
  }
  int wh[H_I];
#pragma unroll
  for (int h = 0; h < H_I; ++h) wh[h] = static_cast<int>(w[h]);
  const int8_t* kbase = k_idx + static_cast<int64_t>(b) * Tk * D_I + 16 * g4;

  // k fragments of the 2x16 MFMA rows at positions pos0 + stride*(16u + m),
  // m = lane % 16 (positions past pmax read row pmax; never counted)
  auto load_keys = [&](int pos0, int stride, v4i (&dst)[U][NCH]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int keyc = min(pos0 + stride * (16 * u + r), pmax);
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        dst[u][c] = *reinterpret_cast<const v4i*>(kbase + static_cast<int64_t>(keyc) * D_I + 64 * c);
    }
  };
  // scores of this lane's row at positions pos0 + stride*(16u + 4*g4 + e): per
  // 16-position tile, every head's MFMA first, then the weighted ReLU sum
  auto score = [&](const v4i (&ka)[U][NCH], v4i (&sacc)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i acc[H_I];
#pragma unroll
      for (int h = 0; h < H_I; ++h) {
        acc[h] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          acc[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka[u][c], bq[h][c], acc[h], 0, 0, 0);
      }
      sacc[u] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < H_I; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[u][e] = mad_i24(wh[h], max(acc[h][e], 0), sacc[u][e]);
    }
  };
  // f(position, score) over this lane's causal positions of a strided sweep
  auto sweep = [&](int stride, int last, auto&& f) {
    const int span = 32 * stride;  // positions covered by one step
    v4i ka[U][NCH];
    load_keys(0, stride, ka);
    for (int pos0 = 0; pos0 <= last; pos0 += span) {
      v4i kn[U][NCH];
      load_keys(pos0 + span, stride, kn);
      v4i sacc[U];
      score(ka, sacc);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = pos0 + stride * (16 * u + 4 * g4 + e);
          if (pos <= p) f(pos, sacc[u][e]);
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NCH; ++c) ka[u][c] = kn[u][c];
    }
  };

  __syncthreads();
  // 1. coarse sample
  sweep(SEL_SS1, pmax, [&](int, int32_t s) {
    if (listed) {
      const int cb = sel_cbin(s);
      atomicAdd(&sm.hist[r][cb >> 1], 1u << (16 * (cb & 1)));
    }
  });
  __syncthreads();
  if (lane < 16 && listed) {
    const int ns = p / SEL_SS1 + 1;
    const uint32_t tgt = static_cast<uint32_t>(sel_target(K, ns, n));
    uint32_t cum = 0;
    int cb = 0;
    for (int bb = SEL_CB - 1; bb >= 0; --bb) {
      cum += (sm.hist[r][bb >> 1] >> (16 * (bb & 1))) & 0xffffu;
      if (cum >= tgt) {
        cb = bb;
        break;
      }
    }
    sm.cb[r] = cb;
  }
  __syncthreads();
  for (int j = lane; j < 16 * (SEL_FB / 2); j += 64) sm.hist[j / (SEL_FB / 2)][j % (SEL_FB / 2)] = 0u;
  __syncthreads();
  // 2. fine sample inside the coarse bin; the count above it; the sampled range
  uint32_t ulo = 0, uhi = 0;
  int fsh = 0;
  const int cb = listed ? sm.cb[r] : 0;
  if (listed) {
    sel_cbin_range(cb, ulo, uhi);
    fsh = sel_fshift(ulo, uhi);
  }
  uint32_t above = 0, kmin = 0xffffffffu, kmax = 0u;
  sweep(SEL_SS2, pmax, [&](int, int32_t s) {
    if (!listed) return;
    const uint32_t key = score_key(s);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
    const int sb = sel_cbin(s);
    if (sb > cb) {
      ++above;
    } else if (sb == cb) {
      const uint32_t fb = (key - ulo) >> fsh;
      atomicAdd(&sm.hist[r][fb >> 1], 1u << (16 * (fb & 1)));
    }
  });
  // the row's four lanes combine their counts and ranges
  above += __shfl_xor(above, 16, 64);
  above += __shfl_xor(above, 32, 64);
  kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), 16, 64)));
  kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), 32, 64)));
  kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), 16, 64)));
  kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), 32, 64)));
  __syncthreads();
  if (lane < 16 && listed) {
    const int ns = p / SEL_SS2 + 1;
    const uint32_t tgt = static_cast<uint32_t>(sel_target(K, ns, n));
    uint32_t t;
    if (above >= tgt) {
      // the coarse sample put the bin too low: everything above it
      t = uhi + 1u;
    } else {
      uint32_t cum = above;
      t = ulo;  // the whole bin when even it falls short
      for (int fb = SEL_FB - 1; fb >= 0; --fb) {
        cum += (sm.hist[r][fb >> 1] >> (16 * (fb & 1))) & 0xffffu;
        if (cum >= tgt) {
          t = ulo + (static_cast<uint32_t>(fb) << fsh);
          break;
        }
      }
      // too few samples to reach the target: every position is a candidate
      if (cum < tgt) t = 0u;
    }
    sm.thr[r] = key_score(t);
    // the candidates' histogram spans the sampled keys from the threshold up
    const uint32_t hb = max(t, kmin);
    sm.hb[r] = hb;
    sm.hsh[r] = kmax > hb ? sel_fshift(hb, kmax) : 0;
  }
  for (int j = lane; j < 16 * (SEL_FB / 2); j += 64) sm.hist[j / (SEL_FB / 2)][j % (SEL_FB / 2)] = 0u;
  __syncthreads();

  // 3. full pass: every causal position at or above the row's threshold. Each
  // step first stores the previous step's candidates (their slots came from one
  // LDS atomic per lane, issued a step earlier), then issues the next step's
  // key loads, then scores this step: the stores are older than every load a
  // later wait covers.
  const int32_t thr = sm.thr[r];
  const uint32_t hb = sm.hb[r];
  const int hsh = sm.hsh[r];
  const int plist = listed ? p : -1;  // causal limit of the listed positions
  // steps wholly at or below every listed row's limit need no position test
  int pmin = listed ? p : INT32_MAX;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) pmin = min(pmin, __shfl_xor(pmin, off, 64));
  pmin = __builtin_amdgcn_readfirstlane(pmin);
  int2* crow = cand + (static_cast<int64_t>(b) * Tq + (i < Tq ? i : 0)) * cap;
  v4i ka[U][NCH];
  load_keys(0, 1, ka);
  uint32_t pm = 0u, pslot = 0u;
  v4i ps[U] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
  int ppos = 0;
  for (int pos0 = 0; pos0 <= pmax + 32; pos0 += 32) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_sched_barrier(0);
    // the previous step's candidates
    if (pm != 0u) {
      uint32_t mm = pm, slot = pslot;
      while (mm != 0u) {
        const int k = __ffs(static_cast<int>(mm)) - 1;  // bit 4u + e: position 16u + 4*g4 + e
        mm &= mm - 1u;
        const bool hi = (k & 4) != 0, b1 = (k & 2) != 0, b0 = (k & 1) != 0;
        const int32_t a0 = hi ? ps[1][0] : ps[0][0], a1 = hi ? ps[1][1] : ps[0][1];
        const int32_t a2 = hi ? ps[1][2] : ps[0][2], a3 = hi ? ps[1][3] : ps[0][3];
        const int32_t c0 = b1 ? a2 : a0, c1 = b1 ? a3 : a1;
        const int32_t sc = b0 ? c1 : c0;
        if (slot < static_cast<uint32_t>(cap)) {
          crow[slot] = make_int2(sc, ppos + 4 * (k & 4) + 4 * g4 + (k & 3));
          const uint32_t hbin = sel_hbin(score_key(sc), hb, hsh);
          atomicAdd(&sm.hist[r][hbin >> 1], 1u << (16 * (hbin & 1)));
        }
        ++slot;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pos0 > pmax) break;
    v4i kn[U][NCH];
    load_keys(pos0 + 32, 1, kn);
    __builtin_amdgcn_sched_barrier(0);
    v4i sacc[U];
    score(ka, sacc);
    uint32_t m = 0u;
    if (pos0 + 31 <= pmin) {  // uniform
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) m |= static_cast<uint32_t>(sacc[u][e] >= thr) << (4 * u + e);
      m = listed ? m : 0u;
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = pos0 + 16 * u + 4 * g4 + e;
          m |= static_cast<uint32_t>((sacc[u][e] >= thr) & (pos <= plist)) << (4 * u + e);
        }
    }
    pm = m;
    ps[0] = sacc[0];
    ps[1] = sacc[1];
    ppos = pos0;
    if (m != 0u) pslot = atomicAdd(&sm.cnt[r], static_cast<uint32_t>(__popc(m)));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c) ka[u][c] = kn[u][c];
  }
  __syncthreads();
  if (lane < 16 && i < Tq) {
    const uint32_t c = sm.cnt[r];
    cnt[static_cast<int64_t>(b) * Tq + i] = c;
    SelMeta mt{hb, hsh, -1, 0u};
    if (listed && c >= static_cast<uint32_t>(K) && c <= static_cast<uint32_t>(cap)) {
      uint32_t cum = 0;
      for (int bb = SEL_FB - 1; bb >= 0; --bb) {
        const uint32_t h = (sm.hist[r][bb >> 1] >> (16 * (bb & 1))) & 0xffffu;
        if (cum + h >= static_cast<uint32_t>(K)) {
          mt.kbin = bb;
          mt.above = cum;
          break;
        }
        cum += h;
      }
    }
    meta[static_cast<int64_t>(b) * Tq + i] = mt;
  }
}

constexpr int SEL_SMALL = 1024;  // list entries in the K-th score's bin resolved in LDS

// One workgroup per (row, sequence). The list of row (b, i) holds cnt entries
// (at most cap stored) and its histogram summary meta. The row's Top-K is every
// listed key in a bin above meta.kbin plus the (K - meta.above) best of the
// entries in that bin (ranked by direct count), set in an LDS bit map of the
// row and compacted in position order. idx rows at idx + (b*out_tq + i)*K.
// Rows whose list cannot give their Top-K (count outside [K, cap], or more
// than SEL_SMALL entries in the K-th bin) go to the fallback list.
__global__ __launch_bounds__(SEL_NT) void sel_rows_kernel(
    int Tq, int Tk, int K, int cap, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int2* __restrict__ cand,
    const uint32_t* __restrict__ cnt, const SelMeta* __restrict__ meta,
    int32_t* __restrict__ idx, int out_tq, uint32_t* __restrict__ nfb,
    int32_t* __restrict__ fb_rows) {
  extern __shared__ __align__(16) uint32_t keep[];  // ceil(Tk/32) words
  __shared__ int2 small[SEL_SMALL];
  __shared__ uint32_t scratch[SEL_NT / 64 + 2];
  __shared__ uint32_t nsmall;

  const int t = threadIdx.x;
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int kvl0 = kv_len[b];
  const int kvl = kvl0 <= Tk ? kvl0 : 0;
  const int64_t p64 = static_cast<int64_t>(q_offset[b]) + i;
  const bool rok = p64 >= 0 && p64 < kvl;
  const int n = rok ? static_cast<int>(p64) + 1 : 0;
  int32_t* out = idx + (static_cast<int64_t>(b) * out_tq + i) * K;
  if (n <= K) {  // every position kept, or an invalid row
    for (int j = t; j < K; j += SEL_NT) out[j] = j < n ? j : -1;
    return;
  }
  const int64_t row = static_cast<int64_t>(b) * Tq + i;
  const uint32_t c = cnt[row];
  const SelMeta mt = meta[row];
  if (mt.kbin < 0) {  // count outside [K, cap]: the threshold missed
    if (t == 0) fb_rows[atomicAdd(nfb, 1u)] = static_cast<int32_t>(row);
    return;
  }
  const int nc = static_cast<int>(c);
  const int nw = (n + 31) / 32;
  for (int j = t; j < nw; j += SEL_NT) keep[j] = 0u;
  if (t == 0) nsmall = 0u;
  __syncthreads();
  const int2* crow = cand + row * cap;
  const uint32_t kb = static_cast<uint32_t>(mt.kbin);
  for (int j = t; j < nc; j += SEL_NT) {
    const int2 e = crow[j];
    const uint32_t hbin = sel_hbin(score_key(e.x), mt.hb, mt.hsh);
    if (hbin > kb) {
      atomicOr(&keep[e.y >> 5], 1u << (e.y & 31));
    } else if (hbin == kb) {
      const uint32_t sl = atomicAdd(&nsmall, 1u);
      if (sl < static_cast<uint32_t>(SEL_SMALL)) small[sl] = e;
    }
  }
  __syncthreads();
  const int ns = static_cast<int>(nsmall);
  if (ns > SEL_SMALL) {  // uniform: read after the barrier
    if (t == 0) fb_rows[atomicAdd(nfb, 1u)] = static_cast<int32_t>(row);
    return;
  }
  // the bin's entries: kept when fewer than K - above of them precede it under
  // (score desc, position asc)
  const uint32_t need = static_cast<uint32_t>(K) - mt.above;
  for (int j = t; j < ns; j += SEL_NT) {
    const int2 ej = small[j];
    uint32_t rank = 0;
    for (int q = 0; q < ns; ++q) {
      const int2 eq = small[q];
      rank += (eq.x > ej.x || (eq.x == ej.x && eq.y < ej.y)) ? 1u : 0u;
    }
    if (rank < need) atomicOr(&keep[ej.y >> 5], 1u << (ej.y & 31));
  }
  __syncthreads();
  // ordered compaction: thread t takes words [t*wpt, (t+1)*wpt)
  const int wpt = (nw + SEL_NT - 1) / SEL_NT;
  const int w0 = t * wpt;
  uint32_t mine = 0;
  for (int j = 0; j < wpt; ++j)
    if (w0 + j < nw) mine += static_cast<uint32_t>(__popc(keep[w0 + j]));
  uint32_t tot;
  uint32_t slot = block_excl_scan(mine, scratch, &tot);
  for (int j = 0; j < wpt; ++j) {
    const int wj = w0 + j;
    if (wj >= nw) break;
    uint32_t word = keep[wj];
    while (word != 0u) {
      const int bit = __ffs(static_cast<int>(word)) - 1;
      word &= word - 1u;
      if (slot < static_cast<uint32_t>(K)) out[slot] = 32 * wj + bit;
      ++slot;
    }
  }
}

// The rows the list could not finish, exactly: scores of the whole row into the
// workgroup's scratch row, then the Top-K kernel's own row selection.
template <int H_I, int D_I>
__global__ __launch_bounds__(TOPK_NT) void sel_fallback_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const int8_t* __restrict__ w,
    const uint32_t* __restrict__ nfb, const int32_t* __restrict__ fb_rows,
    int32_t* __restrict__ scratch, int64_t srow_stride, int32_t* __restrict__ idx, int out_tq) {
  __shared__ union {
    SelectLds radix;
    Select2Lds mask2;
  } sm;
  __shared__ __align__(16) int8_t qrow[H_I * D_I];
  const uint32_t nrows = *nfb;
  int32_t* S = scratch + static_cast<int64_t>(blockIdx.x) * srow_stride;
  for (uint32_t j = blockIdx.x; j < nrows; j += gridDim.x) {
    const int64_t row = fb_rows[j];
    const int b = static_cast<int>(row / Tq);
    const int i = static_cast<int>(row % Tq);
    const int p = q_offset[b] + i;  // a listed row is valid with more than K candidates
    const int n = p + 1;
    for (int e = threadIdx.x; e < H_I * D_I; e += TOPK_NT)
      qrow[e] = q_idx[row * H_I * D_I + e];
    __syncthreads();
    const int8_t* kb = k_idx + static_cast<int64_t>(b) * Tk * D_I;
    for (int s = threadIdx.x; s < n; s += TOPK_NT) {
      const int* kr = reinterpret_cast<const int*>(kb + static_cast<int64_t>(s) * D_I);
      int acc = 0;
#pragma unroll
      for (int h = 0; h < H_I; ++h) {
        const int* qh = reinterpret_cast<const int*>(qrow + h * D_I);
        int dot = 0;
#pragma unroll
        for (int c = 0; c < D_I / 4; ++c) dot = __builtin_amdgcn_sdot4(qh[c], kr[c], dot, false);
        acc += static_cast<int>(w[h]) * max(dot, 0);
      }
      S[s] = acc;
    }
    __syncthreads();
    int32_t* out = idx + (static_cast<int64_t>(b) * out_tq + i) * K;
    if (!(n <= kSel2MaxN && select_row_2pass(S, n, K, out, nullptr, sm.mask2))) {
      __syncthreads();
      select_row(S, n, K, out, nullptr, sm.radix);
    }
    __syncthreads();  // the next row reuses qrow, S and the LDS
  }
}

// ------------------------------------------------------------------ host side

// Dynamic LDS of the per-row selection: the bit map of the history.
static size_t sel_rows_lds(int Tk) { return static_cast<size_t>((Tk + 31) / 32) * sizeof(uint32_t); }

bool sel_supported(const Geom& g, int64_t wsb, int64_t wsq) {
  // each wave sweeps its rows' whole history: only calls with many rows fill
  // the chip (fewer rows take the materialised path, parallel over positions)
  return g.block <= 1 && wsb == 0 && wsq == 0 && (g.d_I == 64 || g.d_I == 128) &&
         g.H_I <= 8 && g.H_I * g.d_I <= 512 && g.Tk > kWaveTopkMax && g.Tk <= kSelMaxTk &&
         static_cast<int64_t>(g.B) * g.Tq >= kSelMinRows && g.K <= 4096 &&
         sel_rows_lds(g.Tk) <= 32768;
}

SelLayout sel_layout(const Geom& g) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  SelLayout L{};
  L.cap = sel_cap(g.K);
  const size_t rows = static_cast<size_t>(g.B) * g.Tq;
  L.srow = (static_cast<int64_t>(g.Tk) + 3) / 4 * 4;
  size_t o = 0;
  L.cand = o;  o += al(rows * L.cap * sizeof(int2));
  L.cnt = o;   o += al(rows * sizeof(uint32_t));
  L.meta = o;  o += al(rows * sizeof(SelMeta));
  L.nfb = o;   o += al(sizeof(uint32_t));
  L.fbrows = o; o += al(rows * sizeof(int32_t));
  L.scratch = o; o += al(static_cast<size_t>(SEL_FB_GRID) * L.srow * sizeof(int32_t));
  L.total = o;
  return L;
}

template <int H_I, int D_I>
static hipError_t launch_sel_hd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                const int8_t* w, int32_t* idx, int out_tq, void* ws,
                                hipStream_t st) {
  const SelLayout L = sel_layout(g);
  char* base = static_cast<char*>(ws);
  int2* cand = reinterpret_cast<int2*>(base + L.cand);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(base + L.cnt);
  SelMeta* meta = reinterpret_cast<SelMeta*>(base + L.meta);
  uint32_t* nfb = reinterpret_cast<uint32_t*>(base + L.nfb);
  int32_t* fbrows = reinterpret_cast<int32_t*>(base + L.fbrows);
  int32_t* scratch = reinterpret_cast<int32_t*>(base + L.scratch);
  {
    KernelTimer timer(LCI_KERNEL_SEL_SCAN, st);
    hipLaunchKernelGGL((sel_scan_kernel<H_I, D_I>), dim3((g.Tq + 15) / 16, g.B), dim3(64), 0,
                       st, g.Tq, g.Tk, g.K, L.cap, g.q_offset, g.kv_len, q_idx, k_idx, w, cand,
                       cnt, meta, nfb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sel_rows_lds(g.Tk);
  {
    KernelTimer timer(LCI_KERNEL_SEL_ROWS, st);
    hipLaunchKernelGGL(sel_rows_kernel, dim3(g.Tq, g.B), dim3(SEL_NT), lds, st, g.Tq, g.Tk, g.K,
                       L.cap, g.q_offset, g.kv_len, cand, cnt, meta, idx, out_tq, nfb, fbrows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_SEL_FALLBACK, st);
    hipLaunchKernelGGL((sel_fallback_kernel<H_I, D_I>), dim3(SEL_FB_GRID), dim3(TOPK_NT), 0, st,
                       g.Tq, g.Tk, g.K, g.q_offset, g.kv_len, q_idx, k_idx, w, nfb, fbrows,
                       scratch, L.srow, idx, out_tq);
  }
  return hipGetLastError();
}

template <int H_I>
static hipError_t launch_sel_h(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                               const int8_t* w, int32_t* idx, int out_tq, void* ws,
                               hipStream_t st) {
  if constexpr (H_I * 64 <= 512) {
    if (g.d_I == 64) return launch_sel_hd<H_I, 64>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
  }
  if constexpr (H_I * 128 <= 512) {
    if (g.d_I == 128) return launch_sel_hd<H_I, 128>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sel(const Geom& g, const int8_t* q_idx, const int8_t* k_idx, const int8_t* w,
                      int32_t* idx, int out_tq, void* ws, hipStream_t st) {
  switch (g.H_I) {
    case 1: return launch_sel_h<1>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
    case 2: return launch_sel_h<2>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
    case 4: return launch_sel_h<4>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
    case 8: return launch_sel_h<8>(g, q_idx, k_idx, w, idx, out_tq, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
