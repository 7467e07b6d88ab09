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
//   sel_scan_kernel   one workgroup of four waves per 16 consecutive query rows
//                     of a sequence, each wave taking every fourth step of each
//                     sweep. For rows with more than `cap` candidates, two
//                     sampled passes set a per-row threshold t: every 32nd
//                     position fills a 64-bin histogram (sign and bit length of
//                     the score), which names the coarse bin holding the
//                     estimated K-th score; every 8th position then fills 256
//                     linear sub-bins of that bin. t is the lowest score of the
//                     sub-bin where the count of sampled scores at or above it
//                     first reaches K*f + 4*sqrt(K*f) + 2 (f: the sampled
//                     fraction of the row), so that about K + 4 standard
//                     deviations of the row's positions score at least t. One
//                     full pass then scores every causal position (int8 MFMA
//                     16x16x64, positions as MFMA rows, one indexer head per
//                     MFMA, as in the scoring kernel) and appends each (score,
//                     position) with score >= t to the scanning lane's part of
//                     the row's candidate list (16 parts of cap/16 entries, one
//                     per wave and lane of the row, each counted in a
//                     register). Rows with few positions may list every one.
//   sel_rows_kernel   one workgroup per row. When the list holds every position
//                     whose score is >= t and at least K of them (no part past
//                     its capacity, K or more in all), the row's Top-K is the
//                     Top-K of the list: a histogram of the listed keys names
//                     the bin of the K-th key under (score desc, position asc),
//                     keys above it are kept and the bin's own entries ranked by
//                     direct count in LDS, the kept positions set in an LDS bit
//                     map of the row (ties at the K-th score: the lowest
//                     positions), and an ordered compaction of the map writes
//                     the ascending index row. Any other count (the threshold
//                     missed: too few or too many scores >= t) puts the row on
//                     the fallback list.
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
// Waves of a scan workgroup, each taking every SEL_NW-th step of every sweep,
// and parts of a row's candidate list (one per wave and lane of the row).
constexpr int SEL_NW = 4;
constexpr int SEL_PARTS = 4 * SEL_NW;

// Candidate list capacity for K: the expected count plus seven standard
// deviations of the sampled estimate, and a margin for the sub-bin width.
int sel_cap(int K) {
  const double kf = static_cast<double>(K);
  const double expect = kf + 4.0 * sqrt(kf * SEL_SS2) + 2.0 * SEL_SS2;
  const double c = expect + 7.0 * sqrt(SEL_SS2 * expect) + 64.0;
  return (static_cast<int>(c) + 255) / 256 * 256;
}

// Capacity of each of the SEL_PARTS parts of a list: an even share of the
// list's capacity plus a quarter for the parts' own spread (a row listing
// cap candidates fills its fullest part past the even share: on Prefill 64K
// one row in about 800 overflowed the even share), a multiple of 16.
int sel_part_cap(int K) {
  const int share = sel_cap(K) / SEL_PARTS;
  return (share + share / 4 + 15) / 16 * 16;
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
  uint32_t hist[16][SEL_FB / 2];   // coarse (first SEL_CB / 2 words of a row), then fine
  uint32_t above[16];              // fine-sampled scores above the coarse bin, per row
  uint32_t kmin[16], kmax[16];     // range of the fine-sampled keys, per row
  int32_t thr[16];                 // threshold of each row
  int32_t cb[16];                  // coarse bin of each row
  uint32_t hb[16];                 // key at the bottom of the candidates' histogram
  int32_t hsh[16];                 // its bin width, log2
};

// Per-row summary the scan leaves for the row kernel: the range of the
// sampled keys from the threshold up, as 256 histogram bins of width 2^hsh
// over keys from hb up (keys below hb in bin 0, keys past the top in bin 255).
struct SelMeta {
  uint32_t hb;
  int32_t hsh;
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

// One workgroup of SEL_NW waves: 16 query rows rb*16 .. rb*16+15 of sequence b
// (a set's rows). Wave v takes the steps s = v, v + SEL_NW, ... of each sweep,
// so the waves see the same mix of positions and finish together, and the
// many workgroups, longest rows first, keep every SIMD busy to the end.
// q_idx [B, Tq, H_I, D_I] (this set's heads), k_idx [B, Tk, D_I], w [H_I]
// shared by every row. cand [B*Tq][SEL_PARTS][cap/SEL_PARTS] int2 (score,
// position), cnt [B*Tq][SEL_PARTS] (each part's true count, possibly above its
// capacity), meta [B*Tq]. nfb: the fallback list's length, zeroed here for the
// row kernel that follows.
template <int H_I, int D_I>
__global__ __launch_bounds__(64 * SEL_NW, 4) void sel_scan_kernel(
    int Tq, int Tk, int K, int cap, int capp, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const int8_t* __restrict__ w, int2* __restrict__ cand,
    uint32_t* __restrict__ cnt, SelMeta* __restrict__ meta, uint32_t* __restrict__ nfb) {
  constexpr int NCH = D_I / 64;  // 64-deep MFMA steps over d_I
  constexpr int U = 2;           // 16-position tiles per step
  __shared__ SelScanLds sm;
  const int lrow = SEL_PARTS * capp;  // entries of a row's list
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrb = (Tq + 15) / 16;
  const int rb = nrb - 1 - static_cast<int>(blockIdx.x);  // longest rows first
  const int b = blockIdx.y;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *nfb = 0u;
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
  if (tid < 16) {
    sm.thr[r] = INT32_MIN;
    sm.above[r] = 0u;
    sm.kmin[r] = 0xffffffffu;
    sm.kmax[r] = 0u;
  }
  for (int j = tid; j < 16 * (SEL_CB / 2); j += 64 * SEL_NW)
    sm.hist[j / (SEL_CB / 2)][j % (SEL_CB / 2)] = 0u;
  // every wave holds the same rows: these are uniform over the workgroup
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
  // f(position, score) over this lane's causal positions of this wave's steps
  // of a strided sweep
  auto sweep = [&](int stride, int last, auto&& f) {
    const int span = 32 * stride;  // positions covered by one step
    v4i ka[U][NCH];
    load_keys(wv * span, stride, ka);
    for (int pos0 = wv * span; pos0 <= last; pos0 += SEL_NW * span) {
      v4i kn[U][NCH];
      load_keys(pos0 + SEL_NW * span, stride, kn);
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
  if (tid < 16 && listed) {
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
  for (int j = tid; j < 16 * (SEL_FB / 2); j += 64 * SEL_NW)
    sm.hist[j / (SEL_FB / 2)][j % (SEL_FB / 2)] = 0u;
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
  // the row's lanes of every wave combine their counts and ranges
  above += __shfl_xor(above, 16, 64);
  above += __shfl_xor(above, 32, 64);
  kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), 16, 64)));
  kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), 32, 64)));
  kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), 16, 64)));
  kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), 32, 64)));
  if (lane < 16 && listed) {
    atomicAdd(&sm.above[r], above);
    atomicMin(&sm.kmin[r], kmin);
    atomicMax(&sm.kmax[r], kmax);
  }
  __syncthreads();
  if (tid < 16 && listed) {
    const int ns = p / SEL_SS2 + 1;
    const uint32_t tgt = static_cast<uint32_t>(sel_target(K, ns, n));
    const uint32_t ab = sm.above[r];
    uint32_t t;
    if (ab >= tgt) {
      // the coarse sample put the bin too low: everything above it
      t = uhi + 1u;
    } else {
      uint32_t cum = ab;
      t = ulo;  // the whole bin when even it falls short
      for (int fb = SEL_FB - 1; fb >= 0; --fb) {
        cum += (sm.hist[r][fb >> 1] >> (16 * (fb & 1))) & 0xffffu;
        if (cum >= tgt) {
          t = ulo + (static_cast<uint32_t>(fb) << fsh);
          break;
        }
      }
      // too few samples to reach the target: a row of at most cap positions
      // lists all of them; a longer one keeps the whole coarse bin (exact
      // either way: a list short of K sends the row to the fallback)
      if (cum < tgt && n <= cap) t = 0u;
    }
    sm.thr[r] = key_score(t);
    // the candidates' histogram spans the sampled keys from the threshold up
    const uint32_t hb = max(t, sm.kmin[r]);
    const uint32_t km = sm.kmax[r];
    sm.hb[r] = hb;
    sm.hsh[r] = km > hb ? sel_fshift(hb, km) : 0;
  }
  __syncthreads();

  // 3. full pass: every causal position at or above the row's threshold goes
  // to its own part of the row's list (part 4*v + g4 for lane g4 of the row in
  // wave v, which sees positions 16u + 4*g4 + e of its 32-position steps), of
  // capp entries, counted in a register: no slot is shared. Rows that keep
  // every position list nothing: no score reaches INT32_MAX (|S| <= 2^30 with
  // H_I*d_I <= 512).
  const int32_t thr = listed ? sm.thr[r] : INT32_MAX;
  const int plist = listed ? p : -1;  // causal limit of the listed positions
  // steps wholly at or below every listed row's limit need no position test
  int pmin = listed ? p : INT32_MAX;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) pmin = min(pmin, __shfl_xor(pmin, off, 64));
  pmin = __builtin_amdgcn_readfirstlane(pmin);
  // The workgroup's rows' lists as one buffer: every step issues the same
  // eight stores, a position that is no candidate with an offset past the
  // buffer, which the range check drops. The code is then straight-line, so
  // the wait for a step's keys leaves the younger stores in flight.
  const int wrows = min(16, Tq - rb * 16);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(cand + (static_cast<int64_t>(b) * Tq + rb * 16) * lrow), 0,
      wrows * lrow * static_cast<int>(sizeof(int2)), kBufferFlags);
  const int lbase = (r * SEL_PARTS + 4 * wv + g4) * capp * static_cast<int>(sizeof(int2));
  const int llast = lbase + (capp - 1) * static_cast<int>(sizeof(int2));
  constexpr int kDrop = INT32_MIN;  // byte offset 2^31, past the buffer
  // byte offset of this part's next entry (past llast: the part is full, and
  // further entries overwrite its last one, as the row is redone anyway)
  int noff = lbase;
  // the previous step's scores ps, at positions pb + 16u + e (pb = its first
  // position + 4*g4), candidates when >= thr and at or below plim
  auto put = [&](const v4i (&sc4)[U], int pb, int plim) {
#pragma unroll
    for (int k = 0; k < 4 * U; ++k) {
      const int32_t sc = sc4[k >> 2][k & 3];
      const int pos = pb + 16 * (k >> 2) + (k & 3);
      const bool c = (sc >= thr) & (pos <= plim);
      __builtin_amdgcn_raw_buffer_store_b64(v2i{sc, pos}, crs, c ? min(noff, llast) : kDrop, 0, 0);
      noff += c ? static_cast<int>(sizeof(int2)) : 0;
    }
  };
  // one step: the previous step's candidates, the next step's key loads, this
  // step's scores; the two key buffers alternate, so no register with a load
  // in flight is ever copied. The first step's "previous" positions lie past
  // every row's limit, so it stores nothing.
  constexpr int kStep = 32 * SEL_NW;  // positions between a wave's steps
  v4i ps[U] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
  int ppos = INT32_MAX - 64;  // first position of the previous step
  int pplim = -1;             // position limit of the previous step
  auto step = [&](int pos0, const v4i (&kc)[U][NCH], v4i (&kx)[U][NCH]) {
    put(ps, ppos + 4 * g4, pplim);
    __builtin_amdgcn_sched_barrier(0);
    load_keys(pos0 + kStep, 1, kx);
    __builtin_amdgcn_sched_barrier(0);
    score(kc, ps);
    ppos = pos0;
    // steps wholly at or below every listed row's limit need no position test
    pplim = pos0 + 31 <= pmin ? INT32_MAX : plist;
  };
  v4i ka[U][NCH], kb[U][NCH];
  int pos0 = 32 * wv;
  load_keys(pos0, 1, ka);
  for (; pos0 + kStep <= pmax; pos0 += 2 * kStep) {
    step(pos0, ka, kb);
    step(pos0 + kStep, kb, ka);
  }
  if (pos0 <= pmax) step(pos0, ka, kb);
  put(ps, ppos + 4 * g4, pplim);  // the last step's (if any ran)
  const uint32_t nlist = static_cast<uint32_t>(noff - lbase) / sizeof(int2);
  if (i < Tq) cnt[(static_cast<int64_t>(b) * Tq + i) * SEL_PARTS + 4 * wv + g4] = nlist;
  if (tid < 16 && i < Tq) meta[static_cast<int64_t>(b) * Tq + i] = SelMeta{sm.hb[r], sm.hsh[r]};
}

constexpr int SEL_SMALL = 1024;  // list entries in the K-th score's bin resolved in LDS
// Entries per thread of the row kernel for the largest part capacity
// (K = 4096: parts of 512 entries, 16 threads each).
constexpr int kSelRowsMaxE = 32;

// One workgroup per (row, sequence). The list of row (b, i) is SEL_PARTS parts
// of cap/SEL_PARTS entries (one per scanning wave and lane), with their counts
// (all counted, at most cap/SEL_PARTS stored each) and the row's histogram
// range meta. The kernel histograms the listed keys, finds the bin holding the
// K-th largest; the row's Top-K is every listed key in a higher bin plus the
// best of the entries in that bin (ranked by direct count), set in an LDS bit
// map of the row and compacted in position order. idx rows at
// idx + (b*out_tq + i)*K. Rows whose list cannot give their Top-K (fewer than
// K entries, a part past its capacity, or more than SEL_SMALL entries in the
// K-th bin) go to the fallback list.
// E: entries of a part each thread holds in registers between the two passes
// (at least capp / 16).
template <int E>
__global__ __launch_bounds__(SEL_NT) void sel_rows_kernel(
    int Tq, int Tk, int K, int capp, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int2* __restrict__ cand,
    const uint32_t* __restrict__ cnt, const SelMeta* __restrict__ meta,
    int32_t* __restrict__ idx, int out_tq, uint32_t* __restrict__ nfb,
    int32_t* __restrict__ fb_rows, DenseMasks dm) {
  extern __shared__ __align__(16) uint32_t keep[];  // ceil(Tk/32) words
  __shared__ int2 small[SEL_SMALL];
  __shared__ uint32_t hist[SEL_FB];
  __shared__ uint32_t pc[SEL_PARTS];
  __shared__ uint32_t scratch[SEL_NT / 64 + 2];
  __shared__ uint32_t nsmall, kbin, above;
  static_assert(SEL_NT == SEL_FB, "one thread per histogram bin");
  static_assert(SEL_NT == 16 * SEL_PARTS, "16 threads per part of a list");

  const int t = threadIdx.x;
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int kvl0 = kv_len[b];
  const int kvl = kvl0 <= Tk ? kvl0 : 0;
  const int64_t p64 = static_cast<int64_t>(q_offset[b]) + i;
  const bool rok = p64 >= 0 && p64 < kvl;
  const int n = rok ? static_cast<int>(p64) + 1 : 0;
  const int64_t orow = static_cast<int64_t>(b) * out_tq + i;
  int32_t* out = idx + orow * K;
  // the tile path's row flag and mask (dm.mask set): rows with p + 1 <= lim
  // take the tile kernel, under a bit mask of their kept positions; an
  // invalid row (n = 0) is the tile kernel's empty row
  const bool tile = dm.mask != nullptr && n <= dm.lim;
  if (dm.mask != nullptr && !tile && t == 0) dm.flag[orow] = kRowGather;
  if (n <= K) {  // every position kept, or an invalid row
    for (int j = t; j < K; j += SEL_NT) out[j] = j < n ? j : -1;
    if (tile) {
      uint32_t* mrow = dm.mask + orow * dm.Wm;
      for (int wd = t; wd < dm.Wm; wd += SEL_NT) {
        const int lo = 32 * wd;
        mrow[wd] = n >= lo + 32 ? 0xffffffffu : (n > lo ? (1u << (n - lo)) - 1u : 0u);
      }
      if (t == 0) dm.flag[orow] = rok ? kRowAll : kRowEmpty;
    }
    return;
  }
  const int64_t row = static_cast<int64_t>(b) * Tq + i;
  if (t < SEL_PARTS) pc[t] = cnt[row * SEL_PARTS + t];
  hist[t] = 0u;
  __syncthreads();
  uint32_t listed = 0, cmax = 0;
#pragma unroll
  for (int g = 0; g < SEL_PARTS; ++g) {
    listed += pc[g];
    cmax = max(cmax, pc[g]);
  }
  if (cmax > static_cast<uint32_t>(capp) || listed < static_cast<uint32_t>(K)) {
    // the threshold missed (uniform: every thread read the same counts)
    if (t == 0) fb_rows[atomicAdd(nfb, 1u)] = static_cast<int32_t>(row);
    return;
  }
  const SelMeta mt = meta[row];
  // 16 threads per part: thread t reads entries t % 16, t % 16 + 16, ... of
  // part t / 16
  const int2* cpart = cand + (row * SEL_PARTS + (t >> 4)) * capp;
  const int npart = static_cast<int>(pc[t >> 4]);
  // the thread's entries, all loads in flight together; kept in registers for
  // both passes
  int2 ent[E];
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int j = (t & 15) + 16 * q;
    ent[q] = j < npart ? cpart[j] : make_int2(0, 0);
  }
  // 1. the listed keys' histogram; the bin of the K-th largest
#pragma unroll
  for (int q = 0; q < E; ++q)
    if ((t & 15) + 16 * q < npart)
      atomicAdd(&hist[sel_hbin(score_key(ent[q].x), mt.hb, mt.hsh)], 1u);
  __syncthreads();
  {
    // thread t takes bin 255 - t: the count above it is the scan of the bins before
    const uint32_t h = hist[SEL_FB - 1 - t];
    uint32_t htot;
    const uint32_t ab = block_excl_scan(h, scratch, &htot);
    if (ab < static_cast<uint32_t>(K) && static_cast<uint32_t>(K) <= ab + h) {
      kbin = static_cast<uint32_t>(SEL_FB - 1 - t);
      above = ab;
    }
  }
  const int nw = (n + 31) / 32;
  for (int j = t; j < nw; j += SEL_NT) keep[j] = 0u;
  if (t == 0) nsmall = 0u;
  __syncthreads();
  // 2. keys above the K-th bin are kept; the bin's own entries are gathered
  const uint32_t kb = kbin;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    if ((t & 15) + 16 * q >= npart) break;
    const int2 e = ent[q];
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
  const uint32_t need = static_cast<uint32_t>(K) - above;
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
  if (tile) {  // the kept map is final: it is the row's mask (zero past p)
    uint32_t* mrow = dm.mask + orow * dm.Wm;
    for (int wd = t; wd < dm.Wm; wd += SEL_NT) mrow[wd] = wd < nw ? keep[wd] : 0u;
    if (t == 0) dm.flag[orow] = kRowMasked;
  }
  // ordered compaction: thread t takes words [t*wpt, (t+1)*wpt)
  const int wpt = (nw + SEL_NT - 1) / SEL_NT;
  const int w0 = t * wpt;
  uint32_t mine = 0;
  for (int j = 0; j < wpt; ++j)
    if (w0 + j < nw) mine += static_cast<uint32_t>(__popc(keep[w0 + j]));
  uint32_t tot;
  uint32_t slot = block_excl_scan(mine, scratch, &tot);
  // the index row is built in LDS (the bin entries' array, free after the
  // ranking) and stored by consecutive lanes: each thread's own run of slots
  // written straight to memory would touch a separate cache line per lane
  int32_t* const ostage = reinterpret_cast<int32_t*>(small);
  const bool staged = K <= 2 * SEL_SMALL;  // uniform
  for (int j = 0; j < wpt; ++j) {
    const int wj = w0 + j;
    if (wj >= nw) break;
    uint32_t word = keep[wj];
    while (word != 0u) {
      const int bit = __ffs(static_cast<int>(word)) - 1;
      word &= word - 1u;
      if (slot < static_cast<uint32_t>(K)) {
        if (staged) ostage[slot] = 32 * wj + bit;
        else out[slot] = 32 * wj + bit;
      }
      ++slot;
    }
  }
  if (staged) {
    __syncthreads();
    const int nout = static_cast<int>(min(tot, static_cast<uint32_t>(K)));
    for (int j = t; j < nout; j += SEL_NT) out[j] = ostage[j];
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
    int32_t* __restrict__ scratch, int64_t srow_stride, int32_t* __restrict__ idx, int out_tq,
    DenseMasks dm) {
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
    const int64_t orow = static_cast<int64_t>(b) * out_tq + i;
    int32_t* out = idx + orow * K;
    if (!(n <= kSel2MaxN && select_row_2pass(S, n, K, out, nullptr, sm.mask2))) {
      __syncthreads();
      select_row(S, n, K, out, nullptr, sm.radix);
    }
    __syncthreads();  // the next row reuses qrow, S and the LDS
    if (dm.mask != nullptr && n <= dm.lim) {
      // the tile path's mask from the finished index row (rare rows: global
      // atomics on the zeroed mask row)
      uint32_t* mrow = dm.mask + orow * dm.Wm;
      for (int wd = threadIdx.x; wd < dm.Wm; wd += TOPK_NT) mrow[wd] = 0u;
      __threadfence();
      __syncthreads();
      for (int j = threadIdx.x; j < K; j += TOPK_NT) {
        const int32_t sp = out[j];
        if (sp >= 0) atomicOr(&mrow[sp >> 5], 1u << (sp & 31));
      }
      if (threadIdx.x == 0) dm.flag[orow] = kRowMasked;
    }
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
         sel_part_cap(g.K) <= 16 * kSelRowsMaxE && sel_rows_lds(g.Tk) <= 32768;
}

SelLayout sel_layout(const Geom& g) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  SelLayout L{};
  L.cap = sel_cap(g.K);
  const size_t rows = static_cast<size_t>(g.B) * g.Tq;
  L.srow = (static_cast<int64_t>(g.Tk) + 3) / 4 * 4;
  size_t o = 0;
  L.capp = sel_part_cap(g.K);
  L.cand = o;  o += al(rows * SEL_PARTS * L.capp * sizeof(int2));
  L.cnt = o;   o += al(rows * SEL_PARTS * sizeof(uint32_t));  // one count per part of a list
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
                                const DenseMasks& dm, hipStream_t st) {
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
    hipLaunchKernelGGL((sel_scan_kernel<H_I, D_I>), dim3((g.Tq + 15) / 16, g.B), dim3(64 * SEL_NW), 0,
                       st, g.Tq, g.Tk, g.K, L.cap, L.capp, g.q_offset, g.kv_len, q_idx, k_idx, w, cand,
                       cnt, meta, nfb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sel_rows_lds(g.Tk);
  {
    KernelTimer timer(LCI_KERNEL_SEL_ROWS, st);
    const int e = (L.capp + 15) / 16;  // entries per thread
    const dim3 grid(g.Tq, g.B);
    if (e <= 8)
      hipLaunchKernelGGL(sel_rows_kernel<8>, grid, dim3(SEL_NT), lds, st, g.Tq, g.Tk, g.K, L.capp,
                         g.q_offset, g.kv_len, cand, cnt, meta, idx, out_tq, nfb, fbrows, dm);
    else if (e <= 20)
      hipLaunchKernelGGL(sel_rows_kernel<20>, grid, dim3(SEL_NT), lds, st, g.Tq, g.Tk, g.K, L.capp,
                         g.q_offset, g.kv_len, cand, cnt, meta, idx, out_tq, nfb, fbrows, dm);
    else
      hipLaunchKernelGGL(sel_rows_kernel<kSelRowsMaxE>, grid, dim3(SEL_NT), lds, st, g.Tq, g.Tk,
                         g.K, L.capp, g.q_offset, g.kv_len, cand, cnt, meta, idx, out_tq, nfb,
                         fbrows, dm);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_SEL_FALLBACK, st);
    hipLaunchKernelGGL((sel_fallback_kernel<H_I, D_I>), dim3(SEL_FB_GRID), dim3(TOPK_NT), 0, st,
                       g.Tq, g.Tk, g.K, g.q_offset, g.kv_len, q_idx, k_idx, w, nfb, fbrows,
                       scratch, L.srow, idx, out_tq, dm);
  }
  return hipGetLastError();
}

template <int H_I>
static hipError_t launch_sel_h(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                               const int8_t* w, int32_t* idx, int out_tq, void* ws,
                               const DenseMasks& dm, hipStream_t st) {
  if constexpr (H_I * 64 <= 512) {
    if (g.d_I == 64) return launch_sel_hd<H_I, 64>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
  }
  if constexpr (H_I * 128 <= 512) {
    if (g.d_I == 128) return launch_sel_hd<H_I, 128>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sel(const Geom& g, const int8_t* q_idx, const int8_t* k_idx, const int8_t* w,
                      int32_t* idx, int out_tq, void* ws, const DenseMasks* masks,
                      hipStream_t st) {
  const DenseMasks dm = masks ? *masks : DenseMasks{};
  switch (g.H_I) {
    case 1: return launch_sel_h<1>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
    case 2: return launch_sel_h<2>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
    case 4: return launch_sel_h<4>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
    case 8: return launch_sel_h<8>(g, q_idx, k_idx, w, idx, out_tq, ws, dm, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
