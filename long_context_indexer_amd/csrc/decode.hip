// Fused decode (one query row per sequence over a long history) on gfx950.
//
// "How Fine-Grained Sparse Attention Reshapes Long-Context Architecture",
// section "Engineering Practices from an Open-Weight Perspective": per-step
// decode work decouples from context length once only K positions are read.
// The indexer still reads the whole history's indexer keys ("Hybrid Sparse
// Attention for Long-Context LLMs", section "Indexer + Top-K ...", step 1), so
// the decode step is bound by HBM: L*d_I bytes of indexer keys plus K rows of
// keys and values per query.
//
// With one query per sequence the parallelism comes from splitting the history:
//   dec_score    (chunks x B) int8-MFMA scores of 4096 positions per workgroup,
//                written to workspace, and the chunk's 2048-bin histogram over a
//                monotone float-like binning of the int32 score (exponent + 5
//                mantissa bits, both signs), built in LDS and stored whole;
//   dec_thresh   (B) sums the chunk histograms, then finds the bin b* holding
//                the K-th largest score and the count of positions above it;
//   dec_cand     (chunks x B) every workgroup counts its positions above b*
//                and writes the (score, position) pairs inside b* to its own
//                slice of the sequence's candidate list;
//   dec_resolve  (B) gathers the candidate slices, selects the exact K-th score v* and
//                the position cut s* that keeps the lowest-position ties, then
//                turns per-chunk counts into output offsets (a candidate list
//                that overflows its capacity falls back to the exact one-workgroup
//                selection over the whole row);
//   dec_compact  (chunks x B) ordered compaction: keeps S > v* or (S == v* and
//                s <= s*), writing ascending positions at the chunk's offset.
// The selected set is exactly the K best positions under (score desc, position
// asc): every position in a higher bin is kept, every position in a lower bin
// dropped, and the split inside b* is resolved exactly.
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"
#include "decode.h"
#include "select_row.h"

namespace lci {

constexpr int DEC_BINS = 2048;
constexpr int DEC_CBINS = DEC_BINS / 32;  // coarse bins: fine bin / 32 (sign and exponent)
constexpr int DEC_NT = 256;

struct DecRow {
  int valid;
  int64_t n;  // candidates 0..n-1
};

__device__ __forceinline__ DecRow dec_row(int Tk, const int32_t* q_offset, const int32_t* kv_len,
                                          int b) {
  const int kvl = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]);
  DecRow r;
  r.valid = kvl <= Tk && p >= 0 && p < kvl;
  r.n = r.valid ? p + 1 : 0;
  return r;
}

// Sum of p[c * stride] over c = c0, c0 + step, ... < nc, eight loads in flight.
__device__ __forceinline__ uint32_t strided_sum(const uint32_t* __restrict__ p, int c0, int nc,
                                                int step, int64_t stride) {
  uint32_t acc = 0;
  int c = c0;
  for (; c + 7 * step < nc; c += 8 * step) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[static_cast<int64_t>(c + u * step) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; c < nc; c += step) acc += p[static_cast<int64_t>(c) * stride];
  return acc;
}

// One workgroup per sequence: the bin b* holding the K-th largest score and
// the count of positions in higher bins, read by the candidate and resolve
// kernels. Two levels over the stored chunk histograms: the 64 coarse bins
// (sign and exponent) summed over the chunks give the coarse bin holding the
// K-th score, then only its 32 fine bins are summed (96 words per chunk read
// instead of 2048).
__global__ __launch_bounds__(DEC_NT) void dec_thresh_kernel(
    int Tk, int K, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const uint32_t* __restrict__ fhist, const uint32_t* __restrict__ chist, int nchunks,
    uint32_t* __restrict__ bsel) {
  __shared__ uint32_t red[DEC_NT];
  __shared__ uint32_t res[2];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const DecRow rw = dec_row(Tk, q_offset, kv_len, b);
  if (rw.n <= K) return;
  const int nc = static_cast<int>((rw.n + kDecChunk - 1) / kDecChunk);  // chunks with positions
  const uint32_t uK = static_cast<uint32_t>(K);
  // coarse: thread t sums coarse bin t % 64 over chunks t / 64, t / 64 + 4, ...
  red[t] = strided_sum(chist + static_cast<int64_t>(b) * nchunks * DEC_CBINS + lane, t >> 6, nc,
                       DEC_NT / 64, DEC_CBINS);
  __syncthreads();
  if (t < 64) {
    // lane l takes coarse bin 63 - l: the inclusive scan runs from the top bin down
    const int cb = DEC_CBINS - 1 - lane;
    uint32_t v = 0;
#pragma unroll
    for (int g = 0; g < DEC_NT / 64; ++g) v += red[g * 64 + cb];
    const uint32_t incl = wave_incl_scan(v);
    if (incl - v < uK && uK <= incl) {
      res[0] = static_cast<uint32_t>(cb);
      res[1] = incl - v;
    }
  }
  __syncthreads();
  const int cbin = static_cast<int>(res[0]);
  const uint32_t abovec = res[1];
  // fine: thread t sums fine bin 32 cbin + t % 32 over chunks t / 32, t / 32 + 8, ...
  red[t] = strided_sum(fhist + static_cast<int64_t>(b) * nchunks * DEC_BINS + 32 * cbin + (t & 31),
                       t >> 5, nc, DEC_NT / 32, DEC_BINS);
  __syncthreads();
  if (t < 64) {
    const int f = 31 - lane;  // lanes 32..63 carry nothing
    uint32_t v = 0;
    if (lane < 32)
#pragma unroll
      for (int g = 0; g < DEC_NT / 32; ++g) v += red[g * 32 + f];
    const uint32_t incl = wave_incl_scan(v);
    const uint32_t krem = uK - abovec;
    if (lane < 32 && incl - v < krem && krem <= incl) {
      bsel[2 * b] = static_cast<uint32_t>(32 * cbin + f);
      bsel[2 * b + 1] = abovec + incl - v;
    }
  }
}

// Scoring uses v_mfma_i32_16x16x64_i8 with the history positions as the 16
// columns: lane l loads 16 bytes at offset 16*(l/16) of position l%16, so one
// load instruction covers 16 consecutive 64-byte indexer keys (1 KiB, fully
// coalesced) for d_I = 64. MFMA rows are the H_I indexer heads (at most 16) of
// the single query; lane l holds heads 4*(l/16)+i of position l%16, so the
// weighted ReLU sum is completed across the lane groups with two xor-shuffles.
// Loads are unconditional (positions past the end are clamped to a valid row
// and their scores dropped) and double-buffered in two named register sets, so
// the compiler can keep the next step's loads in flight during this step's
// MFMAs; scores are staged in LDS and written out, with the histogram, at the end.
template <int H_I, int D_I>
__global__ __launch_bounds__(DEC_NT) void dec_score_kernel(
    int Tk, int K, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx,
    const int8_t* __restrict__ w, int64_t wsb, int32_t* __restrict__ S,
    uint32_t* __restrict__ fhist, uint32_t* __restrict__ chist) {
  constexpr int NCH = D_I / 64 > 0 ? D_I / 64 : 1;  // 64-deep MFMA steps
  constexpr int U = 4;                             // 16-position tiles per step
  constexpr int STEP = 16 * U;
  __shared__ uint32_t lh[DEC_BINS];
  __shared__ int32_t sl[kDecChunk];
  const int b = blockIdx.y;
  const DecRow rw = dec_row(Tk, q_offset, kv_len, b);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDecChunk;
  if (rw.n <= K || base >= rw.n) return;  // nothing to select for this chunk
  for (int j = threadIdx.x; j < DEC_BINS; j += DEC_NT) lh[j] = 0u;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int grp = lane >> 4;
  // A operand: lane l supplies row (head) l%16, bytes 16*(l/16) of each 64-deep step;
  // for d_I = 32 the upper 32 bytes of the step are zero in A (B may hold anything)
  v4i a[NCH];
  {
    const int hh = lane & 15;
    const bool ok = hh < H_I && 16 * grp < D_I;
    const int8_t* src = q_idx + (static_cast<int64_t>(b) * H_I + (ok ? hh : 0)) * D_I + 16 * grp;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v4i z = {0, 0, 0, 0};
      a[c] = ok ? *reinterpret_cast<const v4i*>(src + 64 * c) : z;
    }
  }
  int wh[4];  // weights of the heads this lane holds: 4*grp + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * grp + i;
    wh[i] = hh < H_I ? static_cast<int>(w[b * wsb + hh]) : 0;
  }

  const int64_t nend = min(base + kDecChunk, rw.n);
  const int64_t wbeg = base + wv * (kDecChunk / 4);
  const int64_t wend = min(wbeg + kDecChunk / 4, nend);
  const int8_t* kb = k_idx + static_cast<int64_t>(b) * Tk * D_I + 16 * (grp % (D_I / 16 < 4 ? D_I / 16 : 4));

  auto load = [&](int64_t kt, v4i (&dst)[U][NCH]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = min(kt + 16 * u + (lane & 15), wend - 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) dst[u][c] = *reinterpret_cast<const v4i*>(kb + key * D_I + 64 * c);
    }
  };
  auto score = [&](int64_t kt, const v4i (&src)[U][NCH]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[c], src[u][c], acc, 0, 0, 0);
      int s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) s += __mul24(wh[i], max(acc[i], 0));
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      const int64_t key = kt + 16 * u + (lane & 15);
      if (lane < 16 && key < wend) sl[key - base] = s;
    }
  };
  if (wbeg < wend) {
    v4i bufA[U][NCH], bufB[U][NCH];
    load(wbeg, bufA);
    for (int64_t kt = wbeg; kt < wend; kt += 2 * STEP) {
      load(kt + STEP, bufB);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
      score(kt, bufA);
      load(kt + 2 * STEP, bufA);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + STEP < wend) score(kt + STEP, bufB);
    }
  }
  __syncthreads();
  // write the chunk's scores (coalesced) and histogram them
  int32_t* Sb = S + static_cast<int64_t>(b) * Tk;
  const int cnt = static_cast<int>(nend - base);
  for (int j = threadIdx.x; j < cnt; j += DEC_NT) {
    const int32_t sv = sl[j];
    Sb[base + j] = sv;
    atomicAdd(&lh[score_bin(sv)], 1u);
  }
  __syncthreads();
  // this chunk's histogram, stored whole (no cross-workgroup atomics), and
  // its coarse form (32 fine bins per coarse bin)
  const int64_t ci = static_cast<int64_t>(b) * gridDim.x + blockIdx.x;
  uint32_t* hb = fhist + ci * DEC_BINS;
  for (int j = threadIdx.x; j < DEC_BINS; j += DEC_NT) hb[j] = lh[j];
  if (threadIdx.x < DEC_CBINS) {
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) cs += lh[32 * threadIdx.x + ((j + threadIdx.x) & 31)];
    chist[ci * DEC_CBINS + threadIdx.x] = cs;
  }
}

__global__ __launch_bounds__(DEC_NT) void dec_cand_kernel(
    int Tk, int K, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ S, const uint32_t* __restrict__ bsel, uint32_t* __restrict__ ncand,
    int2* __restrict__ cand, uint32_t* __restrict__ ngt, int nchunks) {
  constexpr int E = kDecChunk / DEC_NT;
  __shared__ uint32_t scratch[DEC_NT / 64 + 2];
  const int b = blockIdx.y;
  const DecRow rw = dec_row(Tk, q_offset, kv_len, b);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDecChunk;
  const int64_t ci = static_cast<int64_t>(b) * nchunks + blockIdx.x;
  if (rw.n <= K || base >= rw.n) {
    if (threadIdx.x == 0) {
      ngt[ci] = 0u;
      ncand[ci] = 0u;
    }
    return;
  }
  const int bstar = static_cast<int>(bsel[2 * b]);
  const int64_t nend = min(base + kDecChunk, rw.n);
  const int32_t* Sb = S + static_cast<int64_t>(b) * Tk;
  // element e of this thread: position base + e*DEC_NT + tid (coalesced)
  int32_t val[E];
  uint32_t gt = 0, nc = 0, cmask = 0;
  // every load issued before any is used (clamped to the chunk's last position)
#pragma unroll
  for (int e = 0; e < E; ++e) val[e] = Sb[min(base + e * DEC_NT + threadIdx.x, nend - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t s = base + e * DEC_NT + threadIdx.x;
    const int bin = s < nend ? score_bin(val[e]) : -1;
    gt += bin > bstar ? 1u : 0u;
    if (bin == bstar) {
      cmask |= 1u << e;
      ++nc;
    }
  }
  uint32_t tot_c;
  const uint32_t ex = block_excl_scan(nc, scratch, &tot_c);
  uint32_t tot_g;
  block_excl_scan(gt, scratch, &tot_g);
  if (threadIdx.x == 0) {
    ncand[ci] = tot_c;
    ngt[ci] = tot_g;
  }
  // this chunk's candidates, in its own slice of the list (at most kDecChunk)
  uint32_t slot = ex;
  int2* cb = cand + ci * kDecChunk;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (cmask & (1u << e)) {
      cb[slot] = make_int2(val[e], static_cast<int>(base + e * DEC_NT + threadIdx.x));
      ++slot;
    }
}

// k-th largest (1-based) of the keys key(i) for i < n with valid(i), radix select
// over LDS-resident data; returns the key. Requires at least k valid keys.
template <typename F>
__device__ uint32_t lds_kth_largest(int n, uint32_t k, F keyf, uint32_t* hist, uint32_t* scratch,
                                    uint32_t* red, uint32_t* found) {
  constexpr int NT = TOPK_NT;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    uint32_t u;
    if (keyf(i, u)) {
      lo = min(lo, u);
      hi = max(hi, u);
    }
  }
  block_minmax(lo, hi, red);
  if (lo == hi) return lo;
  const int top = 32 - __clz(lo ^ hi);
  uint32_t mask = ~low_mask(top);
  uint32_t prefix = lo & mask;
  uint32_t krem = k;
  int shift = top;
  while (shift > 0) {
    const int nb = min(11, shift);
    shift -= nb;
    const uint32_t bmask = low_mask(nb);
    for (int j = threadIdx.x; j < TOPK_BINS; j += NT) hist[j] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint32_t u;
      if (keyf(i, u) && (u & mask) == prefix) atomicAdd(&hist[(u >> shift) & bmask], 1u);
    }
    __syncthreads();
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
    prefix |= found[0] << shift;
    krem -= found[1];
    mask |= bmask << shift;
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(TOPK_NT) void dec_resolve_kernel(
    int Tk, int K, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ S, const uint32_t* __restrict__ bsel,
    const uint32_t* __restrict__ ncand, const int2* __restrict__ cand,
    const uint32_t* __restrict__ ngt, uint32_t* __restrict__ off, int nchunks,
    int32_t* __restrict__ thr, int32_t* __restrict__ idx) {
  __shared__ SelectLds sm;
  __shared__ int cval[kDecCap];
  __shared__ int cpos[kDecCap];
  __shared__ uint32_t ccount[kDecMaxChunks];
  const int b = blockIdx.x;
  const DecRow rw = dec_row(Tk, q_offset, kv_len, b);
  int32_t* out = idx + static_cast<int64_t>(b) * K;
  int32_t* th = thr + 4 * b;
  if (rw.n <= K) {  // every candidate is kept (or the row is invalid)
    for (int j = threadIdx.x; j < K; j += TOPK_NT) out[j] = j < rw.n ? j : -1;
    if (threadIdx.x == 0) th[0] = 0;
    return;
  }
  // per-chunk candidate counts -> where each chunk's candidates go in LDS
  const int nch = static_cast<int>((rw.n + kDecChunk - 1) / kDecChunk);
  const uint32_t* cn = ncand + static_cast<int64_t>(b) * nchunks;
  for (int c = threadIdx.x; c < nch; c += TOPK_NT) ccount[c] = cn[c];
  __syncthreads();
  uint32_t nc = 0;
  for (int c0 = 0; c0 < nch; c0 += TOPK_NT) {
    const int c = c0 + threadIdx.x;
    const uint32_t v = c < nch ? ccount[c] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, sm.scratch, &tot);
    if (c < nch) ccount[c] = nc + ex;  // exclusive start of chunk c
    nc += tot;
  }
  __syncthreads();
  if (nc > static_cast<uint32_t>(kDecCap)) {
    // too many equal-bin candidates for LDS: exact selection over the whole row
    select_row(S + static_cast<int64_t>(b) * Tk, rw.n, K, out, nullptr, sm);
    if (threadIdx.x == 0) th[0] = 0;
    return;
  }
  // positions in bins above the candidate bin are all kept
  const uint32_t krem = static_cast<uint32_t>(K) - bsel[2 * b + 1];
  // gather the chunks' lists: entry j of the merged list comes from the last
  // chunk whose start is <= j (empty chunks share their successor's start);
  // eight loads in flight per thread
  {
    const int2* cbase = cand + static_cast<int64_t>(b) * nchunks * kDecChunk;
    for (uint32_t j0 = 0; j0 < nc; j0 += 8 * TOPK_NT) {
      int2 cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // nc >= 1 here (at least K - (count above b*) candidates); entries
        // past nc read the last one and are not stored
        const uint32_t j = min(j0 + u * TOPK_NT + threadIdx.x, nc - 1);
        int lo = 0, hi = nch - 1;  // largest c with ccount[c] <= j
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (ccount[mid] <= j) lo = mid;
          else hi = mid - 1;
        }
        cv[u] = cbase[static_cast<int64_t>(lo) * kDecChunk + (j - ccount[lo])];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t j = j0 + u * TOPK_NT + threadIdx.x;
        if (j < nc) {
          cval[j] = cv[u].x;
          cpos[j] = cv[u].y;
        }
      }
    }
  }
  __syncthreads();
  const int n = static_cast<int>(nc);
  // exact K-th score among the candidates
  const uint32_t vkey = lds_kth_largest(
      n, krem,
      [&](int i, uint32_t& u) {
        u = score_key(cval[i]);
        return true;
      },
      sm.hist, sm.scratch, sm.red, sm.found);
  const int32_t vstar = key_score(vkey);
  uint32_t ngt2 = 0;
  for (int j = threadIdx.x; j < n; j += TOPK_NT) ngt2 += cval[j] > vstar ? 1u : 0u;
  ngt2 = wave_sum(ngt2);
  if ((threadIdx.x & 63) == 0) sm.red[threadIdx.x >> 6] = ngt2;
  __syncthreads();
  uint32_t cgt = 0;
  for (int w2 = 0; w2 < TOPK_NT / 64; ++w2) cgt += sm.red[w2];
  __syncthreads();
  const uint32_t r = krem - cgt;  // ties at v* to keep, lowest positions first
  // r-th smallest position among the ties = r-th largest of the complemented positions
  const uint32_t ckey = lds_kth_largest(
      n, r,
      [&](int i, uint32_t& u) {
        u = ~static_cast<uint32_t>(cpos[i]);
        return cval[i] == vstar;
      },
      sm.hist, sm.scratch, sm.red, sm.found);
  const int32_t scut = static_cast<int32_t>(~ckey);
  // per-chunk selected counts (LDS) -> exclusive offsets
  uint32_t* ob = off + static_cast<int64_t>(b) * nchunks;
  const uint32_t* gb = ngt + static_cast<int64_t>(b) * nchunks;
  for (int c = threadIdx.x; c < nchunks; c += TOPK_NT) ccount[c] = gb[c];
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += TOPK_NT) {
    const int v = cval[j], s = cpos[j];
    if (v > vstar || (v == vstar && s <= scut)) atomicAdd(&ccount[s / kDecChunk], 1u);
  }
  __syncthreads();
  uint32_t carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += TOPK_NT) {
    const int c = c0 + threadIdx.x;
    const uint32_t v = c < nchunks ? ccount[c] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, sm.scratch, &tot);
    if (c < nchunks) ob[c] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    th[0] = 1;
    th[1] = vstar;
    th[2] = scut;
  }
}

__global__ __launch_bounds__(DEC_NT) void dec_compact_kernel(
    int Tk, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ S, const int32_t* __restrict__ thr,
    const uint32_t* __restrict__ off, int nchunks, int K, int32_t* __restrict__ idx) {
  constexpr int E = kDecChunk / DEC_NT;
  constexpr int NW = DEC_NT / 64;
  __shared__ uint32_t cnt[E * NW];
  const int b = blockIdx.y;
  const int32_t* th = thr + 4 * b;
  if (th[0] != 1) return;
  const DecRow rw = dec_row(Tk, q_offset, kv_len, b);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDecChunk;
  if (base >= rw.n) return;
  const int32_t vstar = th[1], scut = th[2];
  const int32_t* Sb = S + static_cast<int64_t>(b) * Tk;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // position of element e of this thread: base + e*DEC_NT + tid, i.e. position
  // order is (e, wave, lane): a ballot per e ranks lanes, LDS counts rank (e, wave)
  uint64_t km[E];
  int32_t vals[E];  // every load issued before any is used
#pragma unroll
  for (int e = 0; e < E; ++e) vals[e] = Sb[min(base + e * DEC_NT + threadIdx.x, rw.n - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t s = base + e * DEC_NT + threadIdx.x;
    const int32_t v = vals[e];
    const bool keep = s < rw.n && (v > vstar || (v == vstar && s <= scut));
    km[e] = __ballot(keep);
    if (lane == 0) cnt[e * NW + wv] = __popcll(km[e]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = off[static_cast<int64_t>(b) * nchunks + blockIdx.x];
    for (int j = 0; j < E * NW; ++j) {
      const uint32_t c = cnt[j];
      cnt[j] = run;
      run += c;
    }
  }
  __syncthreads();
  int32_t* out = idx + static_cast<int64_t>(b) * K;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((km[e] >> lane) & 1ull) {
      const uint32_t pos = cnt[e * NW + wv] + __popcll(km[e] & below);
      if (pos < static_cast<uint32_t>(K)) out[pos] = static_cast<int32_t>(base + e * DEC_NT + threadIdx.x);
    }
}

// ---------------------------------------------------------------- host side

DecLayout decode_layout(const Geom& g) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  DecLayout L{};
  L.nchunks = static_cast<int>((static_cast<int64_t>(g.Tk) + kDecChunk - 1) / kDecChunk);
  size_t o = 0;
  L.scores = o;  o += al(static_cast<size_t>(g.B) * g.Tk * sizeof(int32_t));
  L.hist = o;    o += al(static_cast<size_t>(g.B) * L.nchunks * DEC_BINS * sizeof(uint32_t));
  L.ncand = o;   o += al(static_cast<size_t>(g.B) * L.nchunks * sizeof(uint32_t));
  L.cand = o;    o += al(static_cast<size_t>(g.B) * L.nchunks * kDecChunk * sizeof(int2));
  L.ngt = o;     o += al(static_cast<size_t>(g.B) * L.nchunks * sizeof(uint32_t));
  L.off = o;     o += al(static_cast<size_t>(g.B) * L.nchunks * sizeof(uint32_t));
  L.thr = o;     o += al(static_cast<size_t>(g.B) * 4 * sizeof(int32_t));
  L.bsel = o;    o += al(static_cast<size_t>(g.B) * 2 * sizeof(uint32_t));
  L.idx = o;     o += al(static_cast<size_t>(g.B) * g.K * sizeof(int32_t));
  L.attn = o;
  L.splits = sparse_attn_pick_splits(g);
  o += al(sparse_attn_workspace(g, L.splits));
  L.chist = o;   o += al(static_cast<size_t>(g.B) * L.nchunks * DEC_CBINS * sizeof(uint32_t));
  L.total = o;
  return L;
}

template <int H_I, int D_I>
static hipError_t launch_score_hd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                  const int8_t* w, int64_t wsb, int32_t* S, uint32_t* hist,
                                  uint32_t* chist, int nchunks, hipStream_t st) {
  {
    KernelTimer timer(LCI_KERNEL_DEC_SCORE, st);
    hipLaunchKernelGGL((dec_score_kernel<H_I, D_I>), dim3(nchunks, g.B), dim3(DEC_NT), 0, st, g.Tk,
                       g.K, g.q_offset, g.kv_len, q_idx, k_idx, w, wsb, S, hist, chist);
  }
  return hipGetLastError();
}

template <int H_I>
static hipError_t launch_score_h(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                 const int8_t* w, int64_t wsb, int32_t* S, uint32_t* hist,
                                 uint32_t* chist, int nchunks, hipStream_t st) {
  switch (g.d_I) {
    case 32: return launch_score_hd<H_I, 32>(g, q_idx, k_idx, w, wsb, S, hist, chist, nchunks, st);
    case 64: return launch_score_hd<H_I, 64>(g, q_idx, k_idx, w, wsb, S, hist, chist, nchunks, st);
    case 128:
      if constexpr (H_I * 128 <= 1024)
        return launch_score_hd<H_I, 128>(g, q_idx, k_idx, w, wsb, S, hist, chist, nchunks, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                         const int8_t* w, int64_t wsb, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const uint16_t* gate,
                         const uint16_t* mix, float scale, uint16_t* out,
                         float* lse, int32_t* idx_out, void* workspace, hipStream_t st) {
  const DecLayout L = decode_layout(g);
  char* ws = static_cast<char*>(workspace);
  int32_t* S = reinterpret_cast<int32_t*>(ws + L.scores);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
  uint32_t* chist = reinterpret_cast<uint32_t*>(ws + L.chist);
  uint32_t* ncand = reinterpret_cast<uint32_t*>(ws + L.ncand);
  int2* cand = reinterpret_cast<int2*>(ws + L.cand);
  uint32_t* ngt = reinterpret_cast<uint32_t*>(ws + L.ngt);
  uint32_t* off = reinterpret_cast<uint32_t*>(ws + L.off);
  int32_t* thr = reinterpret_cast<int32_t*>(ws + L.thr);
  uint32_t* bsel = reinterpret_cast<uint32_t*>(ws + L.bsel);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);

  hipError_t e = hipSuccess;
  switch (g.H_I) {
    case 1: e = launch_score_h<1>(g, q_idx, k_idx, w, wsb, S, hist, chist, L.nchunks, st); break;
    case 2: e = launch_score_h<2>(g, q_idx, k_idx, w, wsb, S, hist, chist, L.nchunks, st); break;
    case 4: e = launch_score_h<4>(g, q_idx, k_idx, w, wsb, S, hist, chist, L.nchunks, st); break;
    case 8: e = launch_score_h<8>(g, q_idx, k_idx, w, wsb, S, hist, chist, L.nchunks, st); break;
    case 16: e = launch_score_h<16>(g, q_idx, k_idx, w, wsb, S, hist, chist, L.nchunks, st); break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_DEC_THRESH, st);
    hipLaunchKernelGGL(dec_thresh_kernel, dim3(g.B), dim3(DEC_NT), 0, st, g.Tk, g.K, g.q_offset,
                       g.kv_len, hist, chist, L.nchunks, bsel);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_DEC_CAND, st);
    hipLaunchKernelGGL(dec_cand_kernel, dim3(L.nchunks, g.B), dim3(DEC_NT), 0, st, g.Tk, g.K,
                       g.q_offset, g.kv_len, S, bsel, ncand, cand, ngt, L.nchunks);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_DEC_RESOLVE, st);
    hipLaunchKernelGGL(dec_resolve_kernel, dim3(g.B), dim3(TOPK_NT), 0, st, g.Tk, g.K, g.q_offset,
                       g.kv_len, S, bsel, ncand, cand, ngt, off, L.nchunks, thr, idx);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_DEC_COMPACT, st);
    hipLaunchKernelGGL(dec_compact_kernel, dim3(L.nchunks, g.B), dim3(DEC_NT), 0, st, g.Tk,
                       g.q_offset, g.kv_len, S, thr, off, L.nchunks, g.K, idx);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_sparse_attn(g, q, k, v, idx, gate, mix, scale, out, lse, L.splits, ws + L.attn,
                            false,
                            st);
}

}  // namespace lci
