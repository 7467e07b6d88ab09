// Block-granular Top-K (gfx950): the selection keeps blocks of positions
// instead of single positions.
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer + Top-K: How
// Fine-Grained Sparse Attention Works", steps 1-2: the scorer rates positions
// or blocks, and the selection keeps the top K positions or blocks. A block j
// holds positions j*block .. j*block + block - 1 and rates as its best causal
// position; K blocks are kept under the order used for positions (higher
// score, then lower block index). The index row lists the kept blocks' causal
// positions in ascending order (K*block entries, -1 padded), so the attention
// kernels take it like any other index row.
//
// One workgroup per query row, everything in LDS:
//   1. block maxima of the row's position scores (order-preserving uint32
//      keys): each lane takes 4 consecutive positions (one 16-byte load when
//      the row is aligned), eight loads in flight per lane; a wave's load
//      covers 256 consecutive positions, i.e. whole blocks, so the max over
//      the lanes of a block (xor shuffles) is the block's, and its first lane
//      stores it: no atomics;
//   2. rows of at most 256 blocks: each thread ranks one block against all
//      the others (broadcast LDS reads), and one workgroup scan in block order
//      gives the kept blocks their slots;
//      longer rows: radix select over the block keys, 8 bits per pass (LDS
//      histogram with integer atomics, so the result does not depend on their
//      order) finds the exact K-th key v* and r = how many blocks with key v*
//      are kept; a compaction in block order follows (each thread owns a
//      contiguous range of blocks; two workgroup scans give every kept block
//      its slot: keys > v*, and the first r keys == v*);
//   3. expansion of the kept blocks into positions, coalesced stores; with the
//      dense-tile attention path on, the row's bit mask over positions and its
//      row flag as well.
#include "../../include/lci.h"
#include "common.h"
#include "internal.h"

namespace lci {

namespace {

constexpr int BT_NT = 256;

// order-preserving keys of int32 scores (0 is the key of INT32_MIN)
__device__ __forceinline__ uint32_t bkey(int32_t s) { return static_cast<uint32_t>(s) ^ 0x80000000u; }
__device__ __forceinline__ int32_t bscore(uint32_t k) { return static_cast<int32_t>(k ^ 0x80000000u); }

__device__ __forceinline__ uint32_t low_bits(int r) {
  return r >= 32 ? 0xffffffffu : (r <= 0 ? 0u : (1u << r) - 1u);
}

// Rows of more than BT_NT blocks: radix select of the K-th largest block key,
// then the ordered compaction. Fills blist[0..K) and the kept bits.
__device__ void select_blocks_radix(const uint32_t* key, int nb, int K, int32_t* blist,
                                    uint32_t* kept, uint32_t* hist, uint32_t* scratch,
                                    uint32_t* found) {
  const int t = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u, krem = static_cast<uint32_t>(K);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0u;
    __syncthreads();
    for (int j = t; j < nb; j += BT_NT) {
      const uint32_t k = key[j];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t takes digit 255 - t: its exclusive prefix counts the larger digits
    const uint32_t c = hist[255 - t];
    uint32_t tot;
    const uint32_t above = block_excl_scan(c, scratch, &tot);
    if (above < krem && krem <= above + c) {
      found[0] = static_cast<uint32_t>(255 - t);
      found[1] = above;
    }
    __syncthreads();
    prefix |= found[0] << shift;
    pmask |= 255u << shift;
    krem -= found[1];
    __syncthreads();
  }
  const uint32_t vstar = prefix;  // keys > vstar are kept, and the first krem keys == vstar

  // compaction in block order over contiguous ranges
  const int E = (nb + BT_NT - 1) / BT_NT;
  const int j0 = min(t * E, nb), j1 = min(j0 + E, nb);
  uint32_t ngt = 0, neq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = key[j];
    ngt += k > vstar;
    neq += k == vstar;
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan(neq, scratch, &tot);
  const uint32_t eq_keep = eq_before >= krem ? 0u : min(neq, krem - eq_before);
  uint32_t slot = block_excl_scan(ngt + eq_keep, scratch, &tot);
  uint32_t eq_seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = key[j];
    bool keep = k > vstar;
    if (k == vstar) {
      keep = eq_seen < krem;
      ++eq_seen;
    }
    if (keep) {
      blist[slot++] = j;
      atomicOr(&kept[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(BT_NT) void block_topk_kernel(
    int Tq, int Tk, int K, int lb, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ scores, int64_t stride,
    int64_t batch_rows, int row_begin, int row_count, int32_t* __restrict__ idx,
    int32_t* __restrict__ sel, uint32_t* __restrict__ dmask, uint8_t* __restrict__ dflag, int Wm, int lim) {
  __shared__ __align__(16) uint32_t key[kBlockTopkMaxBlocks];
  __shared__ int32_t blist[kBlockTopkMaxKeep];
  __shared__ uint32_t kept[kBlockTopkMaxBlocks / 32];  // bit j: block j is kept
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scratch[BT_NT / 64 + 2];
  __shared__ uint32_t found[2];
  static_assert(BT_NT == 256, "one thread per histogram bin");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int rr = blockIdx.x;
  const int b = blockIdx.y;
  const int row = row_begin + rr;
  const int64_t grow = static_cast<int64_t>(b) * Tq + row;
  const int block = 1 << lb;
  const int KP = K << lb;
  int32_t* out = idx + grow * KP;
  int32_t* outs = sel ? sel + grow * K : nullptr;
  const int kvl = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + row;
  const bool valid = kvl <= Tk && p >= 0 && p < kvl;
  const int n = valid ? static_cast<int>(p + 1) : 0;
  const int nb = (n + block - 1) >> lb;
  const int32_t* S = scores + (static_cast<int64_t>(b) * batch_rows + rr) * stride;

  // 1. block maxima
  for (int j = t; j < (nb + 31) / 32; j += BT_NT) kept[j] = 0u;
  // keys past the last block up to a multiple of 4 read as the minimum (the
  // ranking below reads keys four at a time)
  if (t < 4 && nb + t < kBlockTopkMaxBlocks) key[nb + t] = 0u;
  // 16-byte loads when every row starts 16-byte aligned: the clamped last load
  // then ends inside the row
  const bool vec = (reinterpret_cast<uintptr_t>(S) & 15) == 0 && (stride & 3) == 0;
  const int wbase = (t >> 6) * 256 + 4 * lane;  // this lane's first position in a 1024 chunk
  const int lanes = block >= 4 ? block >> 2 : 1;  // lanes that share a block
  for (int s0 = 0; s0 < n; s0 += 8 * 1024) {
    int4 v[8];
    if (vec) {
      const int last4 = (n - 1) & ~3;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const int4*>(S + min(s0 + u * 1024 + wbase, last4));
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u * 1024 + wbase;
        v[u] = make_int4(S[min(s, n - 1)], S[min(s + 1, n - 1)], S[min(s + 2, n - 1)],
                         S[min(s + 3, n - 1)]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * 1024 + wbase;
      // positions at or past n read as the minimum key
      const uint32_t k0 = s < n ? bkey(v[u].x) : 0u, k1 = s + 1 < n ? bkey(v[u].y) : 0u;
      const uint32_t k2 = s + 2 < n ? bkey(v[u].z) : 0u, k3 = s + 3 < n ? bkey(v[u].w) : 0u;
      if (block == 2) {
        if (s < n) key[s >> 1] = max(k0, k1);
        if (s + 2 < n) key[(s >> 1) + 1] = max(k2, k3);
      } else {
        uint32_t m = max(max(k0, k1), max(k2, k3));
        for (int o = 1; o < lanes; o <<= 1)
          m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o, 64)));
        if ((lane & (lanes - 1)) == 0 && s < n) key[s >> lb] = m;
      }
    }
  }
  __syncthreads();

  if (nb <= K) {  // every block is kept (or the row is invalid): positions 0..n-1
    for (int e = t; e < KP; e += BT_NT) out[e] = e < n ? e : -1;
    if (outs)
      for (int j = t; j < K; j += BT_NT) outs[j] = j < nb ? bscore(key[j]) : INT32_MIN;
    if (dmask) {
      if (t == 0) dflag[grow] = valid ? kRowAll : kRowEmpty;
      for (int w = t; w < Wm; w += BT_NT) dmask[grow * Wm + w] = low_bits(n - 32 * w);
    }
    return;
  }

  // 2. the K best blocks, in block order
  if (nb <= BT_NT) {
    // rank of block t: how many blocks come before it in the order (keys read
    // four at a time; the padding keys past nb never come before a block)
    const uint32_t kt = t < nb ? key[t] : 0u;
    uint32_t rank = 0;
    const uint4* k4 = reinterpret_cast<const uint4*>(key);
    for (int i = 0; i < nb; i += 4) {
      const uint4 q = k4[i >> 2];
      rank += (q.x > kt) | ((q.x == kt) & (i < t));
      rank += (q.y > kt) | ((q.y == kt) & (i + 1 < t));
      rank += (q.z > kt) | ((q.z == kt) & (i + 2 < t));
      rank += (q.w > kt) | ((q.w == kt) & (i + 3 < t));
    }
    const bool keep = t < nb && rank < static_cast<uint32_t>(K);
    uint32_t tot;
    const uint32_t slot = block_excl_scan(keep ? 1u : 0u, scratch, &tot);
    if (keep) {
      blist[slot] = t;
      atomicOr(&kept[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
  } else {
    select_blocks_radix(key, nb, K, blist, kept, hist, scratch, found);
  }

  // 3. the kept blocks' causal positions, ascending (only the last causal block
  // can be partial, and it is the highest kept block when kept)
  for (int e = t; e < KP; e += BT_NT) {
    const int s = (blist[e >> lb] << lb) + (e & (block - 1));
    out[e] = s < n ? s : -1;
  }
  if (outs)
    for (int j = t; j < K; j += BT_NT) outs[j] = bscore(key[blist[j]]);
  if (dmask == nullptr) return;
  // the tile path takes rows whose history is at most lim positions long
  const bool tile = n <= lim;
  if (t == 0) dflag[grow] = tile ? kRowMasked : kRowGather;
  if (!tile) return;
  for (int w = t; w < Wm; w += BT_NT) {
    const int p0 = 32 * w;
    uint32_t word = 0u;
    if (p0 >= n) {
      // past the row's history (the row's trailing words): nothing kept
    } else if (lb >= 5) {
      const int j = p0 >> lb;  // one block covers the word
      if (j < nb && ((kept[j >> 5] >> (j & 31)) & 1u)) word = 0xffffffffu;
    } else {
      // 32 >> lb blocks per word, starting at a multiple of 32 >> lb: their kept
      // bits, each widened to `block` bits
      const int j = p0 >> lb;
      const int per = 32 >> lb;
      const uint32_t bits = (kept[j >> 5] >> (j & 31)) & ((per == 32) ? 0xffffffffu : ((1u << per) - 1u));
      for (int q = 0; q < per; ++q)
        if ((bits >> q) & 1u) word |= low_bits(block) << (q << lb);
    }
    dmask[grow * Wm + w] = word & low_bits(n - p0);
  }
}

}  // namespace

hipError_t launch_block_topk(const Geom& g, const int32_t* scores, int64_t stride,
                             int64_t batch_rows, int row_begin, int row_count, int32_t* idx,
                             int32_t* sel, const DenseMasks* dm, hipStream_t st) {
  const int lb = __builtin_ctz(static_cast<unsigned>(g.block));
  dim3 grid(static_cast<uint32_t>(row_count), static_cast<uint32_t>(g.B));
  {
    KernelTimer timer(LCI_KERNEL_TOPK, st);
    hipLaunchKernelGGL(block_topk_kernel, grid, dim3(BT_NT), 0, st, g.Tq, g.Tk, g.K, lb,
                       g.q_offset, g.kv_len, scores, stride, batch_rows, row_begin, row_count, idx, sel,
                       dm ? dm->mask : nullptr, dm ? dm->flag : nullptr, dm ? dm->Wm : 0,
                       dm ? dm->lim : 0);
  }
  return hipGetLastError();
}

}  // namespace lci
