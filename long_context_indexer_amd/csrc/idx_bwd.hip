// Gradients of the scorer's distillation loss (gfx950).
//
// "How Fine-Grained Sparse Attention Reshapes Long-Context Architecture in
// Large Models", section "How Indexer + Top-K Works at Runtime": the indexer's
// selection distribution is distilled from a full-attention teacher, without
// which an early indexer is near random and its gradients weak; "Hybrid Sparse
// Attention for Long-Context LLMs", section "Engineering and Evaluation
// Recommendations", training side: the scorer is trained jointly. The loss
// (a reading; the pages give none): for query row i and its index row, the
// scorer's distribution over the entries is softmax_t(tau * S_t) with
//   S_t = sum_h w_h max(0, d_ht),  d_ht = qI[i,h] . kI[idx_t]   (exact int32),
// and L_i = sum_t T_t (log T_t - log p_t) for the teacher's weights T. With
// q, k, w taken as real numbers and the ReLU's derivative 0 at 0:
//   g_t = tau (p_t sum_u T_u - T_t),
//   dw[i,h]   = sum_t g_t max(0, d_ht),
//   dq[i,h,:] = w_h sum_t g_t [d_ht > 0] kI[idx_t],
//   dk[s,:]  += g_t sum_h w_h [d_ht > 0] qI[i,h]   for every entry with idx_t = s.
// With index sets (per-head index rows, as in the runtime pseudocode of the
// first page and the Indexer + Top-K pseudocode of the second), set g is the
// scorer of its group of H_I/sets heads over its own index rows and teacher:
// each set has the loss above on its heads, and dk sums over the sets. The sets
// run one after another; their dk sums meet in one fixed-point accumulator.
//
//   ibwd_row_kernel    one workgroup per query row: the entries' scores from the
//                      int8 rows (v_dot4 over d_I, exact), the softmax of tau*S
//                      and the loss (workgroup reductions in a fixed order), g
//                      and the heads' ReLU masks kept per entry for dk; dw
//                      reduced in a fixed order; dq on bf16 MFMA from the
//                      entries' key rows staged in LDS 128 at a time, with g
//                      split exactly into three bf16 parts.
//   ibwd_count/fill    the transpose of the index rows: for each position, the
//                      entries that point at it (counts, an exclusive scan,
//                      then the entry numbers in any order).
//   ibwd_dk_kernel     one wave per 256 entries of the position-ordered list:
//                      dk[s, j] (lane j) sums, over the entries of s, g_t u_tj
//                      with u_t = sum_h w_h [d_ht > 0] qI[i,h] (exact: v_dot4
//                      of the row's heads of feature j, read from a transposed
//                      copy of the query rows, with the entry's masked
//                      weights), each product rounded to 32 fraction bits
//                      and added as a 64-bit integer: the sum does not depend
//                      on the entries' order, so dk is deterministic.
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"

namespace lci {

constexpr int IB_NT = 256;
constexpr double kIbFix = 4294967296.0;  // 2^32: fraction bits of the dk sums

// Sum over the workgroup in a fixed order (wave shuffles, then the waves in order).
__device__ __forceinline__ float ib_block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < IB_NT / 64; ++w) s += red[w];
  return s;
}
__device__ __forceinline__ float ib_block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int w = 0; w < IB_NT / 64; ++w) s = fmaxf(s, red[w]);
  return s;
}

// One workgroup per query row (blockIdx.x = b*Tq + i) and one index set: H_I is
// the set's heads, the first of them at q_idx, dq and dw (rows of q_heads
// heads); the set's index row, teacher row and loss of (b, i) are row
// b*brow + i of idx, teacher and loss. Dynamic LDS: K floats of g (z first),
// the K positions, K 16-bit head masks (bit h: d_ht > 0; 0 for skipped entries).
template <int H_I, int D_I>
__global__ __launch_bounds__(IB_NT) void ibwd_row_kernel(
    int Tq, int Tk, int K, int q_heads, int64_t brow, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const int8_t* __restrict__ w, int64_t wsb, int64_t wsq,
    const int32_t* __restrict__ idx, const float* __restrict__ teacher, float tau,
    float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw,
    float* __restrict__ g_ent, uint16_t* __restrict__ m_ent) {
  static_assert(D_I % 16 == 0 && H_I * (D_I / 4) <= IB_NT, "thread mapping of dq");
  constexpr int NW = D_I / 4;  // int8 quads of a row
  static_assert(H_I <= 16, "16-bit head masks");
  extern __shared__ __align__(16) float gz[];  // K floats, K positions, K 16-bit masks
  int* sidx = reinterpret_cast<int*>(gz + K);
  uint16_t* hmask = reinterpret_cast<uint16_t*>(sidx + K);
  __shared__ __align__(16) int qrow[H_I * NW];
  __shared__ float red[IB_NT / 64];
  // dq on MFMA: key rows of KCH entries as bf16, one row of KTS per feature
  // (padded so a 16-byte read by 16 lanes of 16 features touches every bank
  // once); afterwards the waves' partial sums
  constexpr int KCH = 128;
  constexpr int KTS = KCH + 8;
  constexpr int KMT = (H_I + 7) / 8;  // MFMA row tiles (8 heads x 3 parts each)
  constexpr int KNT = D_I / 32;       // MFMA column tiles (32 features each)
  static_assert(D_I % 32 == 0 && KCH == 2 * IB_NT / 4 && 16 * H_I <= 2 * KTS,
                "dq staging and the partial sums' room");
  __shared__ __align__(16) uint16_t kT[D_I * KTS];

  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / Tq);
  const int i = static_cast<int>(row % Tq);
  const int kvl0 = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
  const bool rok = kvl0 <= Tk && p >= 0 && p < kvl0;
  const int64_t irow = static_cast<int64_t>(b) * brow + i;  // the set's index row
  float* dqr = dq + row * q_heads * D_I;
  float* dwr = dw + row * q_heads;
  for (int j = t; j < H_I * D_I; j += IB_NT) dqr[j] = 0.f;
  if (t < H_I) dwr[t] = 0.f;
  if (loss && t == 0) loss[irow] = 0.f;
  if (!rok) return;
  const int* qsrc = reinterpret_cast<const int*>(q_idx + row * q_heads * D_I);
  for (int j = t; j < H_I * NW; j += IB_NT) qrow[j] = qsrc[j];
  int wh[H_I];
  const int8_t* wr = w + b * wsb + static_cast<int64_t>(i) * wsq;
#pragma unroll
  for (int h = 0; h < H_I; ++h) wh[h] = static_cast<int>(wr[h]);
  __syncthreads();
  const int32_t* ir = idx + irow * K;
  const float* Tr = teacher + irow * K;
  const int8_t* kb = k_idx + static_cast<int64_t>(b) * Tk * D_I;

  // 1. z_t = tau * S_t for the valid entries (-inf for the others), max
  // A thread takes its entries e0 + u IB_NT (u < EB) together: the positions,
  // then the key rows, every load issued before any is used (one memory
  // latency per EB entries); then head by head, the head's query quads read
  // once from LDS for all EB rows (a compiler barrier per head keeps the
  // query row out of registers). Entries past K or outside 0..p read row 0
  // and are not used.
  constexpr int KQ = NW / 4;  // 16-byte pieces of a row
  constexpr int EB = 2;
  float mloc = -INFINITY;
  for (int e0 = t; e0 < K; e0 += EB * IB_NT) {
    int sv[EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int e = e0 + u * IB_NT;
      sv[u] = e < K ? ir[e] : -1;
    }
    int4 kq[EB][KQ];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int s = sv[u] >= 0 && sv[u] <= p ? sv[u] : 0;
      const int4* kr = reinterpret_cast<const int4*>(kb + static_cast<int64_t>(s) * D_I);
#pragma unroll
      for (int c = 0; c < KQ; ++c) kq[u][c] = kr[c];
    }
    int S[EB];
    uint32_t hm[EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) S[u] = 0, hm[u] = 0u;
#pragma unroll
    for (int h = 0; h < H_I; ++h) {
#pragma unroll
      for (int u = 0; u < EB; ++u) asm volatile("" : "+v"(S[u]) : : "memory");
      int4 qq[KQ];
#pragma unroll
      for (int c = 0; c < KQ; ++c) qq[c] = reinterpret_cast<const int4*>(qrow + h * NW)[c];
#pragma unroll
      for (int u = 0; u < EB; ++u) {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < KQ; ++c) {
          acc = __builtin_amdgcn_sdot4(qq[c].x, kq[u][c].x, acc, false);
          acc = __builtin_amdgcn_sdot4(qq[c].y, kq[u][c].y, acc, false);
          acc = __builtin_amdgcn_sdot4(qq[c].z, kq[u][c].z, acc, false);
          acc = __builtin_amdgcn_sdot4(qq[c].w, kq[u][c].w, acc, false);
        }
        S[u] += wh[h] * max(acc, 0);
        hm[u] |= (acc > 0 ? 1u : 0u) << h;
      }
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int e = e0 + u * IB_NT;
      if (e >= K) break;
      const bool ok = sv[u] >= 0 && sv[u] <= p;
      const float z = ok ? tau * static_cast<float>(S[u]) : -INFINITY;
      gz[e] = z;
      sidx[e] = sv[u];
      hmask[e] = static_cast<uint16_t>(ok ? hm[u] : 0u);
      mloc = fmaxf(mloc, z);
    }
  }
  const float m = ib_block_max(mloc, red);
  if (m == -INFINITY) return;  // no valid entry: zeros (written above)
  // 2. softmax normaliser and the teacher's mass
  float zs = 0.f, ts = 0.f;
  for (int e = t; e < K; e += IB_NT) {
    const float z = gz[e];
    if (z == -INFINITY) continue;
    zs += __expf(z - m);
    ts += Tr[e];
  }
  const float Z = ib_block_sum(zs, red);
  const float Tsum = ib_block_sum(ts, red);
  const float logZ = m + __logf(Z);
  // 3. loss and g; g and the masks kept per entry for dk
  float lloc = 0.f;
  float* gr = g_ent + row * K;
  uint16_t* mr = m_ent + row * K;
  for (int e = t; e < K; e += IB_NT) {
    const float z = gz[e];
    float g = 0.f;
    if (z != -INFINITY) {
      const float logp = z - logZ;
      const float pt = __expf(logp);
      const float te = Tr[e];
      if (te > 0.f) lloc += te * (__logf(te) - logp);
      g = tau * (pt * Tsum - te);
    }
    gz[e] = g;  // the same thread reads it back below, after a barrier
    gr[e] = g;
    mr[e] = hmask[e];
  }
  const float L = ib_block_sum(lloc, red);  // its barriers publish g and the masks
  if (loss && t == 0) loss[irow] = L;
  // 4. dq[h, :] = w_h sum_t G[h, t] kI[idx_t] with G[h, t] = g_t [d_ht > 0]: a
  // product [heads x entries] x [entries x features] on bf16 MFMA. Per chunk of
  // KCH entries the key rows go to LDS as bf16 (exact for int8), feature-major;
  // wave wv multiplies entries 32 wv .. 32 wv + 31 of the chunk. G enters split
  // exactly into three bf16 parts (g = hi + mid + lo to 24 bits; each product
  // with an int8 value is exact in fp32): A-operand row m = 8 part + h % 8 of
  // tile h / 8, so a lane's accumulators hold the three parts of the same heads
  // (elements c, 4 + c, 8 + c) and add them itself. The waves' sums meet in LDS,
  // added in wave order: deterministic.
  {
    const int lane = t & 63, wv = t >> 6;
    const int ln = lane & 31, hf = lane >> 5;
    const int part = ln >> 3;  // 0 hi, 1 mid, 2 lo, 3 unused rows
    v16f acc[KMT][KNT];
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < KNT; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;
    // thread t stages entries c0 + 2 pr and c0 + 2 pr + 1, features q FPT .. + FPT - 1,
    // as bf16 pairs, one dword per feature (zeros for entries without a passing
    // head); the next chunk's key bytes are loaded while this chunk multiplies
    constexpr int FPT = D_I / 4;
    const int pr = t >> 2, q = t & 3;
    uint32_t kw[2][FPT / 4];
    auto load_chunk = [&](int c0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = c0 + 2 * pr + u;
        const bool on = e < K && hmask[e] != 0;
        const int* kr = reinterpret_cast<const int*>(
            kb + static_cast<int64_t>(on ? sidx[e] : 0) * D_I + q * FPT);
#pragma unroll
        for (int c = 0; c < FPT / 4; ++c) kw[u][c] = on ? static_cast<uint32_t>(kr[c]) : 0u;
      }
    };
    load_chunk(0);  // g, positions and masks are visible (the loss sum's barriers)
    for (int c0 = 0; c0 < K; c0 += KCH) {
      __syncthreads();  // the previous chunk is consumed
      {
#pragma unroll
        for (int f = 0; f < FPT; ++f) {
          // an int8 value as bf16: the top half of its exact fp32 bits
          const int sh = 8 * (f & 3);
          const float x0 = static_cast<float>(static_cast<int8_t>(kw[0][f >> 2] >> sh));
          const float x1 = static_cast<float>(static_cast<int8_t>(kw[1][f >> 2] >> sh));
          *reinterpret_cast<uint32_t*>(&kT[(q * FPT + f) * KTS + 2 * pr]) =
              (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
        }
      }
      __syncthreads();
      if (c0 + KCH < K) load_chunk(c0 + KCH);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int el = 32 * wv + 16 * s + 8 * hf;  // this lane's 8 entries (chunk-local)
        v8bf bk[KNT];
#pragma unroll
        for (int nt = 0; nt < KNT; ++nt)
          bk[nt] = *reinterpret_cast<const v8bf*>(&kT[(ln + 32 * nt) * KTS + el]);
        float gv[8];
        uint32_t hm[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = c0 + el + j;
          gv[j] = e < K ? gz[e] : 0.f;
          hm[j] = e < K ? hmask[e] : 0u;
        }
#pragma unroll
        for (int mt = 0; mt < KMT; ++mt) {
          const int h = 8 * mt + (ln & 7);
          v8bf a;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = (part < 3 && h < H_I && ((hm[j] >> h) & 1u)) ? gv[j] : 0.f;
            const __bf16 hi = static_cast<__bf16>(v);
            const float r1 = v - static_cast<float>(hi);
            const __bf16 mid = static_cast<__bf16>(r1);
            const __bf16 lo = static_cast<__bf16>(r1 - static_cast<float>(mid));
            a[j] = part == 0 ? hi : (part == 1 ? mid : lo);
          }
#pragma unroll
          for (int nt = 0; nt < KNT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave is done with the key rows: the area holds the sums
    float* ps = reinterpret_cast<float*>(kT);  // [4 waves][H_I][D_I]
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < KNT; ++nt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int h = 8 * mt + 4 * hf + c;
          if (h < H_I)
            ps[(wv * H_I + h) * D_I + ln + 32 * nt] =
                (acc[mt][nt][c] + acc[mt][nt][4 + c]) + acc[mt][nt][8 + c];
        }
    __syncthreads();
    for (int x = t; x < H_I * D_I; x += IB_NT) {
      float v = ps[x];
#pragma unroll
      for (int w2 = 1; w2 < IB_NT / 64; ++w2) v += ps[w2 * H_I * D_I + x];
      ps[x] = v;  // the sum G kI, kept for dw
      dqr[x] = static_cast<float>(wh[x / D_I]) * v;
    }
    __syncthreads();
    // dw_h = sum_t g_t relu(d_ht) = sum_t G[h, t] d_ht = q_h . (G kI)[h, :]: the
    // same sum read through the unscaled dq row; wave wv takes heads wv, wv + 4,
    // ..., a lane features lane, lane + 64, ..., added in a fixed order
    const int8_t* q8 = reinterpret_cast<const int8_t*>(qrow);
    for (int h = wv; h < H_I; h += IB_NT / 64) {
      float v = 0.f;
      for (int f = lane; f < D_I; f += 64)
        v += static_cast<float>(q8[h * D_I + f]) * ps[h * D_I + f];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) dwr[h] = v;
    }
  }
}

// counts of the valid entries per position (key b*Tk + s); entry e = row*K + t
// of the set is its index rows' entry (b*brow + i)*K + t
__global__ __launch_bounds__(256) void ibwd_count_kernel(int Tq, int Tk, int K, int64_t brow,
                                                         const int32_t* __restrict__ q_offset,
                                                         const int32_t* __restrict__ kv_len,
                                                         const int32_t* __restrict__ idx,
                                                         int64_t nent, int32_t* __restrict__ cnt) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t row = e / K;
    const int b = static_cast<int>(row / Tq);
    const int64_t i = row - static_cast<int64_t>(b) * Tq;
    const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
    const int kvl = kv_len[b];
    const int s = idx[(b * brow + i) * K + (e - row * K)];
    if (kvl <= Tk && p >= 0 && p < kvl && s >= 0 && s <= p)
      atomicAdd(&cnt[static_cast<int64_t>(b) * Tk + s], 1);
  }
}

__global__ __launch_bounds__(256) void ibwd_fill_kernel(int Tq, int Tk, int K, int64_t brow,
                                                        const int32_t* __restrict__ q_offset,
                                                        const int32_t* __restrict__ kv_len,
                                                        const int32_t* __restrict__ idx,
                                                        int64_t nent,
                                                        const int32_t* __restrict__ off,
                                                        int32_t* __restrict__ cursor,
                                                        int32_t* __restrict__ ents,
                                                        int32_t* __restrict__ ekey) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t row = e / K;
    const int b = static_cast<int>(row / Tq);
    const int64_t i = row - static_cast<int64_t>(b) * Tq;
    const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
    const int kvl = kv_len[b];
    const int s = idx[(b * brow + i) * K + (e - row * K)];
    if (kvl <= Tk && p >= 0 && p < kvl && s >= 0 && s <= p) {
      const int64_t key = static_cast<int64_t>(b) * Tk + s;
      const int slot = off[key] + atomicAdd(&cursor[key], 1);
      ents[slot] = static_cast<int32_t>(e);
      ekey[slot] = static_cast<int32_t>(key);
    }
  }
}

// The same count with the counts of a block of rows kept in LDS (one counter
// per position of the sequence: histories up to kIbLdsKeys), so the global
// counters take one atomic per position and block instead of one per entry
// (Prefill 8K: 107 against 205 us). Workgroup (x, b): rows x*IB_TRW ..
// x*IB_TRW + IB_TRW - 1 of sequence b. (The fill done the same way, with one
// global reservation per position and block and the slots handed out in LDS,
// took 467 us against the per-entry atomics' 372.)
constexpr int IB_TRW = 32;
constexpr int kIbLdsKeys = 16384;

// the block's valid entries, one call of f(entry number, position) each
template <typename F>
__device__ __forceinline__ void ibwd_block_entries(int Tq, int Tk, int K, int64_t brow, int b,
                                                   int i0, const int32_t* __restrict__ q_offset,
                                                   const int32_t* __restrict__ kv_len,
                                                   const int32_t* __restrict__ idx, F&& f) {
  const int kvl = kv_len[b];
  if (kvl > Tk) return;
  const int nrows = min(IB_TRW, Tq - i0);
  for (int r = 0; r < nrows; ++r) {
    const int i = i0 + r;
    const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
    if (p < 0 || p >= kvl) continue;  // the row's validity: the same for every thread
    const int32_t* ir = idx + (static_cast<int64_t>(b) * brow + i) * K;
    const int64_t e0 = (static_cast<int64_t>(b) * Tq + i) * K;
    for (int t = threadIdx.x; t < K; t += 256) {
      const int s = ir[t];
      if (s >= 0 && s <= p) f(e0 + t, s);
    }
  }
}

__global__ __launch_bounds__(256) void ibwd_count_lds_kernel(int Tq, int Tk, int K, int64_t brow,
                                                             const int32_t* __restrict__ q_offset,
                                                             const int32_t* __restrict__ kv_len,
                                                             const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ cnt) {
  extern __shared__ uint32_t lc[];  // Tk counters
  const int b = blockIdx.y;
  const int i0 = blockIdx.x * IB_TRW;
  for (int s = threadIdx.x; s < Tk; s += 256) lc[s] = 0u;
  __syncthreads();
  ibwd_block_entries(Tq, Tk, K, brow, b, i0, q_offset, kv_len, idx,
                     [&](int64_t, int s) { atomicAdd(&lc[s], 1u); });
  __syncthreads();
  for (int s = threadIdx.x; s < Tk; s += 256)
    if (lc[s] != 0u) atomicAdd(&cnt[static_cast<int64_t>(b) * Tk + s], static_cast<int32_t>(lc[s]));
}

// Entries grouped by position (the transpose), taken 64 at a time: a wave's
// chunk of the list may span several positions, and a long list spans many
// chunks. Lane k loads the metadata of entry k of the chunk (one coalesced
// pass); then lane j (features j, j + 64) walks the chunk's entries in order,
// EB at a time with every load of the group issued first, adding g_t u_tj
// rounded to 32 fraction bits (exactly: g's mantissa times u in 64 bits, one
// rounding shift) as 64-bit integers; when the position changes, and at the
// end of the chunk, the sums go into the position's accumulator by integer
// atomics. Integer sums do not depend on their order: deterministic.
// Query rows with each feature's heads side by side: qT[row][j] holds
// qI[row, h, j] for the set's heads h = 0 .. H_I-1 (the first at q_idx, rows of
// q_heads heads) as int8 in (H_I + 3) / 4 words (zero padded),
// so the dk kernel reads one feature's heads with one or two dword loads and
// sums them with v_dot4. One thread per (row, feature).
template <int H_I, int D_I>
__global__ __launch_bounds__(256) void ibwd_qt_kernel(int64_t rows, int q_heads,
                                                      const int8_t* __restrict__ q_idx,
                                                      uint32_t* __restrict__ qT) {
  constexpr int NW = (H_I + 3) / 4;
  for (int64_t x = blockIdx.x * 256LL + threadIdx.x; x < rows * D_I; x += gridDim.x * 256LL) {
    const int64_t row = x / D_I;
    const int j = static_cast<int>(x - row * D_I);
    const int8_t* qr = q_idx + row * q_heads * D_I + j;
#pragma unroll
    for (int n = 0; n < NW; ++n) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (4 * n + b < H_I) word |= static_cast<uint32_t>(static_cast<uint8_t>(qr[(4 * n + b) * D_I])) << (8 * b);
      qT[x * NW + n] = word;
    }
  }
}

template <int H_I, int D_I>
__global__ __launch_bounds__(256) void ibwd_dk_kernel(
    int Tq, int K, const uint32_t* __restrict__ qT, const int8_t* __restrict__ w, int64_t wsb,
    int64_t wsq, const int32_t* __restrict__ ents, const int32_t* __restrict__ ekey,
    const float* __restrict__ g_ent, const uint16_t* __restrict__ m_ent,
    unsigned long long* __restrict__ acc_dk, const int32_t* __restrict__ total) {
  constexpr int JL = (D_I + 63) / 64;   // features per lane
  constexpr int NW = (H_I + 3) / 4;     // words of one feature's heads
  const int64_t nlist = *total;         // the valid entries (the count total)
  constexpr int EB = D_I > 64 ? 4 : 8;  // entries per load group
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  // each wave takes SC consecutive entries of the list (64 at a time) and
  // keeps its sums across them: a position's entries are flushed once per
  // wave that holds them, not once per 64
  constexpr int SC = 256;
  for (int64_t s0 = w0 * SC; s0 < nlist; s0 += nw * SC) {
    const int64_t s1 = min<int64_t>(s0 + SC, nlist);
    long long acc[JL];
#pragma unroll
    for (int c = 0; c < JL; ++c) acc[c] = 0;
    int cur = ekey[s0];
    auto flush = [&](int key) {
#pragma unroll
      for (int c = 0; c < JL; ++c) {
        const int j = lane + 64 * c;
        if (j < D_I && acc[c] != 0)
          atomicAdd(acc_dk + static_cast<int64_t>(key) * D_I + j, static_cast<unsigned long long>(acc[c]));
        acc[c] = 0;
      }
    };
    for (int64_t c0 = s0; c0 < s1; c0 += 64) {
      const int n = static_cast<int>(min<int64_t>(64, s1 - c0));
      // this lane's entry of the chunk: its query row, position, the weights of
      // the heads whose ReLU passed it packed like qT's words, and g split as
      // g = mant * 2^(ex - 150) exactly (fp32 bits), so that g*u*2^32 is mant*u
      // (exact in 64 bits) shifted right by 118 - ex, rounded
      int my_row = 0, my_key = -1, my_mant = 0, my_sh = 63;
      uint32_t my_wm[NW];
#pragma unroll
      for (int m = 0; m < NW; ++m) my_wm[m] = 0u;
      if (lane < n) {
        const int e = ents[c0 + lane];
        my_row = e / K;
        my_key = ekey[c0 + lane];
        const int hm = m_ent[e];
        const int b = my_row / Tq;
        const int i = my_row - b * Tq;
        const int8_t* wr = w + b * wsb + static_cast<int64_t>(i) * wsq;
#pragma unroll
        for (int m = 0; m < NW; ++m) {
          uint32_t word = 0;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int hh = 4 * m + bb;
            if (hh < H_I && ((hm >> hh) & 1))
              word |= static_cast<uint32_t>(static_cast<uint8_t>(wr[hh])) << (8 * bb);
          }
          my_wm[m] = word;
        }
        const uint32_t gb = __float_as_uint(g_ent[e]);
        const int ex = static_cast<int>((gb >> 23) & 0xffu);
        my_mant = static_cast<int>(gb & 0x7fffffu) | (ex ? 0x800000 : 0);
        if (gb >> 31) my_mant = -my_mant;
        my_sh = 118 - (ex ? ex : 1);
      }
      for (int k0 = 0; k0 < n; k0 += EB) {
        // the group's entries are the same for every lane: scalar registers
        int rowv[EB], keyv[EB];
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          const int src = min(k0 + k, 63);
          rowv[k] = __builtin_amdgcn_readlane(my_row, src);
          keyv[k] = k0 + k < n ? __builtin_amdgcn_readlane(my_key, src) : -1;
        }
        // feature j's heads of each entry's query row (all loads in flight together)
        uint32_t qv[EB][JL][NW];
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          const uint32_t* qr = qT + static_cast<int64_t>(rowv[k]) * D_I * NW;
#pragma unroll
          for (int c = 0; c < JL; ++c)
#pragma unroll
            for (int m = 0; m < NW; ++m)
              qv[k][c][m] = lane + 64 * c < D_I ? qr[(lane + 64 * c) * NW + m] : 0u;
        }
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          if (keyv[k] < 0) break;  // past the chunk (uniform)
          if (keyv[k] != cur) {   // a new position (uniform)
            flush(cur);
            cur = keyv[k];
          }
          const int src = k0 + k;
          int wm[NW];
#pragma unroll
          for (int m = 0; m < NW; ++m)
            wm[m] = __builtin_amdgcn_readlane(static_cast<int>(my_wm[m]), src);
          const int mant = __builtin_amdgcn_readlane(my_mant, src);
          const int sh = __builtin_amdgcn_readlane(my_sh, src);
#pragma unroll
          for (int c = 0; c < JL; ++c) {
            // u = sum_h w_h [d_h > 0] qI[h, j]: exact int8 dot products
            int u = 0;
#pragma unroll
            for (int m = 0; m < NW; ++m)
              u = __builtin_amdgcn_sdot4(static_cast<int>(qv[k][c][m]), wm[m], u, false);
            const long long prod = static_cast<long long>(mant) * u;
            long long add;
            if (sh <= 0) add = prod << (-sh);
            else if (sh > 62) add = 0;
            else add = (prod + (1ll << (sh - 1))) >> sh;
            acc[c] += add;
          }
        }
      }
    }
    flush(cur);
  }
}

__global__ __launch_bounds__(256) void ibwd_zero_u64_kernel(unsigned long long* __restrict__ p,
                                                            int64_t n) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL) p[i] = 0ull;
}

__global__ __launch_bounds__(256) void ibwd_dk_out_kernel(const unsigned long long* __restrict__ acc,
                                                          float* __restrict__ dk, int64_t n) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL)
    dk[i] = static_cast<float>(static_cast<double>(static_cast<long long>(acc[i])) / kIbFix);
}

// ------------------------------------------------------------------ host side

struct IbwdLayout {
  size_t g, m, cnt, off, cursor, tiles, ents, ekey, acc, qt, total;
};

// g.H_I: the heads of one index set (the sets run one after another and share
// the workspace)
static IbwdLayout ibwd_layout(const Geom& g) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t nent = static_cast<size_t>(g.B) * g.Tq * g.K;
  const size_t keys = static_cast<size_t>(g.B) * g.Tk;
  IbwdLayout L{};
  size_t o = 0;
  L.g = o;      o += al(nent * sizeof(float));
  L.m = o;      o += al(nent * sizeof(uint16_t));
  L.cnt = o;    o += al(keys * sizeof(int32_t));
  L.off = o;    o += al((keys + 1) * sizeof(int32_t));
  L.cursor = o; o += al(keys * sizeof(int32_t));
  L.tiles = o;  o += al(((keys + 1023) / 1024 + 1) * sizeof(int32_t));
  L.ents = o;   o += al(nent * sizeof(int32_t));
  L.ekey = o;   o += al(nent * sizeof(int32_t));
  L.acc = o;    o += al(keys * g.d_I * sizeof(unsigned long long));
  L.qt = o;     o += al(static_cast<size_t>(g.B) * g.Tq * g.d_I * ((g.H_I + 3) / 4) * sizeof(uint32_t));
  L.total = o;
  return L;
}

static Geom ibwd_set_geom(const Geom& g) {
  Geom s = g;
  s.H_I = g.H_I / (g.sets > 1 ? g.sets : 1);
  return s;
}

size_t ibwd_workspace(const Geom& g) { return ibwd_layout(ibwd_set_geom(g)).total; }

__global__ __launch_bounds__(256) void ibwd_fill_i32_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL) p[i] = 0;
}

// g: the geometry of one index set (g.H_I its heads, g.sets the set count);
// set s reads heads s*H_I .. s*H_I + H_I - 1 of rows of H_I*sets heads and
// index rows [B][sets][Tq][K]. The sets run one after another on the stream,
// sharing the workspace; their dk sums meet in one fixed-point accumulator.
template <int H_I, int D_I>
static hipError_t ibwd_launch_hd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                 const int8_t* w, int64_t wsb, int64_t wsq, const int32_t* idx,
                                 const float* teacher, float tau, float* loss, float* dq,
                                 float* dk, float* dw, void* ws, hipStream_t st) {
  const IbwdLayout L = ibwd_layout(g);
  char* base = static_cast<char*>(ws);
  float* g_ent = reinterpret_cast<float*>(base + L.g);
  uint16_t* m_ent = reinterpret_cast<uint16_t*>(base + L.m);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(base + L.off);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + L.cursor);
  int32_t* tiles = reinterpret_cast<int32_t*>(base + L.tiles);
  int32_t* ents = reinterpret_cast<int32_t*>(base + L.ents);
  int32_t* ekey = reinterpret_cast<int32_t*>(base + L.ekey);
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(base + L.acc);
  uint32_t* qt = reinterpret_cast<uint32_t*>(base + L.qt);
  const int ns = g.sets > 1 ? g.sets : 1;
  const int q_heads = H_I * ns;
  const int64_t brow = static_cast<int64_t>(ns) * g.Tq;  // index rows per sequence
  const int64_t keys = static_cast<int64_t>(g.B) * g.Tk;
  const int64_t nent = static_cast<int64_t>(g.B) * g.Tq * g.K;  // entries of one set
  const int64_t rows = static_cast<int64_t>(g.B) * g.Tq;
  const int64_t nacc = keys * g.d_I;
  const uint32_t gk = static_cast<uint32_t>(std::min<int64_t>((keys + 255) / 256, 8192));
  const uint32_t ge = static_cast<uint32_t>(std::min<int64_t>((nent + 255) / 256, 8192));
  const uint32_t ga = static_cast<uint32_t>(std::min<int64_t>((nacc + 255) / 256, 8192));
  const uint32_t gq = static_cast<uint32_t>(std::min<int64_t>((rows * D_I + 255) / 256, 8192));
  // the list holds the valid entries: as many as the count total off[keys];
  // four waves of 256 entries per workgroup
  const uint32_t gd = static_cast<uint32_t>(std::min<int64_t>((nent + 1023) / 1024, 8192));
  const size_t lds = static_cast<size_t>(g.K) * (sizeof(float) + sizeof(int) + sizeof(uint16_t));
  hipError_t e;
  for (int set = 0; set < ns; ++set) {
    const int8_t* qs = q_idx + static_cast<int64_t>(set) * H_I * D_I;
    const int8_t* ws_ = w + set * H_I;
    const int32_t* is = idx + static_cast<int64_t>(set) * g.Tq * g.K;
    const float* ts = teacher + static_cast<int64_t>(set) * g.Tq * g.K;
    float* ls = loss ? loss + static_cast<int64_t>(set) * g.Tq : nullptr;
    float* dqs = dq + static_cast<int64_t>(set) * H_I * D_I;
    float* dws = dw + set * H_I;
    {
      KernelTimer timer(LCI_KERNEL_IBWD, st);
      hipLaunchKernelGGL((ibwd_row_kernel<H_I, D_I>), dim3(static_cast<uint32_t>(rows)),
                         dim3(IB_NT), lds, st, g.Tq, g.Tk, g.K, q_heads, brow, g.q_offset,
                         g.kv_len, qs, k_idx, ws_, wsb, wsq, is, ts, tau, ls, dqs, dws, g_ent,
                         m_ent);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      KernelTimer timer(LCI_KERNEL_IBWD_TRANSPOSE, st);
      hipLaunchKernelGGL(ibwd_fill_i32_kernel, dim3(gk), dim3(256), 0, st, cnt, keys);
      hipLaunchKernelGGL(ibwd_fill_i32_kernel, dim3(gk), dim3(256), 0, st, cursor, keys);
      const bool lds_counts = g.Tk <= kIbLdsKeys;
      const dim3 gb((g.Tq + IB_TRW - 1) / IB_TRW, g.B);
      const size_t lb = static_cast<size_t>(g.Tk) * sizeof(uint32_t);
      if (lds_counts)
        hipLaunchKernelGGL(ibwd_count_lds_kernel, gb, dim3(256), lb, st, g.Tq, g.Tk, g.K, brow,
                           g.q_offset, g.kv_len, is, cnt);
      else
        hipLaunchKernelGGL(ibwd_count_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, brow,
                           g.q_offset, g.kv_len, is, nent, cnt);
      if ((e = launch_exclusive_scan(cnt, keys, off, tiles, st)) != hipSuccess) return e;
      hipLaunchKernelGGL(ibwd_fill_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, brow,
                         g.q_offset, g.kv_len, is, nent, off, cursor, ents, ekey);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      KernelTimer timer(LCI_KERNEL_IBWD_DK, st);
      if (set == 0)
        hipLaunchKernelGGL(ibwd_zero_u64_kernel, dim3(ga), dim3(256), 0, st, acc, nacc);
      hipLaunchKernelGGL((ibwd_qt_kernel<H_I, D_I>), dim3(gq), dim3(256), 0, st, rows, q_heads,
                         qs, qt);
      hipLaunchKernelGGL((ibwd_dk_kernel<H_I, D_I>), dim3(gd), dim3(256), 0, st, g.Tq, g.K, qt,
                         ws_, wsb, wsq, ents, ekey, g_ent, m_ent, acc, off + keys);
      if (set == ns - 1)
        hipLaunchKernelGGL(ibwd_dk_out_kernel, dim3(ga), dim3(256), 0, st, acc, dk, nacc);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int H_I>
static hipError_t ibwd_launch_h(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                const int8_t* w, int64_t wsb, int64_t wsq, const int32_t* idx,
                                const float* teacher, float tau, float* loss, float* dq,
                                float* dk, float* dw, void* ws, hipStream_t st) {
  switch (g.d_I) {
    case 32: return ibwd_launch_hd<H_I, 32>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 64: return ibwd_launch_hd<H_I, 64>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 128:
      if constexpr (H_I * 32 <= IB_NT)
        return ibwd_launch_hd<H_I, 128>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer_bwd(const Geom& gall, const int8_t* q_idx, const int8_t* k_idx,
                              const int8_t* w, int64_t wsb, int64_t wsq, const int32_t* idx,
                              const float* teacher, float tau, float* loss, float* dq, float* dk,
                              float* dw, void* ws, hipStream_t st) {
  const Geom g = ibwd_set_geom(gall);
  switch (g.H_I) {
    case 1: return ibwd_launch_h<1>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 2: return ibwd_launch_h<2>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 4: return ibwd_launch_h<4>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 8: return ibwd_launch_h<8>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    case 16: return ibwd_launch_h<16>(g, q_idx, k_idx, w, wsb, wsq, idx, teacher, tau, loss, dq, dk, dw, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
