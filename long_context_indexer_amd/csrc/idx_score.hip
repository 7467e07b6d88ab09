// Indexer scoring on gfx950: int8 MFMA over low-dimensional indexer heads.
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer + Top-K: How
// Fine-Grained Sparse Attention Works", step 1: a light scorer over
// low-dimensional projections rates every history position for each query. The
// arithmetic (a reading; the pages give no formula) is
//   S[b,i,s] = sum_h w[b,i,h] * max(0, qI[b,i,h,:] . kI[b,s,:])   (int8 in, int32 exact)
//
// The contraction over d_I is a dense GEMM: rows = (query, indexer head) pairs,
// columns = history positions. It runs on v_mfma_i32_32x32x32_i8. The 32 MFMA
// rows of one tile hold 32/H_I queries x H_I heads, placed so that every lane's
// 16 accumulators are complete head groups of its column's queries: the ReLU
// and the weighted head sum then run in-lane with no cross-lane traffic.
//
// MFMA row r = 8*i + 4*hf + j (i, j in 0..3, hf in 0..1) is "slot" 4*i + j of
// lane half hf; slot k holds query hf*(16/H_I) + k/H_I, head k%H_I. The output
// element v of lane l is row 8*(v/4) + 4*(l/32) + v%4, i.e. slot v of half l/32,
// for column (history position) l%32.
#include <type_traits>

#include "common.h"
#include "../../include/lci.h"
#include "internal.h"

namespace lci {

template <int H_I, int D_I, int WQ>
__global__ __launch_bounds__(256) void idx_score_kernel(
    int Tq, int Tk, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx,
    const int8_t* __restrict__ w, int64_t wsb, int64_t wsq, int32_t* __restrict__ scores,
    int64_t row_stride, int64_t batch_rows, int q_heads, int row_begin, int row_count,
    int keys_per_wg) {
  constexpr int QW = 32 / H_I;   // query rows per wave tile
  constexpr int QH = 16 / H_I;   // query rows per lane half
  constexpr int NCH = D_I / 32;  // 32-deep MFMA steps over d_I
  constexpr int WK = 4 / WQ;     // waves along the history axis
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wq = wid % WQ, wk = wid / WQ;
  const int b = blockIdx.z;
  const int r0 = (blockIdx.y * WQ + wq) * QW;  // first local row of this wave
  if (r0 >= row_count) return;
  const int qoff = q_offset[b];
  const int kvl = kv_len[b];
  if (kvl > Tk || kvl <= 0) return;  // invalid sequence: nothing is written
  const int row0 = row_begin + r0;
  // last history position any row of this wave may read
  const int pmax = static_cast<int>(min(static_cast<int64_t>(qoff) + row0 + QW - 1,
                                        static_cast<int64_t>(kvl) - 1));
  const int k_begin = blockIdx.x * keys_per_wg;
  const int k_end = min(k_begin + keys_per_wg, pmax + 1);
  if (k_begin >= k_end) return;

  // A operand: lane supplies MFMA row l%32
  v4i a[NCH];
  {
    const int r = lane & 31;
    const int slot = 4 * (r >> 3) + (r & 3);
    const int hf = (r >> 2) & 1;
    const int qa = hf * QH + slot / H_I;
    const int ha = slot % H_I;
    const int lr = r0 + qa;
    const bool ok = lr < row_count && row_begin + lr < Tq;
    // unconditional loads (rows past the end read row begin, then zeroed), so
    // they are all in flight together
    const int lrc = ok ? lr : 0;
    const int8_t* src = q_idx + ((static_cast<int64_t>(b) * Tq + row_begin + lrc) * q_heads + ha) * D_I +
                        16 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const v4i t = *reinterpret_cast<const v4i*>(src + 32 * c);
      const v4i z = {0, 0, 0, 0};
      a[c] = ok ? t : z;
    }
  }
  // weights and positions of this lane's output rows (lane half l/32)
  int wv[16];
  int prow[QH];      // absolute position of each of the lane's rows (-1: no row)
  int64_t orow[QH];  // output row offsets
#pragma unroll
  for (int qq = 0; qq < QH; ++qq) {
    const int lr = r0 + (lane >> 5) * QH + qq;
    const int row = row_begin + lr;
    const bool ok = lr < row_count && row < Tq;
    const int64_t p = static_cast<int64_t>(qoff) + row;
    prow[qq] = (ok && p >= 0 && p < kvl) ? static_cast<int>(p) : -1;
    orow[qq] = (static_cast<int64_t>(b) * batch_rows + lr) * row_stride;
    const int64_t wrow = b * wsb + static_cast<int64_t>(ok ? row : row_begin) * wsq;
#pragma unroll
    for (int h = 0; h < H_I; ++h) {
      const int wt = static_cast<int>(w[wrow + h]);
      wv[qq * H_I + h] = ok ? wt : 0;
    }
  }

  const int8_t* kbase = k_idx + static_cast<int64_t>(b) * Tk * D_I + 16 * (lane >> 5);
  for (int kt = k_begin + wk * 32; kt < k_end; kt += 32 * WK) {
    const int key = kt + (lane & 31);
    // keys past the history read the last valid row; their scores are never stored
    const int keyc = min(key, kvl - 1);
    v4i bf[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      bf[c] = *reinterpret_cast<const v4i*>(kbase + static_cast<int64_t>(keyc) * D_I + 32 * c);
    v16i acc = {};
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c], bf[c], acc, 0, 0, 0);
#pragma unroll
    for (int qq = 0; qq < QH; ++qq) {
      if (key <= prow[qq]) {  // causal: s <= p (also false for rows without a position)
        int s = 0;
#pragma unroll
        for (int h = 0; h < H_I; ++h) s += __mul24(wv[qq * H_I + h], max(acc[qq * H_I + h], 0));
        scores[orow[qq] + key] = s;
      }
    }
  }
}

// Per-head weights shared by every row (the workloads' [H_I] vector). MFMA
// v_mfma_i32_16x16x64_i8 with the 16 history positions of a tile as the A rows
// and 16 query rows as the B columns, one head per MFMA: lane l's 4
// accumulators are positions 4(l/16)+i of query row l%16, so the weighted ReLU
// sum over heads accumulates in place (2 VALU per head per output, no per-row
// weights) and each lane stores 4 consecutive positions of its row at once.
// A wave scores 16 query rows against 2 tiles (32 positions) per step; the key
// fragments of the next step are loaded while this one is scored.
template <int H_I, int D_I>
__global__ __launch_bounds__(256, 5) void idx_score_q16_kernel(
    int Tq, int Tk, const int32_t* __restrict__ q_offset, const int32_t* __restrict__ kv_len,
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx,
    const int8_t* __restrict__ w, int32_t* __restrict__ scores, int64_t row_stride,
    int64_t batch_rows, int q_heads, int row_begin, int row_count, int keys_per_wg) {
  constexpr int NCH = D_I / 64;  // 64-deep MFMA steps over d_I
  constexpr int U = 2;           // 16-position tiles per step
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int b = blockIdx.z;
  const int r0 = (blockIdx.y * 4 + wv) * 16;  // first local row of this wave
  if (r0 >= row_count) return;
  const int qoff = q_offset[b];
  const int kvl = kv_len[b];
  if (kvl > Tk || kvl <= 0) return;  // invalid sequence: nothing is written
  // last history position any row of this wave may read
  const int pmax = static_cast<int>(min(static_cast<int64_t>(qoff) + row_begin + r0 + 15,
                                        static_cast<int64_t>(kvl) - 1));
  const int k_begin = blockIdx.x * keys_per_wg;
  const int k_end = min(k_begin + keys_per_wg, pmax + 1);
  if (k_begin >= k_end) return;

  // B operands: query row r0 + l%16 of every head, k-bytes 16*(l/16) of each step
  const int lr = r0 + (lane & 15);
  const bool rok = lr < row_count && row_begin + lr < Tq;
  v4i bq[H_I][NCH];
  {
    const int lrc = rok ? lr : r0;  // rows past the end read a valid row, then zeroed
    const int8_t* src = q_idx + (static_cast<int64_t>(b) * Tq + row_begin + lrc) * q_heads * D_I +
                        16 * (lane >> 4);
#pragma unroll
    for (int h = 0; h < H_I; ++h)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const v4i t = *reinterpret_cast<const v4i*>(src + h * D_I + 64 * c);
        const v4i z = {0, 0, 0, 0};
        bq[h][c] = rok ? t : z;
      }
  }
  int wh[H_I];
#pragma unroll
  for (int h = 0; h < H_I; ++h) wh[h] = static_cast<int>(w[h]);

  // this lane's row and its causal limit (-1: the row has no position)
  const int64_t p64 = static_cast<int64_t>(qoff) + row_begin + lr;
  const int plim = (rok && p64 >= 0 && p64 < kvl) ? static_cast<int>(p64) : -1;
  int32_t* orow = scores + (static_cast<int64_t>(b) * batch_rows + (rok ? lr : r0)) * row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && (row_stride & 3) == 0;

  const int8_t* kbase = k_idx + static_cast<int64_t>(b) * Tk * D_I + 16 * (lane >> 4);
  auto load_keys = [&](int kt, v4i (&dst)[U][NCH]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // past the history: a valid row, whose scores are never stored
      const int keyc = min(kt + 16 * u + (lane & 15), kvl - 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        dst[u][c] = *reinterpret_cast<const v4i*>(kbase + static_cast<int64_t>(keyc) * D_I + 64 * c);
    }
  };
  v4i ka[U][NCH];
  load_keys(k_begin, ka);
  for (int kt = k_begin; kt < k_end; kt += 16 * U) {
    v4i kn[U][NCH];
    load_keys(kt + 16 * U, kn);  // next step (clamped reads past the end are unused)
    v4i sacc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sacc[u] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < H_I; ++h)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka[u][c], bq[h][c], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[u][i] += __mul24(wh[h], max(acc[i], 0));
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = kt + 16 * u + 4 * (lane >> 4);  // first of this lane's 4 positions
      if (vec && key + 3 <= plim) {
        *reinterpret_cast<v4i*>(orow + key) = sacc[u];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key + i <= plim) orow[key + i] = sacc[u][i];  // causal: s <= p
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c) ka[u][c] = kn[u][c];
  }
}

template <int H_I, int D_I>
static hipError_t launch_hd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                            const int8_t* w, int64_t wsb, int64_t wsq, int32_t* scores,
                            int64_t stride, int64_t brows, int qh, int row_begin, int row_count,
                            hipStream_t st) {
  constexpr int QW = 32 / H_I;
  if constexpr (D_I >= 64 && H_I * D_I <= 512) {
    if (wsb == 0 && wsq == 0 && row_count >= 64) {
      // shared head weights, many rows: 4 waves x 16 rows, 128 positions per
      // workgroup (short workgroups, 5 waves per SIMD: the scoring is latency
      // bound; on Prefill 8K 128 beat 64, 256 and 512)
      const int keys = 128;
      dim3 grid((g.Tk + keys - 1) / keys, (row_count + 63) / 64, g.B);
      KernelTimer timer(LCI_KERNEL_IDX_SCORE, st);
      hipLaunchKernelGGL((idx_score_q16_kernel<H_I, D_I>), grid, dim3(256), 0, st, g.Tq, g.Tk,
                         g.q_offset, g.kv_len, q_idx, k_idx, w, scores, stride, brows, qh,
                         row_begin, row_count, keys);
      return hipGetLastError();
    }
  }
  if (row_count >= 4 * QW) {
    // many query rows: 4 waves on 4 row tiles share each key tile
    const int keys = 256;
    dim3 grid((g.Tk + keys - 1) / keys, (row_count + 4 * QW - 1) / (4 * QW), g.B);
    {
      KernelTimer timer(LCI_KERNEL_IDX_SCORE, st);
      hipLaunchKernelGGL((idx_score_kernel<H_I, D_I, 4>), grid, dim3(256), 0, st, g.Tq, g.Tk,
                         g.q_offset, g.kv_len, q_idx, k_idx, w, wsb, wsq, scores, stride,
                         brows, qh, row_begin, row_count, keys);
    }
  } else {
    // few query rows (decode): the 4 waves split the history
    const int keys = 1024;
    dim3 grid((g.Tk + keys - 1) / keys, (row_count + QW - 1) / QW, g.B);
    {
      KernelTimer timer(LCI_KERNEL_IDX_SCORE, st);
      hipLaunchKernelGGL((idx_score_kernel<H_I, D_I, 1>), grid, dim3(256), 0, st, g.Tq, g.Tk,
                         g.q_offset, g.kv_len, q_idx, k_idx, w, wsb, wsq, scores, stride,
                         brows, qh, row_begin, row_count, keys);
    }
  }
  return hipGetLastError();
}

template <int H_I>
static hipError_t launch_h(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                           const int8_t* w, int64_t wsb, int64_t wsq, int32_t* scores,
                           int64_t stride, int64_t brows, int qh, int row_begin, int row_count,
                           hipStream_t st) {
  switch (g.d_I) {
    case 32: return launch_hd<H_I, 32>(g, q_idx, k_idx, w, wsb, wsq, scores, stride, brows, qh, row_begin, row_count, st);
    case 64: return launch_hd<H_I, 64>(g, q_idx, k_idx, w, wsb, wsq, scores, stride, brows, qh, row_begin, row_count, st);
    case 128:
      if constexpr (H_I * 128 <= 1024)
        return launch_hd<H_I, 128>(g, q_idx, k_idx, w, wsb, wsq, scores, stride, brows, qh, row_begin, row_count, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_idx_score(const Geom& g, const int8_t* q_idx, int q_heads,
                            const int8_t* k_idx, const int8_t* w, int64_t wsb, int64_t wsq,
                            int32_t* scores, int64_t stride, int64_t batch_rows, int row_begin,
                            int row_count, hipStream_t st) {
  auto go = [&](auto heads) {
    return launch_h<decltype(heads)::value>(g, q_idx, k_idx, w, wsb, wsq, scores, stride,
                                            batch_rows, q_heads, row_begin, row_count, st);
  };
  switch (g.H_I) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 4: return go(std::integral_constant<int, 4>{});
    case 8: return go(std::integral_constant<int, 8>{});
    case 16: return go(std::integral_constant<int, 16>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
