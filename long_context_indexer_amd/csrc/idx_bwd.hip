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
//
//   ibwd_zero_kernel   clears the 32.32 fixed-point accumulator of dk.
//   ibwd_row_kernel    one workgroup per query row: the entries' scores from the
//                      int8 rows (v_dot4 over d_I, exact), the softmax of tau*S
//                      and the loss (workgroup reductions in a fixed order), g;
//                      dw reduced in a fixed order; dq by threads that each own a
//                      head and four features and sum the entries in order; dk
//                      contributions g_t * u_t (u_t = sum_h w_h [d_ht > 0] qI[i,h],
//                      an exact integer vector) added to the accumulator as
//                      64-bit integers (32 fraction bits): integer sums do not
//                      depend on their order, so the result is deterministic.
//   ibwd_dk_kernel     accumulator -> fp32 dk.
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"

namespace lci {

constexpr int IB_NT = 256;
constexpr double kIbFix = 4294967296.0;  // 2^32: fraction bits of the dk accumulator

__global__ __launch_bounds__(256) void ibwd_zero_kernel(unsigned long long* __restrict__ acc,
                                                        int64_t n) {
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x)
    acc[j] = 0ull;
}

__global__ __launch_bounds__(256) void ibwd_dk_kernel(const unsigned long long* __restrict__ acc,
                                                      float* __restrict__ dk, int64_t n) {
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dk[j] = static_cast<float>(static_cast<double>(static_cast<long long>(acc[j])) / kIbFix);
}

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

// One workgroup per query row (blockIdx.x = b*Tq + i). Dynamic LDS: K floats of
// g (z first), K 16-bit head masks (bit h: d_ht > 0; 0 for skipped entries).
template <int H_I, int D_I>
__global__ __launch_bounds__(IB_NT) void ibwd_row_kernel(
    int Tq, int Tk, int K, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int8_t* __restrict__ q_idx,
    const int8_t* __restrict__ k_idx, const int8_t* __restrict__ w, int64_t wsb, int64_t wsq,
    const int32_t* __restrict__ idx, const float* __restrict__ teacher, float tau,
    float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw,
    unsigned long long* __restrict__ dk_acc) {
  static_assert(D_I % 16 == 0 && H_I * (D_I / 4) <= IB_NT, "thread mapping of dq");
  constexpr int NW = D_I / 4;  // int8 quads of a row
  static_assert(H_I <= 16, "16-bit head masks");
  extern __shared__ __align__(16) float gz[];  // K floats, then K 16-bit masks
  uint16_t* hmask = reinterpret_cast<uint16_t*>(gz + K);
  __shared__ __align__(16) int qrow[H_I * NW];
  __shared__ float red[IB_NT / 64];
  __shared__ float dwp[IB_NT / 64][H_I];

  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / Tq);
  const int i = static_cast<int>(row % Tq);
  const int kvl0 = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
  const bool rok = kvl0 <= Tk && p >= 0 && p < kvl0;
  float* dqr = dq + row * H_I * D_I;
  float* dwr = dw + row * H_I;
  for (int j = t; j < H_I * D_I; j += IB_NT) dqr[j] = 0.f;
  if (t < H_I) dwr[t] = 0.f;
  if (loss && t == 0) loss[row] = 0.f;
  if (!rok) return;
  const int* qsrc = reinterpret_cast<const int*>(q_idx + row * H_I * D_I);
  for (int j = t; j < H_I * NW; j += IB_NT) qrow[j] = qsrc[j];
  int wh[H_I];
  const int8_t* wr = w + b * wsb + static_cast<int64_t>(i) * wsq;
#pragma unroll
  for (int h = 0; h < H_I; ++h) wh[h] = static_cast<int>(wr[h]);
  __syncthreads();
  const int32_t* ir = idx + row * K;
  const float* Tr = teacher + row * K;
  const int8_t* kb = k_idx + static_cast<int64_t>(b) * Tk * D_I;

  // the entry's head dot products, exact
  auto dots = [&](int s, int (&d)[H_I]) {
    const int4* kr = reinterpret_cast<const int4*>(kb + static_cast<int64_t>(s) * D_I);
    int4 kq[NW / 4];
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) kq[c] = kr[c];
#pragma unroll
    for (int h = 0; h < H_I; ++h) {
      int acc = 0;
#pragma unroll
      for (int c = 0; c < NW / 4; ++c) {
        acc = __builtin_amdgcn_sdot4(qrow[h * NW + 4 * c], kq[c].x, acc, false);
        acc = __builtin_amdgcn_sdot4(qrow[h * NW + 4 * c + 1], kq[c].y, acc, false);
        acc = __builtin_amdgcn_sdot4(qrow[h * NW + 4 * c + 2], kq[c].z, acc, false);
        acc = __builtin_amdgcn_sdot4(qrow[h * NW + 4 * c + 3], kq[c].w, acc, false);
      }
      d[h] = acc;
    }
  };

  // 1. z_t = tau * S_t for the valid entries (-inf for the others), max
  float mloc = -INFINITY;
  for (int e = t; e < K; e += IB_NT) {
    const int s = ir[e];
    float z = -INFINITY;
    uint32_t hm = 0;
    if (s >= 0 && s <= p) {
      int d[H_I];
      dots(s, d);
      int S = 0;
#pragma unroll
      for (int h = 0; h < H_I; ++h) {
        S += wh[h] * max(d[h], 0);
        hm |= (d[h] > 0 ? 1u : 0u) << h;
      }
      z = tau * static_cast<float>(S);
    }
    gz[e] = z;
    hmask[e] = static_cast<uint16_t>(hm);
    mloc = fmaxf(mloc, z);
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
  // 3. loss, g, dw partials and the dk contributions
  float lloc = 0.f;
  float dwl[H_I];
#pragma unroll
  for (int h = 0; h < H_I; ++h) dwl[h] = 0.f;
  unsigned long long* accb = dk_acc + static_cast<int64_t>(b) * Tk * D_I;
  for (int e = t; e < K; e += IB_NT) {
    const float z = gz[e];
    float g = 0.f;
    if (z != -INFINITY) {
      const float logp = z - logZ;
      const float pt = __expf(logp);
      const float te = Tr[e];
      if (te > 0.f) lloc += te * (__logf(te) - logp);
      g = tau * (pt * Tsum - te);
      const int s = ir[e];
      int d[H_I];
      dots(s, d);
#pragma unroll
      for (int h = 0; h < H_I; ++h) dwl[h] += g * static_cast<float>(max(d[h], 0));
      // u = sum_h w_h [d_h > 0] q_h: exact integers; g*u into the accumulator
      const uint32_t hm = hmask[e];
      unsigned long long* ak = accb + static_cast<int64_t>(s) * D_I;
      const double gf = static_cast<double>(g) * kIbFix;
#pragma unroll 4
      for (int j4 = 0; j4 < NW; ++j4) {
        int u[4] = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < H_I; ++h) {
          const int qw = (hm >> h) & 1u ? qrow[h * NW + j4] : 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) u[c] += wh[h] * static_cast<int>(static_cast<int8_t>(qw >> (8 * c)));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (u[c] != 0)
            atomicAdd(ak + 4 * j4 + c,
                      static_cast<unsigned long long>(__double2ll_rn(gf * static_cast<double>(u[c]))));
      }
    }
    gz[e] = g;  // the same thread reads it back for dq after the barrier
  }
  const float L = ib_block_sum(lloc, red);
  if (loss && t == 0) loss[row] = L;
  // dw: per-wave sums, then the waves in order
#pragma unroll
  for (int h = 0; h < H_I; ++h) {
    float v = dwl[h];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((t & 63) == 0) dwp[t >> 6][h] = v;
  }
  __syncthreads();  // g, masks and the dw partials are visible
  if (t < H_I) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < IB_NT / 64; ++wv) v += dwp[wv][t];
    dwr[t] = v;
  }
  // 4. dq: thread (h, j4) of the first H_I*NW sums its head and four features
  // over the entries in order
  if (t < H_I * NW) {
    const int h = t / NW, j4 = t % NW;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int e = 0; e < K; ++e) {
      if (!((hmask[e] >> h) & 1u)) continue;
      const float g = gz[e];
      const int kw = *reinterpret_cast<const int*>(kb + static_cast<int64_t>(ir[e]) * D_I + 4 * j4);
      a0 += g * static_cast<float>(static_cast<int8_t>(kw));
      a1 += g * static_cast<float>(static_cast<int8_t>(kw >> 8));
      a2 += g * static_cast<float>(static_cast<int8_t>(kw >> 16));
      a3 += g * static_cast<float>(static_cast<int8_t>(kw >> 24));
    }
    const float wf = static_cast<float>(wh[h]);
    *reinterpret_cast<float4*>(dqr + h * D_I + 4 * j4) = make_float4(wf * a0, wf * a1, wf * a2, wf * a3);
  }
}

// ------------------------------------------------------------------ host side

size_t ibwd_workspace(const Geom& g) {
  return static_cast<size_t>(g.B) * g.Tk * g.d_I * sizeof(unsigned long long);
}

template <int H_I, int D_I>
static hipError_t ibwd_launch_hd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                                 const int8_t* w, int64_t wsb, int64_t wsq, const int32_t* idx,
                                 const float* teacher, float tau, float* loss, float* dq,
                                 float* dk, float* dw, void* ws, hipStream_t st) {
  unsigned long long* acc = static_cast<unsigned long long*>(ws);
  const int64_t n = static_cast<int64_t>(g.B) * g.Tk * g.d_I;
  const int nb = static_cast<int>(std::min<int64_t>((n + 255) / 256, 8192));
  {
    KernelTimer timer(LCI_KERNEL_IBWD, st);
    hipLaunchKernelGGL(ibwd_zero_kernel, dim3(nb), dim3(256), 0, st, acc, n);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>(g.K) * (sizeof(float) + sizeof(uint16_t));
  {
    KernelTimer timer(LCI_KERNEL_IBWD, st);
    hipLaunchKernelGGL((ibwd_row_kernel<H_I, D_I>), dim3(static_cast<uint32_t>(g.B) * g.Tq),
                       dim3(IB_NT), lds, st, g.Tq, g.Tk, g.K, g.q_offset, g.kv_len, q_idx, k_idx,
                       w, wsb, wsq, idx, teacher, tau, loss, dq, dw, acc);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    KernelTimer timer(LCI_KERNEL_IBWD, st);
    hipLaunchKernelGGL(ibwd_dk_kernel, dim3(nb), dim3(256), 0, st, acc, dk, n);
  }
  return hipGetLastError();
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

hipError_t launch_indexer_bwd(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                              const int8_t* w, int64_t wsb, int64_t wsq, const int32_t* idx,
                              const float* teacher, float tau, float* loss, float* dq, float* dk,
                              float* dw, void* ws, hipStream_t st) {
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
