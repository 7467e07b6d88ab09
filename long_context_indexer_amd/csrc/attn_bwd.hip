// Gradients of the gated sparse attention (gfx950): dq, dk, dv, dgate, dmix.
//
// The training direction of the layer ("Hybrid Sparse Attention for
// Long-Context LLMs", section "Engineering and Evaluation Recommendations",
// training side): for the forward o = softmax(scale q.k_S) v_S over the
// selected positions S of each row and y = s*o + (1 - s)*x, s = sigmoid(G),
// the chain rule gives
//   do = s*dy, dG = dy*(o - x)*s*(1 - s), dx = (1 - s)*dy,
//   dP_t = do.v_t, delta = sum_t P_t dP_t = do.o, dl_t = P_t (dP_t - delta),
//   dq = scale sum_t dl_t k_t, dk_t += scale dl_t q, dv_t += P_t do.
// Kernels, on the caller's stream:
//   (forward)        the attention without gate recomputes o (bf16) and lse;
//   bwd_prologue     per (row, head): do (stored as bf16: the two passes below
//                    read it once per selected pair), delta (from the fp32 do),
//                    dgate, dmix;
//   bwd_dq           one wave per (row, key/value head g): lanes are (query head
//                    of the group, feature slice), so the dot products of a
//                    selected key with every head of the group are lane-local
//                    sums plus a reduction over the lanes of one head; P is
//                    recomputed from q, k and lse; dq accumulates lane-locally;
//   key transpose    counts per position (integer atomics), an exclusive scan,
//                    and a fill of the rows that selected each position;
//   bwd_dkdv         one wave per (position, key/value head): the rows that
//                    selected it, in any order, each contributing to dk and dv
//                    in 32.32 fixed point (int64): integer sums do not depend on
//                    the order, so dk and dv are deterministic bit for bit.
#include <algorithm>

#include "../../include/lci.h"
#include "attn_dense.h"
#include "common.h"
#include "internal.h"

namespace lci {

namespace {

constexpr float kFix = 4294967296.0f;  // 2^32: the fixed-point scale of dk, dv

// F consecutive bf16 -> float (16-byte loads where F allows)
template <int F>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float (&x)[F]) {
  if constexpr (F >= 8) {
#pragma unroll
    for (int c = 0; c < F / 8; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = bf16_to_f32(static_cast<uint16_t>(w[e]));
        x[8 * c + 2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w[e] >> 16));
      }
    }
  } else if constexpr (F == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_to_f32(static_cast<uint16_t>(u.x));
    x[1] = bf16_to_f32(static_cast<uint16_t>(u.x >> 16));
    x[2] = bf16_to_f32(static_cast<uint16_t>(u.y));
    x[3] = bf16_to_f32(static_cast<uint16_t>(u.y >> 16));
  } else if constexpr (F == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    x[0] = bf16_to_f32(static_cast<uint16_t>(u));
    x[1] = bf16_to_f32(static_cast<uint16_t>(u >> 16));
  } else {
    x[0] = bf16_to_f32(p[0]);
  }
}

// sum over the L consecutive lanes of one head (L a power of two)
template <int L>
__device__ __forceinline__ float head_sum(float v) {
#pragma unroll
  for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// do, delta, dgate, dmix: one wave per (row, head), D/64 features per lane
template <int D>
__global__ __launch_bounds__(256) void bwd_prologue_kernel(
    int64_t nrh, const uint16_t* __restrict__ o, const uint16_t* __restrict__ dy,
    const uint16_t* __restrict__ gate, const uint16_t* __restrict__ mix,
    uint16_t* __restrict__ dO, float* __restrict__ delta, float* __restrict__ dgate,
    float* __restrict__ dmix) {
  constexpr int F = D / 64;
  const int64_t rh = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (rh >= nrh) return;
  const int lane = threadIdx.x & 63;
  const int64_t base = rh * D + lane * F;
  float ov[F], gy[F];
  load_bf16<F>(o + base, ov);
  load_bf16<F>(dy + base, gy);
  float acc = 0.f;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float d_o = gy[f];
    if (gate) {
      const float s = sigmoidf(bf16_to_f32(gate[base + f]));
      const float x = mix ? bf16_to_f32(mix[base + f]) : 0.f;
      d_o = s * gy[f];
      if (dgate) dgate[base + f] = gy[f] * (ov[f] - x) * s * (1.f - s);
      if (dmix) dmix[base + f] = (1.f - s) * gy[f];
    }
    dO[base + f] = f32_to_bf16(d_o);
    acc += d_o * ov[f];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) delta[rh] = acc;
}

// dq: one wave per (row, key/value head g); lane = (head hl of the group, slice sl)
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    int Tq, int Tk, int K, int Hq, int Hkv, const int32_t* __restrict__ kv_len,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const uint16_t* __restrict__ dO,
    const float* __restrict__ delta, float scale, float* __restrict__ dq, int64_t nwaves) {
  constexpr int L = 64 / G;  // lanes per head
  constexpr int F = D / L;   // features per lane
  const int64_t wv = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (wv >= nwaves) return;
  const int lane = threadIdx.x & 63;
  const int hl = lane / L, sl = lane % L;
  const int g = static_cast<int>(wv % Hkv);
  const int64_t row = wv / Hkv;
  const int b = static_cast<int>(row / Tq);
  const int h = g * G + hl;
  const int64_t rh = row * Hq + h;
  const int kvl0 = kv_len[b];
  const int kvl = kvl0 <= Tk ? kvl0 : 0;
  float qv[F], dov[F], acc[F];
  load_bf16<F>(q + rh * D + sl * F, qv);
  load_bf16<F>(dO + rh * D + sl * F, dov);
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
  const float l2 = lse[rh] * LOG2E;  // -inf for a row without entries: no entry is valid then
  const float dlt = delta[rh];
  const float sl2 = scale * LOG2E;
  const int32_t* ir = idx + row * K;
  const int64_t rowstep = static_cast<int64_t>(Hkv) * D;
  const uint16_t* kb = k + (static_cast<int64_t>(b) * Tk * Hkv + g) * D + sl * F;
  const uint16_t* vb = v + (static_cast<int64_t>(b) * Tk * Hkv + g) * D + sl * F;
  constexpr int U = 4;  // entries in flight
  for (int t0 = 0; t0 < K; t0 += U) {
    int sv[U];
    float kx[U][F], vx[U][F];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = t0 + u < K ? ir[t0 + u] : -1;
      sv[u] = s >= 0 && s < kvl ? s : -1;
      const int ss = sv[u] < 0 ? 0 : sv[u];  // invalid entries read row 0 and are dropped
      load_bf16<F>(kb + ss * rowstep, kx[u]);
      load_bf16<F>(vb + ss * rowstep, vx[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        sdot += qv[f] * kx[u][f];
        pdot += dov[f] * vx[u][f];
      }
      sdot = head_sum<L>(sdot);
      pdot = head_sum<L>(pdot);
      if (sv[u] < 0) continue;
      const float p = fast_exp2(sdot * sl2 - l2);
      const float ds = p * (pdot - dlt);
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] += ds * kx[u][f];
    }
  }
#pragma unroll
  for (int f = 0; f < F; ++f) dq[rh * D + sl * F + f] = scale * acc[f];
}

// ---- the transpose of the index rows: for each position, the rows that selected it

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL) p[i] = v;
}

__global__ __launch_bounds__(256) void bwd_count_kernel(int Tq, int Tk, int K,
                                                        const int32_t* __restrict__ kv_len,
                                                        const int32_t* __restrict__ idx,
                                                        int64_t nent, int32_t* __restrict__ cnt) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t row = e / K;
    const int b = static_cast<int>(row / Tq);
    const int kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
    const int s = idx[e];
    if (s >= 0 && s < kvl) atomicAdd(&cnt[static_cast<int64_t>(b) * Tk + s], 1);
  }
}

// exclusive scan of n counts in tiles of 1024 (4 per thread): local scan and tile totals
__global__ __launch_bounds__(256) void scan_tiles_kernel(const int32_t* __restrict__ in, int64_t n,
                                                         int32_t* __restrict__ out,
                                                         int32_t* __restrict__ tiles) {
  __shared__ uint32_t scratch[256 / 64 + 2];
  const int64_t base = blockIdx.x * 1024LL + threadIdx.x * 4;
  int32_t x[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = base + e < n ? in[base + e] : 0;
  const uint32_t sum = static_cast<uint32_t>(x[0] + x[1] + x[2] + x[3]);
  uint32_t tot;
  uint32_t run = block_excl_scan(sum, scratch, &tot);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (base + e < n) out[base + e] = static_cast<int32_t>(run);
    run += static_cast<uint32_t>(x[e]);
  }
  if (threadIdx.x == 0) tiles[blockIdx.x] = static_cast<int32_t>(tot);
}

// exclusive scan of the tile totals (one workgroup, any count) and the grand total at [ntiles]
__global__ __launch_bounds__(1024) void scan_totals_kernel(int32_t* __restrict__ tiles, int ntiles) {
  __shared__ uint32_t scratch[1024 / 64 + 2];
  uint32_t carry = 0;
  for (int t0 = 0; t0 < ntiles; t0 += 1024) {
    const int t = t0 + static_cast<int>(threadIdx.x);
    const uint32_t v = t < ntiles ? static_cast<uint32_t>(tiles[t]) : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, scratch, &tot);
    if (t < ntiles) tiles[t] = static_cast<int32_t>(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) tiles[ntiles] = static_cast<int32_t>(carry);
}

__global__ __launch_bounds__(256) void scan_add_kernel(int32_t* __restrict__ out, int64_t n,
                                                       const int32_t* __restrict__ tiles,
                                                       int ntiles) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i <= n; i += gridDim.x * 256LL)
    out[i] = i < n ? out[i] + tiles[i / 1024] : tiles[ntiles];
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(int Tq, int Tk, int K,
                                                       const int32_t* __restrict__ kv_len,
                                                       const int32_t* __restrict__ idx,
                                                       int64_t nent,
                                                       const int32_t* __restrict__ off,
                                                       int32_t* __restrict__ cursor,
                                                       int32_t* __restrict__ rows) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t row = e / K;
    const int b = static_cast<int>(row / Tq);
    const int kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
    const int s = idx[e];
    if (s >= 0 && s < kvl) {
      const int64_t key = static_cast<int64_t>(b) * Tk + s;
      rows[off[key] + atomicAdd(&cursor[key], 1)] = static_cast<int32_t>(row);
    }
  }
}

// dk, dv: one wave per (position, key/value head g); lane = (head hl, slice sl)
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    int Hq, int Hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows, float scale, float* __restrict__ dk,
    float* __restrict__ dv, int64_t nwaves) {
  constexpr int L = 64 / G;
  constexpr int F = D / L;
  const int lane = threadIdx.x & 63;
  const int hl = lane / L, sl = lane % L;
  const float sl2 = scale * LOG2E;
  for (int64_t wv = blockIdx.x * 4LL + (threadIdx.x >> 6); wv < nwaves; wv += gridDim.x * 4LL) {
    const int g = static_cast<int>(wv % Hkv);
    const int64_t key = wv / Hkv;  // b*Tk + s: the row of k, v, dk, dv
    const int64_t kvrow = (key * Hkv + g) * D + sl * F;
    const int r0 = off[key], r1 = off[key + 1];
    long long ak[F], av[F];
#pragma unroll
    for (int f = 0; f < F; ++f) ak[f] = av[f] = 0;
    if (r1 > r0) {
      float kx[F], vx[F];
      load_bf16<F>(k + kvrow, kx);
      load_bf16<F>(v + kvrow, vx);
      constexpr int U = 2;  // rows in flight
      for (int j0 = r0; j0 < r1; j0 += U) {
        float qx[U][F], dx[U][F], l2[U], dl[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          ok[u] = j0 + u < r1;
          const int64_t row = rows[ok[u] ? j0 + u : r0];
          const int64_t rh = row * Hq + g * G + hl;
          load_bf16<F>(q + rh * D + sl * F, qx[u]);
          load_bf16<F>(dO + rh * D + sl * F, dx[u]);
          l2[u] = lse[rh] * LOG2E;
          dl[u] = delta[rh];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float sdot = 0.f, pdot = 0.f;
#pragma unroll
          for (int f = 0; f < F; ++f) {
            sdot += qx[u][f] * kx[f];
            pdot += dx[u][f] * vx[f];
          }
          sdot = head_sum<L>(sdot);
          pdot = head_sum<L>(pdot);
          if (!ok[u]) continue;
          const float p = fast_exp2(sdot * sl2 - l2[u]);
          const float ds = scale * p * (pdot - dl[u]);
#pragma unroll
          for (int f = 0; f < F; ++f) {
            av[f] += __float2ll_rn(p * dx[u][f] * kFix);
            ak[f] += __float2ll_rn(ds * qx[u][f] * kFix);
          }
        }
      }
    }
    // the heads of the group: lanes with the same slice
#pragma unroll
    for (int o = L; o < 64; o <<= 1) {
#pragma unroll
      for (int f = 0; f < F; ++f) {
        ak[f] += __shfl_xor(ak[f], o, 64);
        av[f] += __shfl_xor(av[f], o, 64);
      }
    }
    if (hl == 0) {
#pragma unroll
      for (int f = 0; f < F; ++f) {
        dk[kvrow + f] = static_cast<float>(static_cast<double>(ak[f]) * (1.0 / 4294967296.0));
        dv[kvrow + f] = static_cast<float>(static_cast<double>(av[f]) * (1.0 / 4294967296.0));
      }
    }
  }
}

template <int D, int G>
hipError_t launch_bwd_dg(const Geom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* idx, const float* lse, const uint16_t* dO, const float* dlt,
                         const int32_t* off, const int32_t* rows, float scale, float* dq,
                         float* dk, float* dv, hipStream_t st) {
  const int64_t nrow_w = static_cast<int64_t>(g.B) * g.Tq * g.Hkv;
  {
    KernelTimer timer(LCI_KERNEL_BWD_DQ, st);
    hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3(static_cast<uint32_t>((nrow_w + 3) / 4)),
                       dim3(256), 0, st, g.Tq, g.Tk, g.K, g.Hq, g.Hkv, g.kv_len, q, k, v, idx,
                       lse, dO, dlt, scale, dq, nrow_w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nkey_w = static_cast<int64_t>(g.B) * g.Tk * g.Hkv;
  {
    KernelTimer timer(LCI_KERNEL_BWD_DKDV, st);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>),
                       dim3(static_cast<uint32_t>(std::min<int64_t>((nkey_w + 3) / 4, 1 << 16))),
                       dim3(256), 0, st, g.Hq, g.Hkv, q, k, v, lse, dO, dlt, off, rows,
                       scale, dk, dv, nkey_w);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const Geom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* idx, const float* lse, const uint16_t* dO, const float* dlt,
                        const int32_t* off, const int32_t* rows, float scale, float* dq,
                        float* dk, float* dv, hipStream_t st) {
  switch (g.Hq / g.Hkv) {
    case 1: return launch_bwd_dg<D, 1>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    case 2: return launch_bwd_dg<D, 2>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    case 4: return launch_bwd_dg<D, 4>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    case 8: return launch_bwd_dg<D, 8>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    case 16: return launch_bwd_dg<D, 16>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// [forward workspace][o bf16][lse][do][delta][counts][offsets (+1)][cursors][tiles (+1)][rows]
BwdLayout bwd_layout(const Geom& g) {
  BwdLayout L{};
  const size_t rows = static_cast<size_t>(g.B) * g.Tq;
  const size_t keys = static_cast<size_t>(g.B) * g.Tk;
  L.splits = sparse_attn_pick_splits(g);
  L.fwd = 0;
  L.o = L.fwd + align256(sparse_attn_workspace(g, L.splits));
  L.lse = L.o + align256(rows * g.Hq * g.d * sizeof(uint16_t));
  L.dO = L.lse + align256(rows * g.Hq * sizeof(float));
  L.delta = L.dO + align256(rows * g.Hq * g.d * sizeof(uint16_t));
  L.cnt = L.delta + align256(rows * g.Hq * sizeof(float));
  L.off = L.cnt + align256(keys * sizeof(int32_t));
  L.cursor = L.off + align256((keys + 1) * sizeof(int32_t));
  L.tiles = L.cursor + align256(keys * sizeof(int32_t));
  L.ntiles = static_cast<int>((keys + 1023) / 1024);
  L.rows = L.tiles + align256((L.ntiles + 1) * sizeof(int32_t));
  L.total = L.rows + align256(rows * g.K * sizeof(int32_t));
  return L;
}

hipError_t launch_sparse_attn_bwd(const Geom& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                                  const uint16_t* mix, const uint16_t* dy, float scale, float* dq,
                                  float* dk, float* dv, float* dgate, float* dmix, void* workspace,
                                  hipStream_t st) {
  const BwdLayout L = bwd_layout(g);
  char* ws = static_cast<char*>(workspace);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + L.o);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  uint16_t* dO = reinterpret_cast<uint16_t*>(ws + L.dO);
  float* dlt = reinterpret_cast<float*>(ws + L.delta);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  // o and lse of the ungated attention
  hipError_t e = launch_sparse_attn(g, q, k, v, idx, nullptr, nullptr, scale, o, lse, L.splits,
                                    ws + L.fwd, false, st);
  if (e != hipSuccess) return e;
  const int64_t nrh = static_cast<int64_t>(g.B) * g.Tq * g.Hq;
  {
    KernelTimer timer(LCI_KERNEL_BWD_PROLOGUE, st);
    if (g.d == 64)
      hipLaunchKernelGGL(bwd_prologue_kernel<64>, dim3(static_cast<uint32_t>((nrh + 3) / 4)),
                         dim3(256), 0, st, nrh, o, dy, gate, mix, dO, dlt, dgate, dmix);
    else
      hipLaunchKernelGGL(bwd_prologue_kernel<128>, dim3(static_cast<uint32_t>((nrh + 3) / 4)),
                         dim3(256), 0, st, nrh, o, dy, gate, mix, dO, dlt, dgate, dmix);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the rows that selected each position
  const int64_t keys = static_cast<int64_t>(g.B) * g.Tk;
  const int64_t nent = static_cast<int64_t>(g.B) * g.Tq * g.K;
  const uint32_t gk = static_cast<uint32_t>(std::min<int64_t>((keys + 255) / 256, 8192));
  const uint32_t ge = static_cast<uint32_t>(std::min<int64_t>((nent + 255) / 256, 8192));
  {
    KernelTimer timer(LCI_KERNEL_BWD_TRANSPOSE, st);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(gk), dim3(256), 0, st, cnt, keys, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(gk), dim3(256), 0, st, cursor, keys, 0);
    hipLaunchKernelGGL(bwd_count_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, g.kv_len,
                       idx, nent, cnt);
    hipLaunchKernelGGL(scan_tiles_kernel, dim3(static_cast<uint32_t>(L.ntiles)), dim3(256), 0, st,
                       cnt, keys, off, tiles);
    hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(1024), 0, st, tiles, L.ntiles);
    hipLaunchKernelGGL(scan_add_kernel, dim3(gk), dim3(256), 0, st, off, keys, tiles, L.ntiles);
    hipLaunchKernelGGL(bwd_fill_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, g.kv_len,
                       idx, nent, off, cursor, rows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (g.d) {
    case 64: return launch_bwd_d<64>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    case 128: return launch_bwd_d<128>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
