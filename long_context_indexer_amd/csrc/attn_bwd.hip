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
//                    with one split it runs the masked-tile kernel, whose row
//                    masks and per-token-block done bytes route each block of
//                    rows to the tile kernels below or to the gather kernels;
//   bwd_prologue     per (row, head): do (stored as bf16), delta (from that bf16
//                    do, as dP below), dgate, dmix;
//   tile path        bwd_dq_tile (query-major, the forward's tile structure) and
//                    bwd_dkdv_tile (key-major: 64 keys per workgroup walking the
//                    row tiles that can see them, in chunks summed in order by
//                    bwd_part_sum): MFMA products over 64-key or 32-row tiles,
//                    P and dS under each row's selection mask;
//   gather path      bwd_dq: one wave per (row, key/value head g), lanes (query
//                    head of the group, feature slice), P recomputed from q, k
//                    and lse; the key transpose (counts per position, an
//                    exclusive scan, a fill of the selecting rows) over the
//                    gather rows only; bwd_dkdv: one wave per (position,
//                    key/value head) over those rows, in 32.32 fixed point
//                    (int64), added to the tile path's dk, dv.
// With several index sets (query head h reads set h / (Hq/sets)) every row
// takes the gather kernels, the position lists are per set, and a dk/dv wave
// walks the lists of every set its key/value head's query heads read.
// Every sum runs in a fixed order or in integers: dq, dk, dv are deterministic
// bit for bit.
#include <algorithm>

#include "../../include/lci.h"
#include "attn_dense.h"
#include "common.h"
#include "internal.h"
#include "tile.h"

namespace lci {

namespace {

constexpr float kFix = 4294967296.0f;  // 2^32: the fixed-point scale of dk, dv

// F consecutive bf16 -> float (16-byte loads where F allows)
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kBwdChunks = 8;
constexpr int kDkdvKeys = 64;              // keys per workgroup of the key-major tile kernel
constexpr int kDkdvThreads = 2 * kDkdvKeys * 2;  // two waves per 32 keys
constexpr size_t kBwdPartMax = size_t(1) << 30;

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
    // delta from the bf16 do the passes below use for dP = do.v, so that
    // sum_t P_t (dP_t - delta) stays at the rounding of o: a row with one
    // entry (P = 1, o = v) then gets dq = 0, as it should
    const uint16_t dob = f32_to_bf16(d_o);
    dO[base + f] = dob;
    acc += bf16_to_f32(dob) * ov[f];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) delta[rh] = acc;
}

// dq: one wave per (row, unit of G query heads that read one key/value head and
// one index set: a key/value head's heads, or an index set's when there are
// more sets than key/value heads); lane = (head hl of the unit, slice sl).
// Gkv: query heads per key/value head; S: index sets (rows [B][S][Tq][K]).
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    int Tq, int Tk, int K, int Hq, int Hkv, int Gkv, int units, int S,
    const int32_t* __restrict__ kv_len,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const uint16_t* __restrict__ dO,
    const float* __restrict__ delta, float scale, float* __restrict__ dq, int64_t nwaves,
    const uint8_t* __restrict__ done, int dbq) {
  constexpr int L = 64 / G;  // lanes per head
  constexpr int F = D / L;   // features per lane
  const int64_t wv = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (wv >= nwaves) return;
  const int lane = threadIdx.x & 63;
  const int hl = lane / L, sl = lane % L;
  const int h0 = static_cast<int>(wv % units) * G;  // the unit's first query head
  const int g = h0 / Gkv;                           // its key/value head
  const int sg = h0 / (Hq / S);                     // its index set
  const int64_t row = wv / units;
  const int b = static_cast<int>(row / Tq);
  const int i = static_cast<int>(row % Tq);
  if (done) {
    // rows of token blocks the tile kernel takes are written there
    if (done[(static_cast<int64_t>(b) * S + sg) * ((Tq + dbq - 1) / dbq) + i / dbq]) return;
  }
  const int h = h0 + hl;
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
  const int32_t* ir = idx + ((static_cast<int64_t>(b) * S + sg) * Tq + i) * K;
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

// a row of a token block the tile kernels take (done non-null: blocks of dbq tokens)
__device__ __forceinline__ bool tile_row(int64_t row, int b, int Tq, const uint8_t* done, int dbq) {
  if (!done) return false;
  const int i = static_cast<int>(row - static_cast<int64_t>(b) * Tq);
  return done[static_cast<int64_t>(b) * ((Tq + dbq - 1) / dbq) + i / dbq] != 0;
}

// index rows [B][S][Tq][K]; the lists are per (sequence, set, position):
// list (b*S + set)*Tk + s holds query rows b*Tq + i (done bytes only with S = 1)
__global__ __launch_bounds__(256) void bwd_count_kernel(int Tq, int Tk, int K, int S,
                                                        const int32_t* __restrict__ kv_len,
                                                        const int32_t* __restrict__ idx,
                                                        int64_t nent, int32_t* __restrict__ cnt,
                                                        const uint8_t* __restrict__ done, int dbq) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t vr = e / K;  // (b*S + set)*Tq + i
    const int b = static_cast<int>(vr / (static_cast<int64_t>(S) * Tq));
    if (tile_row(vr, b, Tq, done, dbq)) continue;
    const int kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
    const int s = idx[e];
    if (s >= 0 && s < kvl) atomicAdd(&cnt[(vr / Tq) * Tk + s], 1);
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

__global__ __launch_bounds__(256) void bwd_fill_kernel(int Tq, int Tk, int K, int S,
                                                       const int32_t* __restrict__ kv_len,
                                                       const int32_t* __restrict__ idx,
                                                       int64_t nent,
                                                       const int32_t* __restrict__ off,
                                                       int32_t* __restrict__ cursor,
                                                       int32_t* __restrict__ rows,
                                                       const uint8_t* __restrict__ done, int dbq) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < nent; e += gridDim.x * 256LL) {
    const int64_t vr = e / K;  // (b*S + set)*Tq + i
    const int b = static_cast<int>(vr / (static_cast<int64_t>(S) * Tq));
    if (tile_row(vr, b, Tq, done, dbq)) continue;
    const int kvl = kv_len[b] <= Tk ? kv_len[b] : 0;
    const int s = idx[e];
    if (s >= 0 && s < kvl) {
      const int64_t key = (vr / Tq) * Tk + s;
      rows[off[key] + atomicAdd(&cursor[key], 1)] =
          static_cast<int32_t>(static_cast<int64_t>(b) * Tq + vr % Tq);
    }
  }
}

// dk, dv: one wave per (position, key/value head g); lane = (head hl, slice sl).
// The G heads of g read index sets s0 .. s0 + nsg - 1 (query head h reads set
// h / (Hq/S)); the wave walks each set's list of rows in set order, a lane
// counting the rows of its own head's set.
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    int Tk, int Hq, int Hkv, int S, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lse, const uint16_t* __restrict__ dO,
    const float* __restrict__ delta, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows, float scale, float* __restrict__ dk,
    float* __restrict__ dv, int64_t nwaves, int add) {
  constexpr int L = 64 / G;
  constexpr int F = D / L;
  const int lane = threadIdx.x & 63;
  const int hl = lane / L, sl = lane % L;
  const float sl2 = scale * LOG2E;
  const int hps = Hq / S;  // query heads per index set
  for (int64_t wv = blockIdx.x * 4LL + (threadIdx.x >> 6); wv < nwaves; wv += gridDim.x * 4LL) {
    const int g = static_cast<int>(wv % Hkv);
    const int64_t key = wv / Hkv;  // b*Tk + s: the row of k, v, dk, dv
    const int64_t kvrow = (key * Hkv + g) * D + sl * F;
    const int64_t b = key / Tk;
    const int64_t spos = key - b * Tk;
    const int s0 = g * G / hps;
    const int nsg = G > hps ? G / hps : 1;
    const int hset = (g * G + hl) / hps;  // this lane's head's set
    int nrows = 0;
    for (int j = 0; j < nsg; ++j) {
      const int64_t lk = (b * S + s0 + j) * Tk + spos;
      nrows += off[lk + 1] - off[lk];
    }
    // add mode: the tile kernel wrote every key; only keys with listed rows change
    if (add && nrows == 0) continue;
    long long ak[F], av[F];
#pragma unroll
    for (int f = 0; f < F; ++f) ak[f] = av[f] = 0;
    if (nrows > 0) {
      float kx[F], vx[F];
      load_bf16<F>(k + kvrow, kx);
      load_bf16<F>(v + kvrow, vx);
      for (int j = 0; j < nsg; ++j) {
        const int64_t lk = (b * S + s0 + j) * Tk + spos;
        const int r0 = off[lk], r1 = off[lk + 1];
        const bool mine = hset == s0 + j;
        constexpr int U = 2;  // rows in flight
        for (int j0 = r0; j0 < r1; j0 += U) {
          float qx[U][F], dx[U][F], l2[U], dl[U];
          bool ok[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            ok[u] = j0 + u < r1 && mine;
            const int64_t row = rows[j0 + u < r1 ? j0 + u : r0];
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
        const float xk = static_cast<float>(static_cast<double>(ak[f]) * (1.0 / 4294967296.0));
        const float xv = static_cast<float>(static_cast<double>(av[f]) * (1.0 / 4294967296.0));
        dk[kvrow + f] = add ? dk[kvrow + f] + xk : xk;
        dv[kvrow + f] = add ? dv[kvrow + f] + xv : xv;
      }
    }
  }
}

// dq on the tile path (token blocks the forward's tile kernel took: every row
// keeps its selection as a bit mask over 64-key tiles). The forward's tile
// structure: a workgroup is one key/value head g and a token block of 4 waves
// x 32 (token, head) rows; per 64-key tile, S^T = K Q^T and dP^T = V dO^T on
// v_mfma_f32_32x32x16_bf16 (K and V rows from LDS), P = exp(scale S - lse)
// under the mask, dS = P (dP - delta), and dQ^T += K^T dS^T with K^T read
// transposed from the K tile (ds_read_b64_tr_b16) and dS^T in the B-operand
// order the C layout already has. No running max: lse is known.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void bwd_dq_tile_kernel(
    int Tq, int Tk, int Hq, int Hkv, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const uint32_t* __restrict__ mask, int Wm,
    const uint8_t* __restrict__ flag, const uint8_t* __restrict__ done, float scale_log2,
    float scale, float* __restrict__ dq, int nbps, int nblk) {
  using C = DenseCfg<D, G>;
  __shared__ __align__(16) uint16_t ks[2][C::BK * C::KP];
  __shared__ __align__(16) uint16_t vsh[2][C::BK * C::KP];

  // the forward's placement: XCD x = blockIdx.x % 8 serves key/value head x / (8/Hkv)
  const int per = 8 / Hkv;
  const int xcd = blockIdx.x & 7;
  const int g = xcd / per;
  const int blk = (blockIdx.x >> 3) * per + xcd % per;
  if (blk >= nblk) return;
  const int b = blk / nbps;
  const int tb = nbps - 1 - blk % nbps;
  if (done[static_cast<int64_t>(b) * nbps + tb] == 0) return;  // a gather-path block
  const int i0 = tb * C::BQ;
  const int iend = min(i0 + C::BQ, Tq);
  const int qo = q_offset[b];
  const int kvl0 = kv_len[b];
  const int kvl = __builtin_amdgcn_readfirstlane(kvl0 <= Tk ? max(kvl0, 0) : 0);
  const int64_t p_last = min(static_cast<int64_t>(qo) + iend - 1, static_cast<int64_t>(kvl) - 1);
  const int nkb = p_last < 0 ? 0 : static_cast<int>(p_last / C::BK) + 1;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r = lane & 31;
  const int hf = lane >> 5;
  const int i = i0 + wv * C::TW + r / G;
  const int h = g * G + r % G;
  const bool rv = i < Tq;
  const int64_t qrow = static_cast<int64_t>(b) * Tq + (rv ? i : 0);
  const int fl = rv ? flag[qrow] : 0;
  const uint32_t* mrow = mask + qrow * Wm;
  const int iw0 = i0 + wv * C::TW;
  const int p_wave_min = qo + iw0;
  const bool wave_all = __all(!rv || fl == kRowAll) && iw0 < Tq;

  // Q^T and dO^T as B operands: lane holds row[16*kk + 8*hf .. +7]
  v8bf qf[C::NKK], df[C::NKK];
  {
    const int64_t rb = (qrow * Hq + h) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      v4i z = {0, 0, 0, 0};
      qf[kk] = __builtin_bit_cast(v8bf, rv ? *reinterpret_cast<const v4i*>(q + rb + 16 * kk) : z);
      df[kk] = __builtin_bit_cast(v8bf, rv ? *reinterpret_cast<const v4i*>(dO + rb + 16 * kk) : z);
    }
  }
  // a row without entries (lse = -inf) or past the block: P = 2^(x - inf) = 0
  const float lr = rv ? lse[qrow * Hq + h] : -INFINITY;
  const float l2 = lr == -INFINITY ? INFINITY : lr * LOG2E;
  const float dl = rv ? delta[qrow * Hq + h] : 0.f;

  constexpr int UPR = D / 8;
  constexpr int RPI = 64 / UPR;
  constexpr int NI = C::BK * UPR / 256;
  const int rowstep = Hkv * D;
  const uint16_t* kbase =
      static_cast<const uint16_t*>(uniform_ptr(k + (static_cast<int64_t>(b) * Tk * Hkv + g) * D));
  const uint16_t* vbase =
      static_cast<const uint16_t*>(uniform_ptr(v + (static_cast<int64_t>(b) * Tk * Hkv + g) * D));
  int voff[NI];
#pragma unroll
  for (int c = 0; c < NI; ++c) {
    const int row = (4 * c + wv) * RPI + lane / UPR;
    const int lu = (lane % UPR) ^ swz<D>(row);
    voff[c] = (row * rowstep + 8 * lu) * 2;
  }
  auto load_tile = [&](const uint16_t* base, int kb, uint16_t* dst) {
    const int key0 = kb * C::BK;
    const int nvalid = min(kvl - key0, C::BK);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base) + static_cast<int64_t>(key0) * rowstep, 0,
        nvalid * rowstep * 2, kBufferFlags);
#pragma unroll
    for (int c = 0; c < NI; ++c)
      load16_to_lds(rs, (LDS_AS uint16_t*)dst + (4 * c + wv) * 512, voff[c]);
  };
  // X^T B of one 64-key tile (two 32-key halves): rows of X from LDS, B per lane
  auto tile_mm = [&](const uint16_t* x_lds, const v8bf* bf, v16f* st) {
    const LDS_AS uint16_t* xs = (const LDS_AS uint16_t*)x_lds;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[kt][e] = 0.f;
      const int krow = 32 * kt + r;
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        const v8bf a = __builtin_bit_cast(
            v8bf, *(const LDS_AS v4i*)(xs + tile_off<D>(krow, 16 * kk + 8 * hf)));
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[kk], st[kt], 0, 0, 0);
      }
    }
  };
  const int wlast = Wm - 1;

  v16f acc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  if (nkb > 0) {
    load_tile(kbase, 0, ks[0]);
    load_tile(vbase, 0, vsh[0]);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) {
      load_tile(kbase, kb + 1, ks[buf ^ 1]);
      load_tile(vbase, kb + 1, vsh[buf ^ 1]);
    }
    uint32_t mw[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint32_t x = mrow[min(2 * kb + kt, wlast)];
      mw[kt] = 2 * kb + kt <= wlast ? x : 0u;
    }
    v16f sc[2], dp[2];
    tile_mm(ks[buf], qf, sc);
    tile_mm(vsh[buf], df, dp);
    const int key0 = kb * C::BK;
    if (!(wave_all && key0 + C::BK - 1 <= p_wave_min)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint32_t m = mw[kt] >> (4 * hf);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int sel = __builtin_amdgcn_sbfe(static_cast<int>(m), 8 * (e >> 2) + (e & 3), 1);
          const int sb = __float_as_int(sc[kt][e]);
          sc[kt][e] = __int_as_float((sb & sel) | (~sel & kNegInfBits));
        }
      }
    }
    // dS^T in the B-operand order of the dQ step s (see the forward's P^T)
    v8bf pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(__builtin_fmaf(sc[kt][e], scale_log2, -l2));
        pb[2 * kt + (e >> 3)][e & 7] = static_cast<__bf16>(p * (dp[kt][e] - dl));
      }
    // dQ^T += K^T dS^T over the 64 keys, four 16-key steps
    const LDS_AS uint16_t* ksl = (const LDS_AS uint16_t*)(ks[buf]);
    const int gi = lane & 15;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int d0 = 32 * dt + 16 * ((lane >> 4) & 1);
        const int k0 = 16 * s2 + 4 * hf;
        LDS_AS v4bf* a0 = (LDS_AS v4bf*)(ksl + tile_off<D>(k0 + gi / 4, d0 + 4 * (gi % 4)));
        LDS_AS v4bf* a1 = (LDS_AS v4bf*)(ksl + tile_off<D>(k0 + 8 + gi / 4, d0 + 4 * (gi % 4)));
        const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a0);
        const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a1);
        const v8bf a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], acc[dt], 0, 0, 0);
      }
    }
    // the barrier waits for the next tile's loads and keeps this tile's
    // buffers until every wave is done with them
    __syncthreads();
  }
  if (!rv) return;
  // lane holds dQ^T rows d = 32 dt + 8 (e/4) + 4 hf + e%4 of its (token, head)
  float* out = dq + (qrow * Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float4 val = make_float4(scale * acc[dt][4 * ii], scale * acc[dt][4 * ii + 1],
                                     scale * acc[dt][4 * ii + 2], scale * acc[dt][4 * ii + 3]);
      *reinterpret_cast<float4*>(out + 32 * dt + 8 * ii + 4 * hf) = val;
    }
}

// dk, dv on the tile path, key-major: a workgroup is one key/value head g and
// a block of 64 keys; 4 waves, two per 32 keys (the MFMA N dimension), each
// pair splitting d (both compute the pair's S and dP). Two workgroups share a
// compute unit (two waves per SIMD, not in step with each other), which hides
// the latency of one wave's chain of reads, MFMAs and exponentials. It walks the row
// tiles (32 (token, head) rows: TW tokens x G heads) of the token blocks the
// forward's tile kernel took, from the last down to the first that can see
// its keys, so that the workgroups of one head read the same Q and dO rows at
// about the same time. Per row tile: S = Q K^T and dP = dO V^T (Q, dO rows
// from LDS, K and V held as B operands), P = exp(scale S - lse) under each
// row's mask, dS = P (dP - delta), then dV^T += dO^T P and dK^T += Q^T dS
// with dO^T and Q^T read transposed from LDS and P, dS in the B-operand order
// the C layout already has. A fixed order of row tiles: deterministic sums.
template <int D, int G>
__global__ __launch_bounds__(kDkdvThreads, 2) void bwd_dkdv_tile_kernel(
    int Tq, int Tk, int Hq, int Hkv, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const uint32_t* __restrict__ mask, int Wm,
    const uint8_t* __restrict__ done, float scale_log2, float scale, float* __restrict__ dk,
    float* __restrict__ dv, int nkbs, int nblk, int nbps, int nch, int ch, int lim,
    float* __restrict__ part) {
  using C = DenseCfg<D, G>;
  constexpr int TW = C::TW;  // tokens per row tile
  constexpr int KB = kDkdvKeys;
  __shared__ __align__(16) uint16_t qs[2][32 * D];
  __shared__ __align__(16) uint16_t os[2][32 * D];
  constexpr int NKQ = KB / 32;          // 32-key groups
  constexpr int NT = kDkdvThreads;      // threads
  __shared__ __align__(16) uint32_t msk[2][NKQ][32];  // [wave][row]: the row's word of the wave's keys
  __shared__ __align__(16) float l2s[2][32];
  __shared__ __align__(16) float dls[2][32];

  // XCD x = blockIdx.x % 8 serves key/value head x / (8/Hkv)
  const int per = 8 / Hkv;
  const int xcd = blockIdx.x & 7;
  const int g = xcd / per;
  const int blk = (blockIdx.x >> 3) * per + xcd % per;
  if (blk >= nblk) return;
  // chunk-major, last chunk first: the workgroups running together walk the
  // same rows (shared in L2), and the last chunk has work for every key block
  const int nb = nblk / (nkbs * nch);
  const int key0 = (blk % nkbs) * KB;
  const int b = blk / nkbs % nb;
  const int c = nch - 1 - blk / (nkbs * nb);
  const int qo = q_offset[b];
  const int kvl0 = kv_len[b];
  const int kvl = __builtin_amdgcn_readfirstlane(kvl0 <= Tk ? max(kvl0, 0) : 0);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r = lane & 31;
  const int hf = lane >> 5;
  const int kq = wv % NKQ;  // the wave's 32 keys
  const int dh = wv / NKQ;  // the wave's half of d
  constexpr int NDH = C::NDT / 2;
  const int key = key0 + 32 * kq + r;

  // K^T and V^T as B operands: lane holds row[16*kk + 8*hf .. +7] of its key
  v8bf kf[C::NKK], vf[C::NKK];
  {
    const bool kv_ok = key < kvl;
    const int64_t rb = ((static_cast<int64_t>(b) * Tk + (kv_ok ? key : 0)) * Hkv + g) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      v4i z = {0, 0, 0, 0};
      kf[kk] = __builtin_bit_cast(v8bf, kv_ok ? *reinterpret_cast<const v4i*>(k + rb + 16 * kk) : z);
      vf[kk] = __builtin_bit_cast(v8bf, kv_ok ? *reinterpret_cast<const v4i*>(v + rb + 16 * kk) : z);
    }
  }

  // row tiles t (tokens t*TW ..): from the first whose last token sees key0
  // to the last token inside the history that may take the tile path
  // (p + 1 <= lim); key blocks at or past lim have no tile rows
  const int64_t i_first = max(static_cast<int64_t>(key0) - qo, int64_t(0));
  const int64_t i_end = min(min(static_cast<int64_t>(Tq), static_cast<int64_t>(kvl) - qo),
                            static_cast<int64_t>(lim) - qo);
  int t_first = static_cast<int>(i_first / TW);
  int t_last = i_end > i_first && key0 < kvl ? static_cast<int>((i_end - 1) / TW) : -1;
  if (nch > 1) {
    // chunk c: row tiles [c ch, (c+1) ch); a chunk outside the walk writes
    // nothing and the sum skips it
    if (t_last < t_first || t_last / ch < c || t_first / ch > c) return;
    t_first = max(t_first, c * ch);
    t_last = min(t_last, (c + 1) * ch - 1);
  }
  // done bytes read as aligned words: uniform loads through the scalar cache
  const uint32_t* done_w = reinterpret_cast<const uint32_t*>(done);
  auto tile_done = [&](int t) {
    const int64_t x = static_cast<int64_t>(b) * nbps + t * TW / C::BQ;
    return ((done_w[x >> 2] >> (8 * (x & 3))) & 0xffu) != 0;
  };
  auto prev_tile = [&](int t) {  // the last tile <= t of a tile-path token block
    while (t >= t_first && !tile_done(t)) --t;
    return t;
  };

  // a row tile is 32 rows of D/8 16-byte units: thread x moves units x,
  // x + NT, ..., to LDS offset 16 x (the unit's place after the swizzle)
  constexpr int UPR = D / 8;
  constexpr int NU = 32 * UPR / NT;
  const int tid = threadIdx.x;
  int roff[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int x = tid + NT * u;
    const int row = x / UPR;
    const int lu = (x % UPR) ^ swz<D>(row);
    roff[u] = (((row / G) * Hq + row % G) * D + 8 * lu) * 2;
  }
  // the next tile's rows pass through registers: loads straight into LDS
  // would make every LDS read of the current tile wait for them
  auto load_rows = [&](int t, v4i* rg) {
    const int i0 = t * TW;
    const int ntok = min(TW, Tq - i0);
    const int64_t e0 = ((static_cast<int64_t>(b) * Tq + i0) * Hq + g * G) * D;
    const int bytes = ((ntok - 1) * Hq + G) * D * 2;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(q + e0), 0, bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(dO + e0), 0, bytes, kBufferFlags);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      rg[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, roff[u], 0, 0));
      rg[NU + u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ro, roff[u], 0, 0));
    }
  };
  auto store_rows = [&](const v4i* rg, int nb) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      *(LDS_AS v4i*)((LDS_AS uint16_t*)qs[nb] + 8 * (tid + NT * u)) = rg[u];
      *(LDS_AS v4i*)((LDS_AS uint16_t*)os[nb] + 8 * (tid + NT * u)) = rg[NU + u];
    }
  };
  // per-row values of tile t: threads 0 .. 32 NKQ - 1 the mask words (one
  // per 32-key group), the next 32 lse, the 32 after delta. One load from a clamped in-range address; the row's
  // validity and the lse transform (log2, +inf for a row without entries)
  // wait until the store, after the tile's work.
  constexpr int TL = 32 * NKQ, TD = TL + 32, TE = TD + 32;
  const int kw = key0 / 32 + min(tid >> 5, NKQ - 1);
  auto stage_load = [&](int t) -> uint32_t {
    const int R = tid & 31;
    const int i = min(t * TW + R / G, Tq - 1);
    const int64_t tok = static_cast<int64_t>(b) * Tq + i;
    const int64_t rh = tok * Hq + g * G + R % G;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tid < TD ? lse : delta) + rh;
    if (tid < TL && Wm > 0) src = mask + tok * Wm + min(kw, Wm - 1);
    return *src;
  };
  auto stage_store = [&](uint32_t x, int t, int nb) {
    const int R = tid & 31;
    const bool ok = t * TW + R / G < Tq;
    if (tid < TL) {
      msk[nb][tid >> 5][R] = ok && kw < Wm ? x : 0u;
    } else if (tid < TD) {
      const float l = __uint_as_float(x);
      l2s[nb][R] = !ok || l == -INFINITY ? INFINITY : l * LOG2E;
    } else if (tid < TE) {
      dls[nb][R] = ok ? __uint_as_float(x) : 0.f;
    }
  };

  v16f av[NDH], ak[NDH];
#pragma unroll
  for (int dt = 0; dt < NDH; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) av[dt][e] = ak[dt][e] = 0.f;

  int t = prev_tile(t_last);
  v4i rg[2 * NU];
  if (t >= t_first) {
    load_rows(t, rg);
    store_rows(rg, 0);
    stage_store(stage_load(t), t, 0);
  }
  __syncthreads();
  int buf = 0;
  const int gi = lane & 15;
  while (t >= t_first) {
    const int tn = prev_tile(t - 1);
    uint32_t xn = 0;
    if (tn >= t_first) {
      load_rows(tn, rg);
      xn = stage_load(tn);
    }
    const LDS_AS uint16_t* qt = (const LDS_AS uint16_t*)qs[buf];
    const LDS_AS uint16_t* ot = (const LDS_AS uint16_t*)os[buf];
    // S and dP: rows x the wave's 32 keys
    v16f sc, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      const int o = tile_off<D>(r, 16 * kk + 8 * hf);
      const v8bf aq = __builtin_bit_cast(v8bf, *(const LDS_AS v4i*)(qt + o));
      const v8bf ao = __builtin_bit_cast(v8bf, *(const LDS_AS v4i*)(ot + o));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kk], sc, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kk], dp, 0, 0, 0);
    }
    // element e is row 8 (e/4) + 4 hf + e%4 of the tile and key r of the wave
    v8bf pp[2], pd[2];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int R0 = 8 * ii + 4 * hf;
      const v4u mw = *(const LDS_AS v4u*)&msk[buf][kq][R0];
      const v4f l2 = *(const LDS_AS v4f*)&l2s[buf][R0];
      const v4f dl = *(const LDS_AS v4f*)&dls[buf][R0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * ii + j;
        // bit r of the row's word keeps this key: a one-bit signed extract
        // gives an all-ones/all-zeros mask for the exponential's bits
        const int sel = __builtin_amdgcn_sbfe(static_cast<int>(mw[j]), r, 1);
        const float p = __int_as_float(
            __float_as_int(fast_exp2(__builtin_fmaf(sc[e], scale_log2, -l2[j]))) & sel);
        pp[e >> 3][e & 7] = static_cast<__bf16>(p);
        pd[e >> 3][e & 7] = static_cast<__bf16>(p * (dp[e] - dl[j]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows, two 16-row steps
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int dt = 0; dt < NDH; ++dt) {
        const int d0 = 32 * (NDH * dh + dt) + 16 * ((lane >> 4) & 1);
        const int k0 = 16 * s2 + 4 * hf;
        const int o0 = tile_off<D>(k0 + gi / 4, d0 + 4 * (gi % 4));
        const int o1 = tile_off<D>(k0 + 8 + gi / 4, d0 + 4 * (gi % 4));
        const v4bf olo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4bf*)(ot + o0));
        const v4bf ohi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4bf*)(ot + o1));
        const v4bf qlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4bf*)(qt + o0));
        const v4bf qhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4bf*)(qt + o1));
        av[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7), pp[s2], av[dt], 0, 0, 0);
        ak[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), pd[s2], ak[dt], 0, 0, 0);
      }
    }
    if (tn >= t_first) {
      store_rows(rg, buf ^ 1);
      stage_store(xn, tn, buf ^ 1);
    }
    // the barrier waits for the next tile's loads and keeps this tile's
    // buffers until every wave is done with them
    __syncthreads();
    t = tn;
    buf ^= 1;
  }
  if (key >= Tk) return;
  // lane holds dV^T rows d = 32 dt + 8 (e/4) + 4 hf + e%4 of its key
  const int64_t ob = ((static_cast<int64_t>(b) * Tk + key) * Hkv + g) * D;
  if (nch > 1) {
    // partials [2][nch][B][Tk][Hkv][D]: dv, then dk
    const int64_t n = static_cast<int64_t>(nb) * Tk * Hkv * D;
    dv = part + c * n;
    dk = part + (nch + c) * n;
  }
#pragma unroll
  for (int dt = 0; dt < NDH; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = 32 * (NDH * dh + dt) + 8 * ii + 4 * hf;
      *reinterpret_cast<float4*>(dv + ob + d) =
          make_float4(av[dt][4 * ii], av[dt][4 * ii + 1], av[dt][4 * ii + 2], av[dt][4 * ii + 3]);
      *reinterpret_cast<float4*>(dk + ob + d) =
          make_float4(scale * ak[dt][4 * ii], scale * ak[dt][4 * ii + 1],
                      scale * ak[dt][4 * ii + 2], scale * ak[dt][4 * ii + 3]);
    }
}

// dk, dv = the sum of the chunks' partials, in chunk order (the chunks that
// the key block's walk touched, as the tile kernel decides them)
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_part_sum_kernel(
    int B, int Tq, int Tk, int Hkv, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const float* __restrict__ part, int nch, int ch, int lim,
    float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int TW = 32 / G;
  const int64_t n = static_cast<int64_t>(B) * Tk * Hkv * D;
  for (int64_t x = (blockIdx.x * 256LL + threadIdx.x) * 4; x < n; x += gridDim.x * 1024LL) {
    const int64_t krow = x / (static_cast<int64_t>(Hkv) * D);  // b*Tk + key
    const int b = static_cast<int>(krow / Tk);
    const int key0 = static_cast<int>(krow % Tk) / kDkdvKeys * kDkdvKeys;
    const int qo = q_offset[b];
    const int kvl0 = kv_len[b];
    const int kvl = kvl0 <= Tk ? max(kvl0, 0) : 0;
    const int64_t i_first = max(static_cast<int64_t>(key0) - qo, int64_t(0));
    const int64_t i_end = min(min(static_cast<int64_t>(Tq), static_cast<int64_t>(kvl) - qo),
                              static_cast<int64_t>(lim) - qo);
    const int t_first = static_cast<int>(i_first / TW);
    const int t_last = i_end > i_first && key0 < kvl ? static_cast<int>((i_end - 1) / TW) : -1;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    if (t_last >= t_first) {
      const int c1 = min(t_last / ch, nch - 1);
      for (int c = t_first / ch; c <= c1; ++c) {
        const float4 a = *reinterpret_cast<const float4*>(part + c * n + x);
        const float4 e = *reinterpret_cast<const float4*>(part + (nch + c) * n + x);
        sv.x += a.x; sv.y += a.y; sv.z += a.z; sv.w += a.w;
        sk.x += e.x; sk.y += e.y; sk.z += e.z; sk.w += e.w;
      }
    }
    *reinterpret_cast<float4*>(dv + x) = sv;
    *reinterpret_cast<float4*>(dk + x) = sk;
  }
}

// dq of the gather rows: one wave per (row, unit); a unit is a key/value head's
// query heads, or an index set's when there are more sets than key/value heads
template <int D>
hipError_t launch_dq_gather(const Geom& g, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* idx, const float* lse,
                            const uint16_t* dO, const float* dlt, float scale, float* dq,
                            const uint8_t* done, int dbq, hipStream_t st) {
  const int units = std::max(g.sets, g.Hkv);
  const int gu = g.Hq / units;  // query heads per wave
  const int64_t nw = static_cast<int64_t>(g.B) * g.Tq * units;
  const dim3 grid(static_cast<uint32_t>((nw + 3) / 4));
  KernelTimer timer(LCI_KERNEL_BWD_DQ, st);
#define LCI_DQ_GATHER(GU)                                                                         \
  hipLaunchKernelGGL((bwd_dq_kernel<D, GU>), grid, dim3(256), 0, st, g.Tq, g.Tk, g.K, g.Hq, g.Hkv, \
                     g.Hq / g.Hkv, units, g.sets, g.kv_len, q, k, v, idx, lse, dO, dlt, scale, dq, \
                     nw, done, dbq)
  switch (gu) {
    case 1: LCI_DQ_GATHER(1); break;
    case 2: LCI_DQ_GATHER(2); break;
    case 4: LCI_DQ_GATHER(4); break;
    case 8: LCI_DQ_GATHER(8); break;
    case 16: LCI_DQ_GATHER(16); break;
    default: return hipErrorInvalidValue;
  }
#undef LCI_DQ_GATHER
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_bwd_dg(const Geom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* idx, const float* lse, const uint16_t* dO, const float* dlt,
                         const int32_t* off, const int32_t* rows, float scale, float* dq,
                         float* dk, float* dv, const DenseMasks* dm, int nch, float* part,
                         hipStream_t st) {
  using C = DenseCfg<D, G>;
  hipError_t e;
  if (dm) {
    // the tile path: token blocks the forward's tile kernel took
    const int nbps = (g.Tq + C::BQ - 1) / C::BQ;
    const int nblk = g.B * nbps;
    const int per = 8 / g.Hkv;
    const int64_t nwg = static_cast<int64_t>((nblk + per - 1) / per) * 8;
    KernelTimer timer(LCI_KERNEL_BWD_DQ, st);
    hipLaunchKernelGGL((bwd_dq_tile_kernel<D, G>), dim3(static_cast<uint32_t>(nwg)), dim3(256), 0,
                       st, g.Tq, g.Tk, g.Hq, g.Hkv, g.q_offset, g.kv_len, q, k, v, dO, lse, dlt,
                       dm->mask, dm->Wm, dm->flag, dm->done, scale * LOG2E, scale, dq, nbps,
                       nblk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_dq_gather<D>(g, q, k, v, idx, lse, dO, dlt, scale, dq, dm ? dm->done : nullptr,
                               C::BQ, st)) != hipSuccess)
    return e;
  if (dm) {
    // every key from the tile-path rows; the gather rows are added below
    const int nbps = (g.Tq + C::BQ - 1) / C::BQ;
    const int nkbs = (g.Tk + kDkdvKeys - 1) / kDkdvKeys;
    const int nblk = g.B * nkbs * nch;
    const int per = 8 / g.Hkv;
    const int64_t nwg = static_cast<int64_t>((nblk + per - 1) / per) * 8;
    const int ntw = (g.Tq + C::TW - 1) / C::TW;
    const int ch = (ntw + nch - 1) / nch;
    {
      KernelTimer timer(LCI_KERNEL_BWD_DKDV, st);
      hipLaunchKernelGGL((bwd_dkdv_tile_kernel<D, G>), dim3(static_cast<uint32_t>(nwg)),
                         dim3(kDkdvThreads), 0, st, g.Tq, g.Tk, g.Hq, g.Hkv, g.q_offset, g.kv_len,
                         q, k, v, dO, lse, dlt, dm->mask, dm->Wm, dm->done, scale * LOG2E, scale,
                         dk, dv, nkbs, nblk, nbps, nch, ch, dm->lim, part);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nch > 1) {
      const int64_t n4 = static_cast<int64_t>(g.B) * g.Tk * g.Hkv * D / 4;
      KernelTimer timer(LCI_KERNEL_BWD_DKDV, st);  // the partial sum
      hipLaunchKernelGGL((bwd_part_sum_kernel<D, G>),
                         dim3(static_cast<uint32_t>(std::min<int64_t>((n4 + 255) / 256, 8192))),
                         dim3(256), 0, st, g.B, g.Tq, g.Tk, g.Hkv, g.q_offset, g.kv_len, part,
                         nch, ch, dm->lim, dk, dv);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  const int64_t nkey_w = static_cast<int64_t>(g.B) * g.Tk * g.Hkv;
  {
    KernelTimer timer(LCI_KERNEL_BWD_DKDV, st);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>),
                       dim3(static_cast<uint32_t>(std::min<int64_t>((nkey_w + 3) / 4, 1 << 16))),
                       dim3(256), 0, st, g.Tk, g.Hq, g.Hkv, g.sets, q, k, v, lse, dO, dlt, off,
                       rows, scale, dk, dv, nkey_w, dm ? 1 : 0);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const Geom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* idx, const float* lse, const uint16_t* dO, const float* dlt,
                        const int32_t* off, const int32_t* rows, float scale, float* dq,
                        float* dk, float* dv, const DenseMasks* dm, int nch, float* part,
                        hipStream_t st) {
  switch (g.Hq / g.Hkv) {
    case 1: return launch_bwd_dg<D, 1>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    case 2: return launch_bwd_dg<D, 2>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    case 4: return launch_bwd_dg<D, 4>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    case 8: return launch_bwd_dg<D, 8>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    case 16: return launch_bwd_dg<D, 16>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

hipError_t launch_exclusive_scan(const int32_t* in, int64_t n, int32_t* out, int32_t* tiles,
                                 hipStream_t st) {
  const int ntiles = static_cast<int>((n + 1023) / 1024);
  const uint32_t gk = static_cast<uint32_t>(std::min<int64_t>((n + 1 + 255) / 256, 8192));
  hipLaunchKernelGGL(scan_tiles_kernel, dim3(static_cast<uint32_t>(ntiles)), dim3(256), 0, st, in,
                     n, out, tiles);
  hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(1024), 0, st, tiles, ntiles);
  hipLaunchKernelGGL(scan_add_kernel, dim3(gk), dim3(256), 0, st, out, n, tiles, ntiles);
  return hipGetLastError();
}


// [forward workspace][o bf16][lse][do][delta][counts][offsets (+1)][cursors][tiles (+1)][rows]
// with the position lists per (sequence, index set, position)
BwdLayout bwd_layout(const Geom& g) {
  BwdLayout L{};
  const size_t rows = static_cast<size_t>(g.B) * g.Tq;
  const size_t keys = static_cast<size_t>(g.B) * g.sets * g.Tk;
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
  L.part = L.rows + align256(rows * g.sets * g.K * sizeof(int32_t));
  // the key-major tile kernel splits each key block's rows into up to
  // kBwdChunks chunks (balance: the first key blocks see every row, the last
  // few), each writing partial dk and dv, as many as fit in kBwdPartMax bytes
  // of partials; with one chunk the kernel writes dk, dv directly
  const size_t pbytes = static_cast<size_t>(g.B) * g.Tk * g.Hkv * g.d * sizeof(float) * 2;
  L.nch = 1;
  if (L.splits == 1 && g.sets == 1)
    for (int n = kBwdChunks; n > 1; n /= 2)
      if (n * pbytes <= kBwdPartMax) {
        L.nch = n;
        break;
      }
  L.total = L.part + (L.nch > 1 ? align256(L.nch * pbytes) : 0);
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
  float* part = L.nch > 1 ? reinterpret_cast<float*>(ws + L.part) : nullptr;
  const int nch = L.nch;
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
  // with one split the forward ran the tile path: its masks, row flags and
  // done bytes sit in the forward workspace. The position lists below hold
  // only the rows of the other token blocks. With several index sets every
  // row takes the gather kernels.
  const DenseMasks dmv = dense_masks(g, ws + L.fwd);
  const DenseMasks* dm = L.splits == 1 && g.sets == 1 ? &dmv : nullptr;
  const uint8_t* done = dm ? dm->done : nullptr;
  const int dbq = dense_block_rows(g.Hq / g.Hkv);
  // the rows that selected each position, per index set
  const int64_t keys = static_cast<int64_t>(g.B) * g.sets * g.Tk;
  const int64_t nent = static_cast<int64_t>(g.B) * g.sets * g.Tq * g.K;
  const uint32_t gk = static_cast<uint32_t>(std::min<int64_t>((keys + 255) / 256, 8192));
  const uint32_t ge = static_cast<uint32_t>(std::min<int64_t>((nent + 255) / 256, 8192));
  {
    KernelTimer timer(LCI_KERNEL_BWD_TRANSPOSE, st);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(gk), dim3(256), 0, st, cnt, keys, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(gk), dim3(256), 0, st, cursor, keys, 0);
    hipLaunchKernelGGL(bwd_count_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, g.sets,
                       g.kv_len, idx, nent, cnt, done, dbq);
    hipLaunchKernelGGL(scan_tiles_kernel, dim3(static_cast<uint32_t>(L.ntiles)), dim3(256), 0, st,
                       cnt, keys, off, tiles);
    hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(1024), 0, st, tiles, L.ntiles);
    hipLaunchKernelGGL(scan_add_kernel, dim3(gk), dim3(256), 0, st, off, keys, tiles, L.ntiles);
    hipLaunchKernelGGL(bwd_fill_kernel, dim3(ge), dim3(256), 0, st, g.Tq, g.Tk, g.K, g.sets,
                       g.kv_len, idx, nent, off, cursor, rows, done, dbq);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (g.d) {
    case 64: return launch_bwd_d<64>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    case 128: return launch_bwd_d<128>(g, q, k, v, idx, lse, dO, dlt, off, rows, scale, dq, dk, dv, dm, nch, part, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
