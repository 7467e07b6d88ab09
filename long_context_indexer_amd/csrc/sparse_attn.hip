// Sparse exact attention over gathered key/value rows + sigmoid output gate (gfx950).
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Indexer + Top-K: How
// Fine-Grained Sparse Attention Works", steps 3-4: standard softmax attention
// over the selected positions only (scaled by 1/sqrt(d)), then a sigmoid gate
// that modulates the output per head and feature; "From Linear Attention to
// Gated Sparse Attention", section 2 (the gate multiplies the attention output).
//
// One workgroup per (query row, split of its index list, group of up to 8
// waves); each wave serves a unit of Gu query heads that read one key/value
// head and one index set: with one index set per row or per key/value head the
// unit is a key/value head's G = Hq/Hkv query heads (grouped-query attention),
// with more sets than key/value heads it is one set's Hq/sets query heads.
// Per chunk of 16 positions of its index set a wave
//   - gathers the 16 key rows of head g straight into MFMA A-operand registers
//     (each lane loads 16 contiguous bytes of one row),
//   - computes S^T = K_sel . Q^T on v_mfma_f32_16x16x32_bf16 (rows = keys,
//     columns = the Gu query heads), so lane l holds keys 4*(l/16)+i of head l%16,
//   - updates an online softmax in base 2 (logits pre-scaled by scale*log2 e),
//   - rounds P to bf16; its register layout is already the B operand of
//     O^T += V^T . P on v_mfma_f32_16x16x16bf16_1k,
//   - stages the 16 value rows in LDS (per-wave region, row pitch padded to
//     avoid bank conflicts) and reads them transposed as the A operand.
// Every per-head statistic lives in the lane that owns that head's column, so
// rescaling needs no cross-lane traffic; the softmax denominator is kept per
// lane and reduced once at the end. With one split the epilogue applies the
// gate (sigmoid(gate) * o, or s*o + (1-s)*x mixed with the other branch's
// output x: the fusion step and pseudocode of the same section) and stores
// bf16; with several splits each writes (m, l, O) and a combine kernel merges
// them in split order (deterministic) and applies the gate.
#include "attn_dense.h"
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"

namespace lci {

#define LDS_AS __attribute__((address_space(3)))

template <int D>
struct AttnCfg {
  static constexpr int NCH = D / 32;          // 32-deep steps for Q.K
  static constexpr int NJB = D / 16;          // 16-wide blocks of the value dim
  static constexpr int PITCH = D + 8;         // LDS row pitch in bf16: rows 16-byte aligned, as the
                                              // transposed LDS read (ds_read_b64_tr_b16) needs
  static constexpr int PART = D + 4;          // floats per split partial: O[D], m, l, l_exact, pad
};

// Merge the splits of one query row in split order (fixed, so deterministic),
// apply the gate and store. A kernel of its own: on a multi-XCD part, handing
// partials from workgroup to workgroup inside one kernel needs an L2 write-back
// per workgroup, a kernel boundary needs one. Thread t owns 2 consecutive
// features of one (row, head) and merges the splits in one pass with a running
// maximum; the loads of different splits are independent, so they overlap.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(int Hq, int splits,
                                                           const float* __restrict__ part,
                                                           const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ mix,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  using C = AttnCfg<D>;
  constexpr int QPH = D / 2;  // threads per head
  const int64_t qrow = blockIdx.x;
  const int t = blockIdx.y * blockDim.x + threadIdx.x;
  if (t >= Hq * QPH) return;
  const int h = t / QPH;
  const int j0 = 2 * (t % QPH);
  const float* pp = part + (qrow * Hq + h) * splits * C::PART;
  float M = -INFINITY, L = 0.f, Lex = 0.f;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float* ps = pp + s * C::PART;
    const float ms = ps[D];
    const float2 os = *reinterpret_cast<const float2*>(ps + j0);
    const float ls = ps[D + 1], lxs = ps[D + 2];
    const float Mn = fmaxf(M, ms);
    // weights relative to the running maximum; a split without entries (-inf)
    // contributes nothing, and nothing is rescaled while M is still -inf
    const float fo = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
    const float fs = (ms == -INFINITY) ? 0.f : fast_exp2(ms - Mn);
    a0 = a0 * fo + fs * os.x;
    a1 = a1 * fo + fs * os.y;
    L = L * fo + fs * ls;
    Lex = Lex * fo + fs * lxs;
    M = Mn;
  }
  const float inv = L > 0.f ? fast_rcp(L) : 0.f;
  const int64_t obase = (qrow * Hq + h) * D + j0;
  float y0 = a0 * inv, y1 = a1 * inv;
  if (gate) {
    const uint32_t g01 = *reinterpret_cast<const uint32_t*>(gate + obase);
    const float s0 = sigmoidf(bf16_to_f32(g01 & 0xffff));
    const float s1 = sigmoidf(bf16_to_f32(g01 >> 16));
    if (mix) {
      const uint32_t x01 = *reinterpret_cast<const uint32_t*>(mix + obase);
      y0 = gate_mix(y0, s0, x01 & 0xffff);
      y1 = gate_mix(y1, s1, x01 >> 16);
    } else {
      y0 *= s0;
      y1 *= s1;
    }
  }
  *reinterpret_cast<uint32_t*>(out + obase) =
      f32_to_bf16(y0) | (static_cast<uint32_t>(f32_to_bf16(y1)) << 16);
  if (lse && j0 == 0) lse[qrow * Hq + h] = Lex > 0.f ? (M + fast_log2(Lex)) * LN2 : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(512) void sparse_attn_kernel(
    int Tq, int Tk, int K, int Hq, int Hkv, int G, int sets, int Gu, int nck,
    const int32_t* __restrict__ kv_len,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ gate, const uint16_t* __restrict__ mix, float scale_log2,
    uint16_t* __restrict__ out,
    float* __restrict__ lse, int splits, int per_split, float* __restrict__ part,
    const uint8_t* __restrict__ done, int dbq, int64_t nitems) {
  using C = AttnCfg<D>;
  // [waves][16][PITCH]; 16-byte aligned wherever the dynamic LDS region starts:
  // its 8-byte writes and transposed reads need aligned rows
  extern __shared__ __align__(16) uint16_t vstage[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  // work items ((b*Tq + row)*splits + split)*nck + chunk of units, strided over
  // the grid; the waves of a workgroup share no LDS and no barrier, so an item
  // ends by returning from the per-item body
  for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) [&] {
  const int64_t rs = item / nck;
  const int split = static_cast<int>(rs % splits);
  const int64_t qrow = rs / splits;
  const int b = static_cast<int>(qrow / Tq);
  // this wave's unit: query heads h0 .. h0 + Gu - 1, of key/value head g and
  // index set sg (query head h reads set h / (Hq/sets))
  const int h0 = (static_cast<int>(item % nck) * nw + wv) * Gu;
  const int g = h0 / G;
  const int sg = h0 / (Hq / sets);
  if (done) {
    // token blocks the tile kernel took (for this wave's index set) are finished
    const int i = static_cast<int>(qrow % Tq);
    const int nbps = (Tq + dbq - 1) / dbq;
    if (done[(static_cast<int64_t>(b) * sets + sg) * nbps + i / dbq]) return;
  }
  const int kvl0 = kv_len[b];
  const int kvl = kvl0 <= Tk ? kvl0 : 0;  // a history longer than its allocation: no entry is read
  const int e_begin = split * per_split;
  const int nent = max(0, min(per_split, K - e_begin));
  // index rows [B][sets][Tq][K]: the wave reads the row of its own set
  const int64_t irow = qrow + (static_cast<int64_t>(b) * (sets - 1) + sg) * Tq;
  const int32_t* ip = idx + irow * K + e_begin;
  uint16_t* vs = vstage + wv * 16 * C::PITCH;

  const int hl = lane & 15;     // this lane's query-head column
  const int grp = lane >> 4;    // lane group 0..3
  const bool hok = hl < Gu;
  const int h = h0 + hl;

  v8bf qf[C::NCH];
  {
    const uint16_t* qp = q + (qrow * Hq + (hok ? h : 0)) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      v4i z = {0, 0, 0, 0};
      v4i t = hok ? *reinterpret_cast<const v4i*>(qp + 32 * c) : z;
      qf[c] = __builtin_bit_cast(v8bf, t);
    }
  }

  float m = -INFINITY;  // running max (base-2 units) of head hl
  float lsum = 0.f;     // this lane's share of the denominator, from the bf16-rounded P
  float lex = 0.f;      // the same from the unrounded P (for lse only)
  v4f o[C::NJB];
#pragma unroll
  for (int jb = 0; jb < C::NJB; ++jb) o[jb] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kbase = k + (static_cast<int64_t>(b) * Tk * Hkv + g) * D;
  const uint16_t* vbase = v + (static_cast<int64_t>(b) * Tk * Hkv + g) * D;
  const int64_t rowstep = static_cast<int64_t>(Hkv) * D;

  // listed position of entry e0 + (lane % 16), read unconditionally (clamped)
  // so every load in the loop is straight-line and the compiler can wait for
  // exactly the loads a step needs; -1 past the end of the list
  const int last = max(nent - 1, 0);
  auto entry = [&](int e0) {
    const int e = e0 + hl;
    const int v0 = ip[min(e, last)];
    return e < nent ? v0 : -1;
  };
  // issue the key fragment and value-row loads of one 16-entry chunk
  auto issue = [&](int sa, v8bf (&kf)[C::NCH], v4i (&vx)[D / 32]) {
    const bool va = sa >= 0 && sa < kvl;
    const int ss = va ? sa : 0;  // invalid entries read row 0 and are masked
    const uint16_t* kp = kbase + ss * rowstep + 8 * grp;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
      kf[c] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kp + 32 * c));
    // value piece t of this lane: row (t*64 + lane) / (D/8) of the chunk
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int piece = t * 64 + lane;
      const int sr = __shfl(ss, piece / (D / 8), 64);
      vx[t] = *reinterpret_cast<const v4i*>(vbase + sr * rowstep + 8 * (piece % (D / 8)));
    }
  };

  LDS_AS uint16_t* vl = (LDS_AS uint16_t*)(vs);
  // one 16-entry chunk: stage V, S^T, online softmax, O^T += V^T P^T
  auto compute = [&](const v8bf (&kf)[C::NCH], const v4i (&vx)[D / 32], bool va) {
    // stage the 16 value rows (row-major, padded pitch); stores and the
    // transposed reads below are DS operations of this wave, in program order
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int piece = t * 64 + lane;
      LDS_AS v2i* dst = (LDS_AS v2i*)(vl + (piece / (D / 8)) * C::PITCH + 8 * (piece % (D / 8)));
      dst[0] = v2i{vx[t][0], vx[t][1]};
      dst[1] = v2i{vx[t][2], vx[t][3]};
    }
    v4f st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], st, 0, 0, 0);

    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool vi = __shfl(static_cast<int>(va), 4 * grp + i, 64) != 0;
      x[i] = vi ? st[i] * scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
    v4s pb;
    float psum = 0.f, pex = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pi = (x[i] == -INFINITY) ? 0.f : fast_exp2(x[i] - m_new);
      const uint16_t hb = f32_to_bf16(pi);
      pb[i] = static_cast<short>(hb);
      psum += bf16_to_f32(hb);
      pex += pi;
    }
    // normalising by the sum of the rounded P keeps the weights a convex combination
    lsum = lsum * alpha + psum;
    lex = lex * alpha + pex;
    m = m_new;
    // V^T by transposed LDS reads: the 16 lanes of group grp read keys 4*grp..4*grp+3,
    // lane hl receives feature 16*jb + hl of those four keys
    const int vr = 4 * grp + hl / 4;
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb) {
      o[jb] *= alpha;
      LDS_AS v4bf* ap = (LDS_AS v4bf*)(vl + vr * C::PITCH + 16 * jb + 4 * (hl % 4));
      const v4s va4 = __builtin_bit_cast(v4s, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(ap));
      o[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va4, pb, o[jb], 0, 0, 0);
    }
  };

  // two named buffers (X for even chunks, Y for odd ones) and two entry
  // registers, so no register with a load in flight is ever copied: the loads
  // of chunk c+1 stay in flight while chunk c is computed
  if (nent > 0) {
    v8bf kx[C::NCH], ky[C::NCH];
    v4i vxx[D / 32], vxy[D / 32];
    int ex = entry(0);
    int ey = entry(16);
    issue(ex, kx, vxx);
    for (int e0 = 0; e0 < nent; e0 += 32) {
      issue(ey, ky, vxy);                     // chunk e0+16 (clamped reads if past the end)
      const bool vx_ok = ex >= 0 && ex < kvl;
      ex = entry(e0 + 32);
      // keep the scheduler from sinking these loads to their use
      __builtin_amdgcn_sched_barrier(0);
      compute(kx, vxx, vx_ok);
      if (e0 + 16 >= nent) break;
      issue(ex, kx, vxx);                     // chunk e0+32
      const bool vy_ok = ey >= 0 && ey < kvl;
      ey = entry(e0 + 48);
      __builtin_amdgcn_sched_barrier(0);
      compute(ky, vxy, vy_ok);
    }
  }

  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  lex += shfl_xor(lex, 16);
  lex += shfl_xor(lex, 32);
  if (!hok) return;
  if (splits > 1) {
    float* pp = part + ((qrow * Hq + h) * splits + split) * C::PART;
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb)
      *reinterpret_cast<v4f*>(pp + 16 * jb + 4 * grp) = o[jb];
    if (grp == 0) {
      pp[D] = m;
      pp[D + 1] = lsum;
      pp[D + 2] = lex;
    }
    return;
  }
  {
    const float inv = lsum > 0.f ? fast_rcp(lsum) : 0.f;
    const int64_t obase = (qrow * Hq + h) * D + 4 * grp;
    // all gate (and mix) loads in flight together (one memory latency)
    v2i gl[C::NJB] = {}, xl[C::NJB] = {};
    if (gate) {
#pragma unroll
      for (int jb = 0; jb < C::NJB; ++jb) gl[jb] = *reinterpret_cast<const v2i*>(gate + obase + 16 * jb);
      if (mix) {
#pragma unroll
        for (int jb = 0; jb < C::NJB; ++jb)
          xl[jb] = *reinterpret_cast<const v2i*>(mix + obase + 16 * jb);
      }
    }
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb) {
      float gv[4] = {1.f, 1.f, 1.f, 1.f};
      if (gate) {
        const uint32_t g01 = static_cast<uint32_t>(gl[jb].x), g23 = static_cast<uint32_t>(gl[jb].y);
        gv[0] = sigmoidf(bf16_to_f32(g01 & 0xffff));
        gv[1] = sigmoidf(bf16_to_f32(g01 >> 16));
        gv[2] = sigmoidf(bf16_to_f32(g23 & 0xffff));
        gv[3] = sigmoidf(bf16_to_f32(g23 >> 16));
      }
      float y[4];
      if (mix) {
        const uint32_t x01 = static_cast<uint32_t>(xl[jb].x), x23 = static_cast<uint32_t>(xl[jb].y);
        const uint16_t xs[4] = {static_cast<uint16_t>(x01), static_cast<uint16_t>(x01 >> 16),
                                static_cast<uint16_t>(x23), static_cast<uint16_t>(x23 >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = gate_mix(o[jb][e] * inv, gv[e], xs[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = o[jb][e] * inv * gv[e];
      }
      uint32_t w0 = f32_to_bf16(y[0]) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16);
      uint32_t w1 = f32_to_bf16(y[2]) | (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16);
      *reinterpret_cast<int2*>(out + obase + 16 * jb) = make_int2(static_cast<int>(w0), static_cast<int>(w1));
    }
    if (lse && grp == 0) lse[qrow * Hq + h] = lex > 0.f ? (m + fast_log2(lex)) * LN2 : -INFINITY;
  }
  }();
}

int sparse_attn_pick_splits(const Geom& g) {
  // one workgroup per CU or more, each with a long run of entries: on
  // Decode-128K (64 rows, K = 2048) 4 splits beat 8, 16 and 32 (gather +
  // combine 60 us against 66-94 us); each split keeps at least 64 listed
  // positions so its partial stays small against the gathered rows
  const int64_t rows = static_cast<int64_t>(g.B) * g.Tq;
  int splits = 1;
  while (rows * splits < 256 && g.K / (splits * 2) >= 64) splits *= 2;
  return splits;
}

size_t sparse_attn_workspace(const Geom& g, int splits) {
  if (splits <= 1) return dense_workspace(g);
  return static_cast<size_t>(g.B) * g.Tq * g.Hq * splits * (g.d + 4) * sizeof(float);
}

template <int D>
static hipError_t launch_d(const Geom& g, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                           const uint16_t* mix,
                           float scale, uint16_t* out, float* lse, int splits, void* ws,
                           bool masks_ready, hipStream_t st) {
  using C = AttnCfg<D>;
  const int G = g.Hq / g.Hkv;
  int per_split = (g.K + splits - 1) / splits;
  per_split = (per_split + 15) / 16 * 16;
  const uint8_t* done = nullptr;
  hipStream_t gst = st;  // the gather kernel's stream
  bool forked = false;
  OverlapStreams ov{};
  if (splits == 1) {
    const DenseMasks dm = dense_masks(g, ws);
    // masks from the Top-K kernel and histories no longer than lim: every row
    // is a tile-kernel row (valid ones qualify, empty ones are written there)
    const bool gather_work = !(masks_ready && g.Tk <= dm.lim);
    const int split = pick_overlap_split(g, dm.lim, gather_work);
    if (split >= 0) {
      // the tile path's flags and done bytes first, then the two kernels at
      // once on disjoint CUs (the tile kernel rewrites the same done bytes)
      hipError_t e0 = masks_ready ? hipSuccess : launch_dense_masks(g, idx, ws, st);
      if (e0 == hipSuccess) e0 = launch_dense_done(g, ws, st);
      if (e0 != hipSuccess) return e0;
      e0 = overlap_fork(split, st, &ov);
      if (e0 == hipSuccess) {
        forked = true;
        gst = ov.gather;
        e0 = launch_dense_attn(g, q, k, v, idx, gate, mix, scale, out, lse, ws, true, ov.tile);
      } else if (e0 == hipErrorNotSupported) {  // no library streams: one after the other
        e0 = launch_dense_attn(g, q, k, v, idx, gate, mix, scale, out, lse, ws, true, st);
      }
      if (e0 != hipSuccess) {
        if (forked) overlap_join(ov, st);
        return e0;
      }
    } else {
      hipError_t e0 =
          launch_dense_attn(g, q, k, v, idx, gate, mix, scale, out, lse, ws, masks_ready, st);
      if (e0 != hipSuccess) return e0;
      if (!gather_work) return hipSuccess;
    }
    done = dm.done;
  }
  // wave units of a row: the key/value heads, or the index sets when there are
  // more sets than key/value heads; up to 8 of them per workgroup
  const int units = std::max(g.sets, g.Hkv);
  const int Gu = g.Hq / units;
  const int nw = std::min(units, 8);
  const int nck = units / nw;
  // a grid of up to 8192 waves strides over the items (rows x splits x unit
  // chunks), so items the tile kernel finished cost one byte read each
  const int64_t nitems = static_cast<int64_t>(g.B) * g.Tq * splits * nck;
  dim3 grid(static_cast<uint32_t>(std::min<int64_t>(nitems, 8192 / nw)));
  const size_t lds = static_cast<size_t>(nw) * 16 * C::PITCH * sizeof(uint16_t);
  {
    KernelTimer timer(LCI_KERNEL_ATTN_GATHER, gst);
    hipLaunchKernelGGL((sparse_attn_kernel<D>), grid, dim3(64 * nw), lds, gst, g.Tq, g.Tk, g.K,
                       g.Hq, g.Hkv, G, g.sets, Gu, nck, g.kv_len, q, k, v, idx, gate, mix,
                       scale * LOG2E, out, lse, splits, per_split, static_cast<float*>(ws), done,
                       dense_block_rows(G), nitems);
  }
  hipError_t e = hipGetLastError();
  if (forked) {
    const hipError_t ej = overlap_join(ov, st);
    if (e == hipSuccess) e = ej;
  }
  if (e != hipSuccess || splits == 1) return e;
  dim3 cgrid(static_cast<uint32_t>(static_cast<int64_t>(g.B) * g.Tq), (g.Hq * (D / 2) + 255) / 256);
  {
    KernelTimer timer(LCI_KERNEL_ATTN_COMBINE, st);
    hipLaunchKernelGGL((attn_combine_kernel<D>), cgrid, dim3(256), 0, st, g.Hq, splits,
                       static_cast<const float*>(ws), gate, mix, out, lse);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const Geom& g, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                              const uint16_t* mix,
                              float scale, uint16_t* out, float* lse, int splits, void* ws,
                              bool masks_ready, hipStream_t st) {
  switch (g.d) {
    case 64:
      return launch_d<64>(g, q, k, v, idx, gate, mix, scale, out, lse, splits, ws, masks_ready, st);
    case 128:
      return launch_d<128>(g, q, k, v, idx, gate, mix, scale, out, lse, splits, ws, masks_ready, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
