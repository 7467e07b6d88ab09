// Dense-tile path of sparse attention for prefill rows whose selected set is a
// large fraction of their causal history (gfx950).
//
// The pages' own formulation ("From Linear Attention to Gated Sparse
// Attention", section 2 pseudocode: build a sparse mask from the Top-K
// positions, then run attention under that mask) computes the same thing as
// gathering the selected rows ("Hybrid Sparse Attention for Long-Context LLMs",
// section "Indexer + Top-K ...", step 3). When a query row keeps a sixteenth
// or more of its causal positions (always so for rows with p < K, where every
// position is kept), streaming contiguous key/value tiles through LDS and
// masking is cheaper than gathering 2 KiB per selected position: each key tile
// is loaded once for 4*32 query rows instead of once per row.
//
// Two kernels:
//   idx_mask_kernel  turns each index row into a bit mask over positions and a
//                    row flag: 2 = the row keeps exactly 0..p, 1 = masked tile
//                    path, 0 = leave the row to the gather kernel (index rows
//                    that are not strictly increasing positions in 0..p, or
//                    rows too sparse for tiles). Every tile-path row gets its
//                    mask (all of 0..p for flag 2).
//   attn_dense_kernel one workgroup = 4 waves = 4*32 (token, query head) rows of
//                    one key/value head g; waves own 32/G tokens x G heads.
//                    Per 64-key tile: K and V tiles go from HBM straight into
//                    LDS (double buffered: V of the next tile and K of the one
//                    after are in flight while this one is computed; one
//                    barrier per tile), then
//                      S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (lane l owns
//                            query row l%32, keys 8i+4*(l/32)+j of each 32-key half),
//                      the row's selection applied by the accumulators'
//                            start values (0 for a kept key, -FLT_MAX for a
//                            dropped one, four keys per LDS table entry),
//                      online softmax in base 2 (max on raw scores,
//                            the scale folded into one FMA per exponent, the
//                            offset moved only when a row's max grows by 2^8),
//                            all lane-local except one exchange with lane l^32,
//                      O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, with V^T read
//                            by ds_read_b64_tr_b16 (each 16-lane group reads a
//                            4-key x 16-feature block transposed into registers).
//                    The epilogue applies the gate (sigmoid(gate) * o, or
//                    mixed with the other branch's output) and stores bf16.
// K and V tiles use an XOR-swizzled LDS layout that keeps every access pattern
// free of bank conflicts. Workgroups are placed so that each XCD (its own L2)
// serves one key/value head (blockIdx.x % 8 picks the XCD), and the longest
// causal tiles start first.
#include <type_traits>

#include "attn_dense.h"
#include "common.h"
#include "../../include/lci.h"
#include "internal.h"
#include "tile.h"

namespace lci {

// ------------------------------------------------------------------ masks

__global__ __launch_bounds__(256) void idx_mask_kernel(
    int Tq, int Tk, int K, int sets, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ idx, int lim, int Wm,
    uint32_t* __restrict__ mask, uint8_t* __restrict__ flag) {
  __shared__ uint32_t bits[kDenseMaxWords];
  __shared__ uint32_t red[8];
  // rows [B][sets][Tq], like the index rows
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / (static_cast<int64_t>(sets) * Tq));
  const int i = static_cast<int>(row % Tq);
  const int kvl = kv_len[b];
  const int64_t p = static_cast<int64_t>(q_offset[b]) + i;
  const bool eligible = kvl <= Tk && p >= 0 && p < kvl && p + 1 <= lim;
  if (!eligible) {
    if (threadIdx.x == 0) flag[row] = kRowGather;
    return;
  }
  for (int w = threadIdx.x; w < Wm; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  const int32_t* ir = idx + row * K;
  int bad = 0;
  uint32_t cnt = 0;
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    const int s = ir[j];
    if (s == -1) {
      // padding may only follow padding
      if (j + 1 < K && ir[j + 1] != -1) bad = 1;
      continue;
    }
    if (s < 0 || s > p) {
      bad = 1;
      continue;
    }
    if (j > 0 && !(ir[j - 1] >= 0 && ir[j - 1] < s)) bad = 1;
    atomicOr(&bits[s >> 5], 1u << (s & 31));
    ++cnt;
  }
  bad = __syncthreads_or(bad);
  cnt = wave_sum(cnt);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
  __syncthreads();
  uint32_t tot = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += red[w];
  const uint8_t f = bad ? kRowGather : (tot == static_cast<uint32_t>(p + 1) ? kRowAll : kRowMasked);
  if (threadIdx.x == 0) flag[row] = f;
  // a row that keeps all of 0..p has exactly those bits set
  if (f != kRowGather)
    for (int w = threadIdx.x; w < Wm; w += blockDim.x) mask[row * Wm + w] = bits[w];
}

// ------------------------------------------------------------ tile kernel

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Lanes l and l^32 combined, with no LDS round trip: v_permlane32_swap of a
// value with itself returns v[l % 32] in one result and v[l % 32 + 32] in the
// other, on every lane.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows whose running max grows by less than this (log2 units) keep their
// softmax offset: P stays <= 2^8, far from overflow, and the O and l rescale
// is skipped for the whole wave unless some row needs it.
constexpr float kRescaleLog2 = 8.0f;

// A dropped key's score starts from -FLT_MAX: adding the QK products of finite
// bf16 rows leaves it at or below -2^127, under any kept score, and its
// exponential underflows to 0. A tile whose maximum is that low kept nothing.
constexpr uint32_t kDroppedBits = 0xff7fffffu;
constexpr float kDroppedMax = -0x1p127f;

// EXACT_L: the softmax denominator sums the fp32 probabilities (needed for the
// log-sum-exp output). Otherwise it sums the bf16-rounded ones that enter the
// PV product, two per dot-product instruction.
// MIX: the gate mixes the output with the other branch's (mix non-null). A
// template flag, not a runtime test: the extra epilogue registers change the
// allocation of the main loop, which costs the unmixed kernel about 4%.
template <int D, int G, bool EXACT_L, bool MIX>
__global__ __launch_bounds__(256, 2) void attn_dense_kernel(
    int Tq, int Tk, int Hq, int Hkv, const int32_t* __restrict__ q_offset,
    const int32_t* __restrict__ kv_len, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ gate, const uint16_t* __restrict__ mix,
    const uint32_t* __restrict__ mask, int Wm,
    const uint8_t* __restrict__ flag, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint8_t* __restrict__ done, int nbps, int nblk, int sets) {
  using C = DenseCfg<D, G>;
  // two K and two V tile buffers (see the pipeline below)
  __shared__ __align__(16) uint16_t ks[2][C::BK * C::KP];
  __shared__ __align__(16) uint16_t vsh[2][C::BK * C::KP];
  uint16_t* const ks0 = ks[0];
  uint16_t* const ks1 = ks[1];
  uint16_t* const vs0 = vsh[0];
  uint16_t* const vs1 = vsh[1];
  // score accumulator start values of four consecutive keys under a 4-bit
  // selection nibble: 0 where the bit keeps the key, the most negative finite
  // float where it drops it (the QK products then leave it far below any score)
  __shared__ __align__(16) uint32_t mlut[16][4];
  if (threadIdx.x < 64) {
    const int nib = threadIdx.x >> 2, bit = threadIdx.x & 3;
    mlut[nib][bit] = ((nib >> bit) & 1) ? 0u : kDroppedBits;
  }

  // XCD-aware placement: XCD x = blockIdx.x % 8 serves key/value head x / (8/Hkv)
  const int per = 8 / Hkv;
  const int xcd = blockIdx.x & 7;
  const int g = xcd / per;
  const int blk = (blockIdx.x >> 3) * per + xcd % per;
  if (blk >= nblk) return;
  const int b = blk / nbps;
  const int tb = nbps - 1 - blk % nbps;  // longest causal range first
  const int i0 = tb * C::BQ;
  const int iend = min(i0 + C::BQ, Tq);
  // masks, flags and done bytes are per index set ([B][sets][...]); query head
  // h reads set h / hps, so this workgroup's heads g*G .. g*G + G - 1 read
  // sets s0 .. s0 + nsg - 1
  const int hps = Hq / sets;
  const int s0 = g * G / hps;
  const int nsg = G > hps ? G / hps : 1;

  // the whole token block must be on this path, in every set its heads read
  // (BQ * nsg <= BQ * G = 128 rows)
  int ok = 1;
  {
    const int t = threadIdx.x;
    const int it = i0 + t / nsg;
    if (t < C::BQ * nsg && it < Tq)
      ok = flag[(static_cast<int64_t>(b) * sets + s0 + t % nsg) * Tq + it] != 0;
  }
  const int all_ok = __syncthreads_and(ok);
  // the gather kernel skips the token blocks this kernel takes
  if (static_cast<int>(threadIdx.x) < nsg)
    done[(static_cast<int64_t>(b) * sets + s0 + threadIdx.x) * nbps + tb] = all_ok ? 1 : 0;
  if (all_ok == 0) return;

  const int qo = q_offset[b];
  // a history longer than its allocation (every row of it is empty) reads no tile
  const int kvl0 = kv_len[b];
  const int kvl = __builtin_amdgcn_readfirstlane(kvl0 <= Tk ? max(kvl0, 0) : 0);
  // last key any row of the block reads (rows past the history read none)
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
  const int64_t srow = (static_cast<int64_t>(b) * sets + h / hps) * Tq;  // row 0 of h's set
  const int fl = rv ? flag[srow + i] : 0;
  const uint32_t* mrow = mask + (srow + (rv ? i : 0)) * Wm;

  // Q^T as the B operand: lane holds Q[row][16*kk + 8*hf .. +7]
  v8bf qf[C::NKK];
  {
    const uint16_t* qp = q + (qrow * Hq + h) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      v4i z = {0, 0, 0, 0};
      v4i t = rv ? *reinterpret_cast<const v4i*>(qp + 16 * kk) : z;
      qf[kk] = __builtin_bit_cast(v8bf, t);
    }
  }

  // K/V tiles go from HBM straight into LDS (buffer_load ... lds: lane l of a
  // wave writes 16 bytes at the instruction's LDS base + 16 l). Wave wv's c-th
  // load fills LDS bytes [1024 (4c + wv), +1024) of the tile, i.e. RPI whole
  // rows; each lane fetches the logical 16-byte unit that the XOR swizzle puts
  // at its physical slot. The buffer resource starts at the tile's first key and
  // ends at the last valid one: keys past kv_len read as zero (finite, masked).
  constexpr int UPR = D / 8;             // 16-byte units per row
  constexpr int RPI = 64 / UPR;          // rows per wave load
  constexpr int NI = C::BK * UPR / 256;  // loads per wave per tile (K and V each)
  const int rowstep = Hkv * D;           // elements between consecutive keys
  // tile addresses and sizes are workgroup-uniform: kept in scalar registers
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
  auto tile_rsrc = [&](const uint16_t* base, int kb) {
    // key0 < kv_len for every tile loaded, so at least one key is valid
    const int key0 = kb * C::BK;
    const int nvalid = min(kvl - key0, C::BK);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base) + static_cast<int64_t>(key0) * rowstep,
                                             0, nvalid * rowstep * 2, kBufferFlags);
  };
  auto load_tile = [&](const uint16_t* base, int kb, uint16_t* dst) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, kb);
#pragma unroll
    for (int c = 0; c < NI; ++c)
      load16_to_lds(rs, (LDS_AS uint16_t*)dst + (4 * c + wv) * 512, voff[c]);
  };

  // S^T of one 64-key tile (two 32-key halves) from the K tile in LDS, the
  // selection applied by the accumulator's start values: element e of half kt
  // (key 32kt + 8(e/4) + 4hf + e%4) starts from the LUT entry of its nibble
  auto tile_scores = [&](const uint16_t* kt_lds, const uint32_t* mw2, v16f* st) {
    const LDS_AS uint16_t* ksl = (const LDS_AS uint16_t*)kt_lds;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint32_t mw = mw2[kt] >> (4 * hf);
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const v4i z = *(const LDS_AS v4i*)(&mlut[(mw >> (8 * jn)) & 15u][0]);
#pragma unroll
        for (int c = 0; c < 4; ++c) st[kt][4 * jn + c] = __int_as_float(z[c]);
      }
      const int krow = 32 * kt + r;
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        const v8bf a = __builtin_bit_cast(
            v8bf, *(const LDS_AS v4i*)(ksl + tile_off<D>(krow, 16 * kk + 8 * hf)));
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st[kt], 0, 0, 0);
      }
    }
  };

  // selection words of a tile, loaded two tiles ahead of its softmax, so they
  // are in registers (the step's barrier waited for them) when its scores are
  // computed. Rows hold an even number of words, two per 64-key tile up to the
  // row limit, so every tile of the block has its words; the index is clamped
  // only for the tiles past the last, whose scores are never used (rows not on
  // the mask path read a valid but unused word too).
  const int wlast = Wm - 1;
  auto mask_words = [&](int kb, uint32_t* w) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) w[kt] = mrow[min(2 * kb + kt, wlast)];
  };

  float m = -INFINITY;  // softmax offset of this row, raw score units (a running max)
  float lsum = 0.f;     // this lane's share of the softmax denominator
  v16f o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;

  // pipeline: while tile kb is in softmax, the scores of tile kb+1 are computed
  // (their K is already in LDS) and V of kb+1 and K of kb+2 are in flight
  if (nkb > 0) {
    load_tile(kbase, 0, ks0);
    load_tile(vbase, 0, vs0);
  }
  if (nkb > 1) load_tile(kbase, 1, ks1);
  uint32_t mw0[2], mwn[2];  // words of tiles 0 and (the next tile) 1
  mask_words(0, mw0);
  mask_words(1, mwn);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // every load done (see the step's end)
  __syncthreads();
  v16f sc[2];
  tile_scores(ks0, mw0, sc);
  __syncthreads();  // every wave is done with K tile 0 before tile 2 replaces it

  // one step per tile; the steps of even and odd tiles are separate copies
  // so each has its buffer addresses as constants
  auto tile_step = [&](int kb, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    uint16_t* const kcur = buf ? ks1 : ks0;  // K of tile kb (scored), refilled with kb+2
    uint16_t* const knxt = buf ? ks0 : ks1;  // K of tile kb+1
    uint16_t* const vcur = buf ? vs1 : vs0;  // V of tile kb
    uint16_t* const vnxt = buf ? vs0 : vs1;  // filled with V of tile kb+1
    if (kb + 1 < nkb) load_tile(vbase, kb + 1, vnxt);
    if (kb + 2 < nkb) load_tile(kbase, kb + 2, kcur);
    uint32_t mwa[2];  // words of tile kb + 2
    mask_words(kb + 2, mwa);

    // scores are finite (dropped keys near -FLT_MAX): IEEE maximum (no NaN
    // quieting) folds into v_maximum3
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = max3f(mx, sc[kt][e], sc[kt][e + 1]);
    mx = max_xor32(mx);
    if (mx < kDroppedMax) mx = -INFINITY;  // no key of this tile kept
    // lazy offset update: only rows whose max grew by kRescaleLog2 or more move
    // their offset (all rows start at -inf, so every row moves on its first
    // kept score); the rescale of O and l runs only if some row of the wave moved
    const bool grow = mx * scale_log2 > m * scale_log2 + kRescaleLog2;
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      // a row with nothing kept yet has O = l = 0: alpha = 2^-inf = 0, never 0*inf
      const float moff_new = (m_new == -INFINITY) ? 0.f : m_new * scale_log2;
      const float alpha = fast_exp2(m * scale_log2 - moff_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= alpha;
    }
    // a row with nothing kept so far has m = -inf: offset 0 (every p is 0)
    const float moff = (m == -INFINITY) ? 0.f : m * scale_log2;

    // scores of the next tile (independent MFMA work beside the exponentials;
    // past the last tile the result is unused)
    v16f sn[2];
    tile_scores(knxt, mwn, sn);

    // P^T as the B operand of the PV step s: e<4 -> half-row i=2(s%2), e>=4 -> i=2(s%2)+1
    v8bf pb[4];
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(sc[kt][e], scale_log2, -moff));
        if constexpr (EXACT_L) psum += pe;
        pb[2 * kt + (e >> 3)][e & 7] = static_cast<__bf16>(pe);
      }
    if constexpr (!EXACT_L) {
      const v2bf one2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
      float ps2 = 0.f;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const v8bf x = pb[qq];
        psum = __builtin_amdgcn_fdot2_f32_bf16(v2bf{x[0], x[1]}, one2, psum, false);
        ps2 = __builtin_amdgcn_fdot2_f32_bf16(v2bf{x[2], x[3]}, one2, ps2, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(v2bf{x[4], x[5]}, one2, psum, false);
        ps2 = __builtin_amdgcn_fdot2_f32_bf16(v2bf{x[6], x[7]}, one2, ps2, false);
      }
      psum += ps2;
    }
    lsum += psum;

    // O^T += V^T P^T over the 64 keys, four 16-key steps
    const LDS_AS uint16_t* vsl = (const LDS_AS uint16_t*)(vcur);
    const int gi = lane & 15;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int d0 = 32 * dt + 16 * ((lane >> 4) & 1);
        const int k0 = 16 * s2 + 4 * hf;
        LDS_AS v4bf* a0 = (LDS_AS v4bf*)(vsl + tile_off<D>(k0 + gi / 4, d0 + 4 * (gi % 4)));
        LDS_AS v4bf* a1 = (LDS_AS v4bf*)(vsl + tile_off<D>(k0 + 8 + gi / 4, d0 + 4 * (gi % 4)));
        const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a0);
        const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a1);
        const v8bf a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], o[dt], 0, 0, 0);
      }
    }
    sc[0] = sn[0];
    sc[1] = sn[1];
    mwn[0] = mwa[0];
    mwn[1] = mwa[1];
    // the barrier waits for this step's tile loads (vmcnt) and makes them
    // visible; it also guarantees every wave is done with the buffers the
    // next step's loads overwrite. The selection words loaded this step are
    // waited for here too (vmcnt 0, other counters untouched): waiting for
    // them later, behind the next step's tile loads, would wait for those.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    tile_step(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < nkb) tile_step(kb + 1, std::integral_constant<int, 1>{});
  }

  lsum = sum_xor32(lsum);
  if (!rv || fl == kRowGather) return;  // an empty row (nothing kept) writes 0 and -inf
  const float inv = lsum > 0.f ? fast_rcp(lsum) : 0.f;
  const int64_t obase = (qrow * Hq + h) * D;
  // every gate (and mix) load is issued before any is used (one memory
  // latency, not one per 8-byte piece); bf16 0 = logit 0 is never read
  // without a gate
  v2i graw[C::NDT][4] = {};
  if (gate) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        graw[dt][ii] = *reinterpret_cast<const v2i*>(gate + obase + 32 * dt + 8 * ii + 4 * hf);
  }
  v2i xraw[MIX ? C::NDT : 1][4] = {};
  if constexpr (MIX) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        xraw[dt][ii] = *reinterpret_cast<const v2i*>(mix + obase + 32 * dt + 8 * ii + 4 * hf);
  }
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = 32 * dt + 8 * ii + 4 * hf;
      float gv[4] = {1.f, 1.f, 1.f, 1.f};
      if (gate) {
        const uint32_t g01 = static_cast<uint32_t>(graw[dt][ii].x);
        const uint32_t g23 = static_cast<uint32_t>(graw[dt][ii].y);
        gv[0] = sigmoidf(bf16_to_f32(g01 & 0xffff));
        gv[1] = sigmoidf(bf16_to_f32(g01 >> 16));
        gv[2] = sigmoidf(bf16_to_f32(g23 & 0xffff));
        gv[3] = sigmoidf(bf16_to_f32(g23 >> 16));
      }
      if constexpr (MIX) {
        const uint32_t x01 = static_cast<uint32_t>(xraw[dt][ii].x);
        const uint32_t x23 = static_cast<uint32_t>(xraw[dt][ii].y);
        const uint16_t xs[4] = {static_cast<uint16_t>(x01), static_cast<uint16_t>(x01 >> 16),
                                static_cast<uint16_t>(x23), static_cast<uint16_t>(x23 >> 16)};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = gate_mix(o[dt][4 * ii + e] * inv, gv[e], xs[e]);
        const uint32_t w0 = f32_to_bf16(y[0]) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16);
        const uint32_t w1 = f32_to_bf16(y[2]) | (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16);
        *reinterpret_cast<int2*>(out + obase + d) = make_int2(static_cast<int>(w0), static_cast<int>(w1));
      } else {
        const uint32_t w0 = f32_to_bf16(o[dt][4 * ii] * inv * gv[0]) |
                            (static_cast<uint32_t>(f32_to_bf16(o[dt][4 * ii + 1] * inv * gv[1])) << 16);
        const uint32_t w1 = f32_to_bf16(o[dt][4 * ii + 2] * inv * gv[2]) |
                            (static_cast<uint32_t>(f32_to_bf16(o[dt][4 * ii + 3] * inv * gv[3])) << 16);
        *reinterpret_cast<int2*>(out + obase + d) = make_int2(static_cast<int>(w0), static_cast<int>(w1));
      }
    }
  if (lse && hf == 0) lse[qrow * Hq + h] = lsum > 0.f ? (m * scale_log2 + fast_log2(lsum)) * LN2 : -INFINITY;
}

// ---------------------------------------------------------------- host side

int dense_block_rows(int G) { return 4 * (32 / G); }

// The done bytes the tile kernel writes, from the row flags alone: token block
// tb of set s is the tile kernel's when every row of it, in every set the
// workgroup's query heads read (nsg consecutive sets), is a tile row.
__global__ __launch_bounds__(256) void dense_done_kernel(int Tq, int sets, int nsg, int BQ,
                                                         int nbps,
                                                         const uint8_t* __restrict__ flag,
                                                         uint8_t* __restrict__ done, int64_t n) {
  for (int64_t x = blockIdx.x * 256LL + threadIdx.x; x < n; x += gridDim.x * 256LL) {
    const int64_t bs = x / nbps;  // b * sets + s
    const int tb = static_cast<int>(x - bs * nbps);
    const int s = static_cast<int>(bs % sets);
    const int64_t b = bs / sets;
    const int sg0 = s - s % nsg;
    const int i1 = min(tb * BQ + BQ, Tq);
    int ok = 1;
    for (int s2 = sg0; s2 < sg0 + nsg; ++s2)
      for (int i = tb * BQ; i < i1; ++i) ok &= flag[(b * sets + s2) * Tq + i] != 0;
    done[x] = ok ? 1 : 0;
  }
}

int dense_row_limit(const Geom& g) {
  return static_cast<int>(std::min<int64_t>(static_cast<int64_t>(kDenseFactor) * g.K, g.Tk));
}

// two words per 64-key tile: the tile kernel reads a tile's words as a pair
int dense_mask_words(const Geom& g) { return 2 * ((dense_row_limit(g) + 63) / 64); }

// [mask: rows x Wm words][flag: rows bytes][done: one byte per token block
// (at most one block per row)], each part 256-byte aligned; rows = B x sets x Tq
size_t dense_workspace(const Geom& g) {
  const size_t rows = static_cast<size_t>(g.B) * g.sets * g.Tq;
  const size_t mbytes = (rows * dense_mask_words(g) * sizeof(uint32_t) + 255) & ~size_t(255);
  return mbytes + 2 * ((rows + 255) & ~size_t(255));
}

DenseMasks dense_masks(const Geom& g, void* ws) {
  const size_t rows = static_cast<size_t>(g.B) * g.sets * g.Tq;
  DenseMasks d;
  d.Wm = dense_mask_words(g);
  d.lim = dense_row_limit(g);
  char* base = static_cast<char*>(ws);
  const size_t mbytes = (rows * d.Wm * sizeof(uint32_t) + 255) & ~size_t(255);
  d.mask = reinterpret_cast<uint32_t*>(base);
  d.flag = reinterpret_cast<uint8_t*>(base + mbytes);
  d.done = reinterpret_cast<uint8_t*>(base + mbytes + ((rows + 255) & ~size_t(255)));
  return d;
}

template <int D, int G, bool EXACT_L, bool MIX>
static hipError_t launch_dense_k(const Geom& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const uint16_t* gate,
                                  const uint16_t* mix, float scale,
                                  uint16_t* out, float* lse, const DenseMasks& dm,
                                  hipStream_t st) {
  using C = DenseCfg<D, G>;
  const int nbps = (g.Tq + C::BQ - 1) / C::BQ;
  const int nblk = g.B * nbps;
  const int per = 8 / g.Hkv;
  const int64_t nwg = static_cast<int64_t>((nblk + per - 1) / per) * 8;
  {
    KernelTimer timer(LCI_KERNEL_ATTN_DENSE, st);
    hipLaunchKernelGGL((attn_dense_kernel<D, G, EXACT_L, MIX>), dim3(static_cast<uint32_t>(nwg)),
                       dim3(256), 0, st,
                       g.Tq, g.Tk, g.Hq, g.Hkv, g.q_offset, g.kv_len, q, k, v, gate, mix, dm.mask,
                       dm.Wm, dm.flag, scale * LOG2E, out, lse, dm.done, nbps, nblk, g.sets);
  }
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_dense_dg(const Geom& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const uint16_t* gate,
                                  const uint16_t* mix, float scale,
                                  uint16_t* out, float* lse, const DenseMasks& dm,
                                  hipStream_t st) {
  if (gate && mix)
    return lse ? launch_dense_k<D, G, true, true>(g, q, k, v, gate, mix, scale, out, lse, dm, st)
               : launch_dense_k<D, G, false, true>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
  return lse ? launch_dense_k<D, G, true, false>(g, q, k, v, gate, nullptr, scale, out, lse, dm, st)
             : launch_dense_k<D, G, false, false>(g, q, k, v, gate, nullptr, scale, out, lse, dm, st);
}

template <int D>
static hipError_t launch_dense_d(const Geom& g, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* gate,
                                 const uint16_t* mix, float scale,
                                 uint16_t* out, float* lse, const DenseMasks& dm, hipStream_t st) {
  switch (g.Hq / g.Hkv) {
    case 1: return launch_dense_dg<D, 1>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    case 2: return launch_dense_dg<D, 2>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    case 4: return launch_dense_dg<D, 4>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    case 8: return launch_dense_dg<D, 8>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    case 16: return launch_dense_dg<D, 16>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dense_masks(const Geom& g, const int32_t* idx, void* ws, hipStream_t st) {
  const DenseMasks dm = dense_masks(g, ws);
  const size_t rows = static_cast<size_t>(g.B) * g.sets * g.Tq;
  KernelTimer timer(LCI_KERNEL_IDX_MASK, st);
  hipLaunchKernelGGL(idx_mask_kernel, dim3(static_cast<uint32_t>(rows)), dim3(256), 0, st, g.Tq,
                     g.Tk, g.K, g.sets, g.q_offset, g.kv_len, idx, dm.lim, dm.Wm, dm.mask,
                     dm.flag);
  return hipGetLastError();
}

hipError_t launch_dense_done(const Geom& g, void* ws, hipStream_t st) {
  const DenseMasks dm = dense_masks(g, ws);
  const int G = g.Hq / g.Hkv;
  const int BQ = dense_block_rows(G);
  const int nbps = (g.Tq + BQ - 1) / BQ;
  const int hps = g.Hq / g.sets;
  const int nsg = G > hps ? G / hps : 1;
  const int64_t n = static_cast<int64_t>(g.B) * g.sets * nbps;
  hipLaunchKernelGGL(dense_done_kernel,
                     dim3(static_cast<uint32_t>(std::min<int64_t>((n + 255) / 256, 4096))),
                     dim3(256), 0, st, g.Tq, g.sets, nsg, BQ, nbps, dm.flag, dm.done, n);
  return hipGetLastError();
}

hipError_t launch_dense_attn(const Geom& g, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                             const uint16_t* mix,
                             float scale, uint16_t* out, float* lse, void* ws, bool masks_ready,
                             hipStream_t st) {
  const DenseMasks dm = dense_masks(g, ws);
  hipError_t e = masks_ready ? hipGetLastError() : launch_dense_masks(g, idx, ws, st);
  if (e != hipSuccess) return e;
  switch (g.d) {
    case 64: return launch_dense_d<64>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    case 128: return launch_dense_d<128>(g, q, k, v, gate, mix, scale, out, lse, dm, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lci
