// Appending new rows to the key, value and indexer-key caches (gfx950).
//
// "Hybrid Sparse Attention for Long-Context LLMs", section "Engineering and
// Evaluation Recommendations": long prompts are prefilled in chunks that reuse
// what is already cached for the scorer. The caches hold, per sequence and
// position, the key and value rows and the indexer key; a chunk of prompt rows
// or a decoded token is appended right after the history, and the following
// prefill or decode call scores and attends against the cache without
// recomputing anything for earlier rows.
//
// Two launches on the caller's stream:
//   kv_append_kernel   a pure copy: workgroup (x, b) moves rows
//                      [8x, 8x + 8) of sequence b, every lane 16-byte units,
//                      all loads of a lane issued before its stores. HBM-bound.
//   kv_lengths_kernel  the new lengths and first positions. It runs after every
//                      copy has read the old lengths, so its output may
//                      overwrite them in place.
#include "../../include/lci.h"
#include "internal.h"

namespace lci {

namespace {

constexpr int kAppendRows = 8;  // rows per workgroup
constexpr int kAppendNT = 256;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Units of 16 bytes: uk per key (and value) row, ui per indexer-key row.
__global__ __launch_bounds__(kAppendNT) void kv_append_kernel(
    int Tn, int Tk, int uk, int ui, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ n_new, const int4* __restrict__ k_new,
    const int4* __restrict__ v_new, const int4* __restrict__ kI_new, int4* __restrict__ k_cache,
    int4* __restrict__ v_cache, int4* __restrict__ kI_cache) {
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kAppendRows;
  const int old = clampi(kv_len[b], 0, Tk);
  const int n = clampi(n_new ? n_new[b] : Tn, 0, Tn);
  // rows of this workgroup that are appended and land inside the cache
  const int rows = min(min(n, Tk - old) - t0, kAppendRows);
  if (rows <= 0) return;
  const int64_t src_row = static_cast<int64_t>(b) * Tn + t0;
  const int64_t dst_row = static_cast<int64_t>(b) * Tk + old + t0;
  // keys and values: rows * uk units each, contiguous in source and destination
  const int nkv = rows * uk;
  const int4* ks = k_new + src_row * uk;
  const int4* vs = v_new + src_row * uk;
  int4* kd = k_cache + dst_row * uk;
  int4* vd = v_cache + dst_row * uk;
  constexpr int U = 4;  // units in flight per lane and tensor
  for (int u0 = threadIdx.x; u0 < nkv; u0 += U * kAppendNT) {
    int4 a[U], c[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = min(u0 + j * kAppendNT, nkv - 1);
      a[j] = ks[u];
      c[j] = vs[u];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * kAppendNT;
      if (u < nkv) {
        kd[u] = a[j];
        vd[u] = c[j];
      }
    }
  }
  const int ni = rows * ui;
  const int4* is = kI_new + src_row * ui;
  int4* id = kI_cache + dst_row * ui;
  for (int u = threadIdx.x; u < ni; u += kAppendNT) id[u] = is[u];
}

// q_offset_out[b] = old length (the position of the first new row),
// kv_len_out[b] = min(old + n, Tk). One thread per sequence reads its old
// length before writing either output.
__global__ __launch_bounds__(kAppendNT) void kv_lengths_kernel(
    int B, int Tn, int Tk, const int32_t* kv_len, const int32_t* __restrict__ n_new,
    int32_t* q_offset_out, int32_t* kv_len_out) {
  for (int b = blockIdx.x * kAppendNT + threadIdx.x; b < B; b += gridDim.x * kAppendNT) {
    const int old = clampi(kv_len[b], 0, Tk);
    const int n = clampi(n_new ? n_new[b] : Tn, 0, Tn);
    if (q_offset_out) q_offset_out[b] = old;
    if (kv_len_out) kv_len_out[b] = min(old + n, Tk);
  }
}

}  // namespace

hipError_t launch_kv_append(const Geom& g, const uint16_t* k_new, const uint16_t* v_new,
                            const int8_t* kI_new, const int32_t* n_new, uint16_t* k_cache,
                            uint16_t* v_cache, int8_t* kI_cache, int32_t* q_offset_out,
                            int32_t* kv_len_out, hipStream_t st) {
  const int uk = g.Hkv * g.d * 2 / 16;
  const int ui = g.d_I / 16;
  dim3 grid(static_cast<uint32_t>((g.Tq + kAppendRows - 1) / kAppendRows), static_cast<uint32_t>(g.B));
  {
    KernelTimer timer(LCI_KERNEL_KV_APPEND, st);
    hipLaunchKernelGGL(kv_append_kernel, grid, dim3(kAppendNT), 0, st, g.Tq, g.Tk, uk, ui,
                       g.kv_len, n_new, reinterpret_cast<const int4*>(k_new),
                       reinterpret_cast<const int4*>(v_new), reinterpret_cast<const int4*>(kI_new),
                       reinterpret_cast<int4*>(k_cache), reinterpret_cast<int4*>(v_cache),
                       reinterpret_cast<int4*>(kI_cache));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!q_offset_out && !kv_len_out)) return e;
  {
    KernelTimer timer(LCI_KERNEL_KV_LENGTHS, st);
    hipLaunchKernelGGL(kv_lengths_kernel, dim3(static_cast<uint32_t>((g.B + kAppendNT - 1) / kAppendNT)),
                       dim3(kAppendNT), 0, st, g.B, g.Tq, g.Tk, g.kv_len, n_new, q_offset_out,
                       kv_len_out);
  }
  return hipGetLastError();
}

}  // namespace lci
