// Measurement aid for bench.py (not part of the library): the rate at which
// this GPU gathers randomly chosen rows of a table, the access pattern of the
// gather attention kernel (every selected position's key and value rows read
// once per query row from a working set the size of the key/value cache).
//
// bench_gather_probe reads rows idx[0..n) of `table` (rows of row_bytes bytes,
// 256 or 1024), XOR-folds them and writes one word per thread to `out` (so no
// load can be dropped), on `stream`. Each wave keeps eight 16-byte loads per
// lane in flight. Returns a hipError_t code (hipErrorInvalidValue for an
// unsupported row size, a table of fewer rows than an index names is the
// caller's error). `out` holds 2048 * 256 words.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kGrid = 2048;
constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int R>
__global__ __launch_bounds__(kThreads) void gather_probe_kernel(const u32x4* __restrict__ table,
                                                                const int32_t* __restrict__ idx,
                                                                int64_t n, uint32_t* __restrict__ out) {
  constexpr int LPR = R / 16;        // lanes per row (16-byte pieces)
  constexpr int RPI = 64 / LPR;      // rows per load instruction
  constexpr int RPS = RPI * kInFlight;  // rows per wave step
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  const int64_t nw = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t r0 = w0 * RPS; r0 + RPS <= n; r0 += nw * RPS) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t row = idx[r0 + u * RPI + lane / LPR];
      v[u] = table[row * LPR + lane % LPR];
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" int bench_gather_probe(const void* table, int row_bytes, const int32_t* idx, int64_t n,
                                  uint32_t* out, hipStream_t stream) {
  const u32x4* t = static_cast<const u32x4*>(table);
  switch (row_bytes) {
    case 256:
      hipLaunchKernelGGL(gather_probe_kernel<256>, dim3(kGrid), dim3(kThreads), 0, stream, t, idx, n, out);
      break;
    case 1024:
      hipLaunchKernelGGL(gather_probe_kernel<1024>, dim3(kGrid), dim3(kThreads), 0, stream, t, idx, n, out);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}
