// Index sets per key/value head (gfx950): the indexer heads of each set as a
// contiguous query array.
//
// With one index set per key/value head (the per-head index rows of the pages'
// pseudocode: "Hybrid Sparse Attention for Long-Context LLMs", Indexer + Top-K
// section), set g is scored by indexer heads g*Hg .. g*Hg + Hg - 1 (Hg =
// H_I/sets). q_idx rows hold all H_I heads; this copy gathers each set's heads
// into [sets][B][Tq][Hg][d_I], so the scoring kernels run on a set as on an
// indexer of Hg heads. A 16-byte-unit copy, HBM-bound (the query rows are small
// beside the history they are scored against).
#include <algorithm>

#include "../../include/lci.h"
#include "internal.h"

namespace lci {

namespace {

__global__ __launch_bounds__(256) void regroup_q_idx_kernel(int64_t rows, int units_row,
                                                            int units_set,
                                                            const int4* __restrict__ src,
                                                            int4* __restrict__ dst) {
  const int64_t total = rows * units_row;
  for (int64_t u = blockIdx.x * 256LL + threadIdx.x; u < total; u += gridDim.x * 256LL) {
    const int64_t row = u / units_row;
    const int c = static_cast<int>(u - row * units_row);
    const int gs = c / units_set;
    dst[(gs * rows + row) * units_set + (c - gs * units_set)] = src[u];
  }
}

}  // namespace

hipError_t launch_regroup_q_idx(const Geom& g, const int8_t* q_idx, int8_t* out,
                                hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(g.B) * g.Tq;
  const int units_row = g.H_I * g.d_I / 16;
  const int units_set = units_row / g.sets;
  const int64_t total = rows * units_row;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(regroup_q_idx_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                     rows, units_row, units_set, reinterpret_cast<const int4*>(q_idx),
                     reinterpret_cast<int4*>(out));
  return hipGetLastError();
}

}  // namespace lci
