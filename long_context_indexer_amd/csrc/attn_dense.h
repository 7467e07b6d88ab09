// Dense-tile path of sparse attention (see attn_dense.hip).
#pragma once

#include <algorithm>

#include "internal.h"

namespace lci {

// A query row takes the tile path when its causal history is at most
// kDenseFactor * K positions long (it then keeps at least 1/kDenseFactor of it).
// Measured on Prefill 64K (K = 2048): tiles cost about 17 ps per (row, causal
// key) and a gathered row about 0.5 us, so they break even near 14.5 K causal
// keys; the attention kernels together took 29.0, 26.9, 25.7, 25.2 and 25.6 ms
// with factors 4, 8, 12, 16 and 20.
constexpr int kDenseFactor = 16;
constexpr int kDenseMaxWords = (kDenseFactor * 4096 + 31) / 32;

int dense_block_rows(int G);
int dense_mask_words(const Geom& g);
size_t dense_workspace(const Geom& g);
// Builds masks/flags in `ws` (dense_workspace bytes; skipped when the Top-K
// kernel wrote them already), runs the tile kernel on every token block whose
// rows all qualify and marks those blocks done for the gather kernel.
hipError_t launch_dense_attn(const Geom& g, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* idx, const uint16_t* gate,
                             const uint16_t* mix,
                             float scale, uint16_t* out, float* lse, void* ws, bool masks_ready,
                             hipStream_t st);

}  // namespace lci
