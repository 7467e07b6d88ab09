// Fused decode path (see decode.hip).
#pragma once

#include "internal.h"

namespace lci {

constexpr int kDecChunk = 4096;      // history positions per scoring workgroup
constexpr int kDecCap = 8192;        // candidates per sequence resolved in LDS
constexpr int kDecMaxChunks = 8192;  // history of at most 2^25 positions

struct DecLayout {
  size_t scores, fhist, chist, ncand, cand, thr, idx, attn, total;
  int nchunks, splits, ss;
  int nsw;  // sample workgroups per sequence
};

DecLayout decode_layout(const Geom& g);
hipError_t launch_decode(const Geom& g, const int8_t* q_idx, const int8_t* k_idx,
                         const int8_t* w, int64_t wsb, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const uint16_t* gate,
                         const uint16_t* mix, float scale, uint16_t* out,
                         float* lse, int32_t* idx_out, void* workspace, hipStream_t stream);

}  // namespace lci
