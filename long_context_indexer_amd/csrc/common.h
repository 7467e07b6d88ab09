// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lci {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned short v4us __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// log2(e): logits are kept in base-2 units so the softmax uses v_exp_f32 (2^x).
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reciprocal by v_rcp_f32 (about 1 ulp) instead of the correctly rounded
// division sequence.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Sigmoid from 2^x: 1 / (1 + 2^(-x*log2 e)).
__device__ __forceinline__ float sigmoidf(float x) {
  return fast_rcp(1.0f + fast_exp2(-x * LOG2E));
}

// The gate mixing an attention output o with the other branch's output x
// (bf16) by s = sigmoid(G): s*o + (1 - s)*x, computed as x + s*(o - x).
__device__ __forceinline__ float gate_mix(float o, float s, uint16_t x) {
  const float xf = bf16_to_f32(x);
  return fmaf(s, o - xf, xf);
}

// Order-preserving map of int32 scores to uint32 keys (sign bit flipped).
__device__ __forceinline__ uint32_t score_key(int32_t s) {
  return static_cast<uint32_t>(s) ^ 0x80000000u;
}
__device__ __forceinline__ int32_t key_score(uint32_t k) {
  return static_cast<int32_t>(k ^ 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, WAVE);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    uint32_t t = __shfl_up(v, off, WAVE);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

// Exclusive prefix sum over a whole workgroup (blockDim.x threads, a multiple
// of 64, at most 1024). `scratch` holds at least blockDim.x/64 + 1 words of LDS.
// Returns this thread's exclusive prefix; *total receives the block sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t* total) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  const int nw = blockDim.x / WAVE;
  uint32_t incl = wave_incl_scan(v);
  if (lane == WAVE - 1) scratch[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < nw ? scratch[lane] : 0u;
    uint32_t wi = wave_incl_scan(w);
    if (lane < nw) scratch[lane] = wi - w;
    if (lane == nw - 1) scratch[nw] = wi;
  }
  __syncthreads();
  uint32_t res = scratch[wid] + incl - v;
  *total = scratch[nw];
  __syncthreads();
  return res;
}

// dword 3 of a raw buffer resource on gfx9-class parts: 32-bit data format.
// Loads past the resource's size read zero; stores past it are dropped.
constexpr int kBufferFlags = 0x00020000;

// A workgroup-uniform pointer, moved to scalar registers (buffer resources must
// live there; without this the compiler may loop over lanes to build them).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace lci
