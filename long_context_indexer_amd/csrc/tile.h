// LDS tiles of keys and values shared by the tile kernels of attention and of
// its gradients: 64-key tiles of one key/value head, XOR-swizzled, filled from
// HBM by direct-to-LDS buffer loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

#define LDS_AS __attribute__((address_space(3)))

namespace lci {

template <int D, int G>
struct DenseCfg {
  static constexpr int TW = 32 / G;   // tokens per wave
  static constexpr int BQ = 4 * TW;   // tokens per workgroup
  static constexpr int BK = 64;       // keys per tile
  static constexpr int KP = D;        // LDS row pitch (bf16); 16-byte units are XOR-swizzled
  static constexpr int NKK = D / 16;  // 16-deep MFMA steps over d for S^T
  static constexpr int NDT = D / 32;  // 32-wide d tiles of O^T
};

// Bank-conflict-free placement of the 16-byte unit u of tile row r: unit
// u ^ swz(r). With this, the 16-row key reads (ds_read_b128, one unit of 16
// consecutive rows), the transposed value reads (4 consecutive rows x 4 units
// per 32-lane phase) and the row stores all touch 16 distinct 16-byte bank
// groups of the 64-bank LDS.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
// element offset of (row, col) in a swizzled tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

constexpr int kNegInfBits = static_cast<int>(0xff800000u);

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 l (dst is wave-uniform); offsets outside the buffer read as zero.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t rs, LDS_AS void* dst,
                                              int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
}

}  // namespace lci
