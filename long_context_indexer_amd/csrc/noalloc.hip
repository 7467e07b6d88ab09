// Allocation-free fused decode: lci_decode_fwd with its workspace carved out
// of a static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in the library's code object, so every GPU the library runs
// on holds one copy of it (kNoAllocScratchBytes) until the process ends. Its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, on the entry's first call there: the array's name in
// host code is only a host-side stand-in and is never passed to a kernel.
#include <mutex>

#include "../../include/lci.h"
#include "internal.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(LCI_NOALLOC_SCRATCH_MIB) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (nullptr and the HIP
// error on failure).
void* device_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t lci_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

lci_status lci_decode_fwd_noalloc(const lci_geom* g, const int8_t* q_idx, const int8_t* k_idx,
                                  const int8_t* w, int64_t w_stride_b, int64_t w_stride_q,
                                  const lci_bf16* q, const lci_bf16* k, const lci_bf16* v,
                                  const lci_bf16* gate, const lci_bf16* mix,
                                  float softmax_scale, lci_bf16* out, float* lse,
                                  int32_t* idx_out, void* stream) {
  // every argument but the workspace is checked first, on the host, by the
  // decode entry itself: without a workspace it returns LCI_ERR_WORKSPACE
  // when all else is valid, and enqueues nothing in either case
  lci_status s = lci_decode_fwd(g, q_idx, k_idx, w, w_stride_b, w_stride_q, q, k, v, gate, mix,
                                softmax_scale, out, lse, idx_out, nullptr, 0, stream);
  if (s != LCI_ERR_WORKSPACE) return s;
  if (lci_workspace_bytes(LCI_ENTRY_DECODE, g) > kNoAllocScratchBytes) return LCI_ERR_SCRATCH;
  hipError_t e = hipSuccess;
  void* ws = device_scratch(&e);
  if (!ws) return static_cast<lci_status>(lci::hip_error_status(e));
  return lci_decode_fwd(g, q_idx, k_idx, w, w_stride_b, w_stride_q, q, k, v, gate, mix,
                        softmax_scale, out, lse, idx_out, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
