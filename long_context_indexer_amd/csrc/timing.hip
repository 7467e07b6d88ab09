// Kernel timing log: optional HIP-event brackets around every kernel launch,
// read back per kernel kind (profiling instrumentation, host code only).
#include <mutex>
#include <vector>

#include "../../include/lci.h"
#include "internal.h"

namespace lci {
namespace {

struct Record {
  int kind;
  hipEvent_t start, stop;
};

struct Log {
  std::mutex mu;
  bool on = false;
  std::vector<Record> pending;   // recorded, not yet read back
  std::vector<hipEvent_t> pool;  // idle events for reuse
  double total_ms[LCI_KERNEL_COUNT] = {};
  int64_t launches[LCI_KERNEL_COUNT] = {};
};

Log& log() {
  static Log l;
  return l;
}

// caller holds the mutex
hipEvent_t take_event(Log& l) {
  if (!l.pool.empty()) {
    hipEvent_t e = l.pool.back();
    l.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// caller holds the mutex: fold finished records of one kind (or all kinds, kind < 0)
hipError_t drain(Log& l, int kind) {
  std::vector<Record> keep;
  hipError_t err = hipSuccess;
  for (const Record& r : l.pending) {
    if (kind >= 0 && r.kind != kind) {
      keep.push_back(r);
      continue;
    }
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e == hipSuccess) {
      l.total_ms[r.kind] += ms;
      l.launches[r.kind] += 1;
    } else if (err == hipSuccess) {
      err = e;
    }
    l.pool.push_back(r.start);
    l.pool.push_back(r.stop);
  }
  l.pending.swap(keep);
  return err;
}

void clear(Log& l) {
  drain(l, -1);
  for (int k = 0; k < LCI_KERNEL_COUNT; ++k) {
    l.total_ms[k] = 0.0;
    l.launches[k] = 0;
  }
}

const char* const kNames[LCI_KERNEL_COUNT] = {
    "idx_score", "topk", "idx_mask", "attn_dense", "attn_gather", "attn_combine",
    "dec_sample", "dec_thresh", "dec_score", "dec_select", "kv_append",
    "kv_lengths", "bwd_prologue", "bwd_dq", "bwd_transpose", "bwd_dkdv", "sel_scan",
    "sel_rows", "sel_fallback", "ibwd_rows", "ibwd_transpose", "ibwd_dk"};

}  // namespace

KernelTimer::KernelTimer(int kind, hipStream_t stream) : kind_(kind), stream_(stream) {
  Log& l = log();
  std::lock_guard<std::mutex> g(l.mu);
  if (!l.on) return;
  start_ = take_event(l);
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
    l.pool.push_back(start_);
    start_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  Log& l = log();
  std::lock_guard<std::mutex> g(l.mu);
  hipEvent_t stop = take_event(l);
  if (!l.on || !stop || hipEventRecord(stop, stream_) != hipSuccess) {
    l.pool.push_back(start_);
    if (stop) l.pool.push_back(stop);
    return;
  }
  l.pending.push_back(Record{kind_, start_, stop});
}

}  // namespace lci

extern "C" {

int lci_kernel_timing(int enable) {
  lci::Log& l = lci::log();
  std::lock_guard<std::mutex> g(l.mu);
  lci::clear(l);
  l.on = enable != 0;
  return LCI_OK;
}

int lci_kernel_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return LCI_ERR_NULL;
  if (kernel < 0 || kernel >= LCI_KERNEL_COUNT) return LCI_ERR_SHAPE;
  lci::Log& l = lci::log();
  std::lock_guard<std::mutex> g(l.mu);
  const hipError_t e = lci::drain(l, kernel);
  *total_ms = l.total_ms[kernel];
  *launches = l.launches[kernel];
  return e == hipSuccess ? LCI_OK : LCI_ERR_HIP;
}

const char* lci_kernel_name(int kernel) {
  if (kernel < 0 || kernel >= LCI_KERNEL_COUNT) return nullptr;
  return lci::kNames[kernel];
}

}  // extern "C"
