// Concurrent tile and gather attention on disjoint compute units (gfx950).
//
// A long prefill splits its rows between the two exact attention paths: the
// tile kernel (short histories, bound by its MFMA and softmax work) and the
// gather kernel (long histories, bound by the rate at which the selected key
// and value rows arrive from the last-level cache). Run one after the other,
// each leaves the resource the other needs idle. Here they run at once on two
// library streams whose compute-unit masks split every XCD: the gather gets
// k of its 32 CUs and the tile kernel t of them (the two sets may share a
// few), the split chosen from a cost model of the two kernels measured on
// Prefill 64K. The caller's stream forks to both
// and joins back through events, so the call stays ordered on that stream.
//
// Measured (Prefill 64K, K = 2048, 8 query heads per key/value head, d = 128;
// kernel-by-kernel event times with the other kernel running):
//   tile kernel on 32 / 20 / 16 / 12 / 8 CUs per XCD: 8.1 / 12.9 / 15.7 / 20.6 / 29.5 ms
//   gather on 32 / 28 / 24 / 20 / 16 / 12 CUs:       16.1 / 17.9 / 17.9 / 19.3 / 21.7 / 28.7 ms
// and with the gather on 20 CUs and the tile kernel on 16 (4 shared): 20.2 /
// 20.0 ms. The tile kernel scales with its CUs, the gather saturates near 24;
// the step took 27.3 ms one after the other, 23.5 ms split 20 / 12 and 23.1
// ms split 20 / 16.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "../../include/lci.h"
#include "internal.h"

namespace lci {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;

// The splits the model may pick: the gather's CUs per XCD (the first k of
// each), the tile kernel's (the last t; with k + t > 32 the middle ones serve
// both), and each kernel's slowdown there with the other one beside it
// (against its time alone on all CUs; the measurements above)
struct Split {
  int k, t;
  double tile_factor, gather_factor;
};
constexpr Split kSplits[] = {{12, 20, 1.58, 1.78}, {16, 16, 1.93, 1.35},
                             {20, 12, 2.53, 1.20}, {20, 16, 2.45, 1.25},
                             {24, 8, 3.62, 1.11}};
constexpr int kNumSplits = sizeof(kSplits) / sizeof(kSplits[0]);
constexpr int kDefaultSplit = 3;  // 20 / 16

struct DeviceStreams {
  bool tried = false;
  bool ok = false;
  hipStream_t tile = nullptr;    // the split's last t CUs of every XCD
  hipStream_t gather = nullptr;  // its first k CUs of every XCD
  hipEvent_t fork = nullptr, tile_done = nullptr, gather_done = nullptr;
};

std::mutex g_mu;  // guards the table and each fork/join sequence
DeviceStreams g_dev[kMaxDevices][kNumSplits];  // per device and split
bool g_exit_hook = false;

// At process exit (before the runtime's own teardown, whose exit hooks were
// registered earlier): wait for the library streams and release them, so no
// masked queue outlives the code that made it.
void release_streams() {
  std::lock_guard<std::mutex> lock(g_mu);
  for (int dev = 0; dev < kMaxDevices; ++dev)
    for (int si = 0; si < kNumSplits; ++si) {
      DeviceStreams& d = g_dev[dev][si];
      if (!d.ok) continue;
      if (hipSetDevice(dev) != hipSuccess) continue;
      hipStreamSynchronize(d.tile);
      hipStreamSynchronize(d.gather);
      hipStreamDestroy(d.tile);
      hipStreamDestroy(d.gather);
      hipEventDestroy(d.fork);
      hipEventDestroy(d.tile_done);
      hipEventDestroy(d.gather_done);
      d.ok = false;
    }
}
std::atomic<int> g_mode{LCI_OVERLAP_AUTO};
std::atomic<long long> g_forks{0};  // calls that ran the two kernels on the library streams

// Cost of each path on the whole GPU, from the Prefill-64K measurements: the
// tile kernel 8.1 ms for 5.4e8 (row, causal key) pairs at 32 query heads of
// 128 (3.7e-15 s per pair, head and feature), the gather 16.1 ms for 137 GB
// of selected key and value rows (8.5 TB/s).
constexpr double kTileSecPerPairHeadDim = 3.7e-15;
constexpr double kGatherBytesPerSec = 8.5e12;

// CU mask bits of this part: bit i selects a CU of XCD i % 8 (measured: a
// stream masked to 8 consecutive bits runs on one CU of every XCD), so a range
// of 8 k bits holds k CUs of every XCD
void cu_masks(const Split& s, uint32_t* tile, uint32_t* gather) {
  constexpr int nbits = kXcds * kCusPerXcd;
  for (int w = 0; w < nbits / 32; ++w) tile[w] = gather[w] = 0u;
  for (int bit = 0; bit < nbits; ++bit) {
    if (bit < kXcds * s.k) gather[bit / 32] |= 1u << (bit % 32);
    if (bit >= nbits - kXcds * s.t) tile[bit / 32] |= 1u << (bit % 32);
  }
}

// The streams and events of this device for split si (created on first use;
// nullptr when they cannot be, and then the call runs on the caller's stream).
DeviceStreams* device_streams(int si, hipStream_t caller) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (si < 0 || si >= kNumSplits) return nullptr;
  // a stream under capture keeps the one-stream order (a graph's kernels do not
  // keep a stream's CU mask)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return nullptr;
  DeviceStreams& d = g_dev[dev][si];
  if (d.ok) return &d;
  if (d.tried) return nullptr;
  d.tried = true;
  if (!g_exit_hook) {
    g_exit_hook = true;
    std::atexit(release_streams);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      prop.multiProcessorCount != kXcds * kCusPerXcd)
    return nullptr;
  uint32_t mt[kXcds * kCusPerXcd / 32], mg[kXcds * kCusPerXcd / 32];
  cu_masks(kSplits[si], mt, mg);
  const uint32_t nw = kXcds * kCusPerXcd / 32;
  if (hipExtStreamCreateWithCUMask(&d.tile, nw, mt) != hipSuccess) return nullptr;
  if (hipExtStreamCreateWithCUMask(&d.gather, nw, mg) != hipSuccess) return nullptr;
  if (!d.fork && hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) != hipSuccess)
    return nullptr;
  if (!d.tile_done && hipEventCreateWithFlags(&d.tile_done, hipEventDisableTiming) != hipSuccess)
    return nullptr;
  if (!d.gather_done &&
      hipEventCreateWithFlags(&d.gather_done, hipEventDisableTiming) != hipSuccess)
    return nullptr;
  d.ok = true;
  return &d;
}

}  // namespace

int pick_overlap_split(const Geom& g, int lim, bool gather_work) {
  const int mode = g_mode;
  if (mode == LCI_OVERLAP_OFF || !gather_work) return -1;
  if (mode == LCI_OVERLAP_ON) return kDefaultSplit;
  // rows at positions 0 .. Tq-1 (a whole prompt: Tq = Tk); other shapes keep
  // the one-stream order, their positions being known only on the device
  if (g.Tq != g.Tk) return -1;
  const double L = static_cast<double>(std::min(lim, g.Tq));
  const double tile_rows_pairs = L * (L + 1.0) / 2.0;
  const double gather_rows = static_cast<double>(g.Tq) - L;
  const double t_tile =
      g.B * tile_rows_pairs * g.Hq * g.d * kTileSecPerPairHeadDim;
  const double t_gather =
      g.B * gather_rows * g.K * g.Hkv * g.d * 4.0 / kGatherBytesPerSec;
  double best = 0.0;
  int pick = -1;
  for (int i = 0; i < kNumSplits; ++i) {
    const Split& s = kSplits[i];
    const double t = std::max(t_tile * s.tile_factor, t_gather * s.gather_factor);
    if (pick < 0 || t < best) {
      best = t;
      pick = i;
    }
  }
  // a split must beat the two kernels one after the other by a margin
  return best < 0.95 * (t_tile + t_gather) ? pick : -1;
}

hipError_t overlap_fork(int split, hipStream_t caller, OverlapStreams* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceStreams* d = device_streams(split, caller);
  if (!d) return hipErrorNotSupported;
  hipError_t e;
  if ((e = hipEventRecord(d->fork, caller)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(d->tile, d->fork, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(d->gather, d->fork, 0)) != hipSuccess) return e;
  out->tile = d->tile;
  out->gather = d->gather;
  out->tile_done = d->tile_done;
  out->gather_done = d->gather_done;
  ++g_forks;
  return hipSuccess;
}

hipError_t overlap_join(const OverlapStreams& s, hipStream_t caller) {
  std::lock_guard<std::mutex> lock(g_mu);
  hipError_t e;
  if ((e = hipEventRecord(s.tile_done, s.tile)) != hipSuccess) return e;
  if ((e = hipEventRecord(s.gather_done, s.gather)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(caller, s.tile_done, 0)) != hipSuccess) return e;
  return hipStreamWaitEvent(caller, s.gather_done, 0);
}

}  // namespace lci

extern "C" long long lci_attn_overlap_forks(void) { return lci::g_forks; }

extern "C" int lci_attn_overlap(int mode) {
  if (mode != LCI_OVERLAP_AUTO && mode != LCI_OVERLAP_OFF && mode != LCI_OVERLAP_ON)
    return LCI_ERR_SHAPE;
  lci::g_mode = mode;
  return LCI_OK;
}
