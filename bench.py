"""Benchmark of the gated fine-grained sparse attention layer on one MI355X.

One step = one fused pass of the whole layer (indexer scoring -> Top-K ->
sparse attention -> sigmoid gate) over one batch of synthetic, seeded inputs
already resident in HBM. The headline workload is the largest single-GPU
prefill, Prefill 64K: batch 1, 65536 causal tokens, 32 query heads over 4 KV
heads, head dim 128, 8 int8 indexer heads of dim 64, K = 2048. The same JSON
line carries the other three timed workloads (Decode 1M: 8 single-token
queries over 1048576-token histories; Prefill 8K; Decode 128K: 64 queries over
131072-token histories), each with its per-kernel breakdown and the roofline of
its own dominant kernel (HIP events on the stream the kernels are launched on),
variants of the Prefill-8K step (block selection, index sets per KV head, the
gradients) and the CPU oracle timed on bounded samples of the headline
prefill and of Decode 1M.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--only WORKLOAD]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tok/s + decode queries/s at K=2048; % of HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic per launch from rocprofv3 counter passes (one pass for FETCH_SIZE,
# one for WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
# reads for a plain 2 GiB device copy kernel (FETCH_SIZE reads 1 GiB for its
# 2 GiB of reads: x2.0; WRITE_SIZE reads 2 GiB for its 2 GiB of writes: x1.0).
# Keyed by (workload, kernel). Valid only for the kernel sources the counters
# were taken on: any change to them turns the figure into null.
TRAFFIC = {
    ("prefill64k", "attn_gather"): dict(
        fetch_kib=60698896.4, write_kib=262190.7, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/sparse_attn.hip", "long_context_indexer_amd/csrc/common.h"],
        sha256="9d1e44aa4e1c05578d0ce0df95e035332296c77f2401efe0829f0c6c5eb64a92"),
    ("prefill64k", "attn_dense"): dict(
        fetch_kib=2436313.1, write_kib=262178.7, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/attn_dense.hip", "long_context_indexer_amd/csrc/attn_dense.h", "long_context_indexer_amd/csrc/tile.h", "long_context_indexer_amd/csrc/common.h"],
        sha256="7b605c37ae27f08f2199cd7a9bfb116bbcc24e858955a4ee0f314501a9973b8c"),
    ("prefill64k", "sel_scan"): dict(
        fetch_kib=226100.5, write_kib=4113768.9, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/idx_select.hip", "long_context_indexer_amd/csrc/common.h", "long_context_indexer_amd/csrc/select_row.h"],
        sha256="3f4c7c7272a3e7855316ae942f4ac0fc96a99088780e996f37d7eb792e11a64a"),
    ("prefill8k", "attn_dense"): dict(
        fetch_kib=121627.7, write_kib=65956.5, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/attn_dense.hip", "long_context_indexer_amd/csrc/attn_dense.h", "long_context_indexer_amd/csrc/tile.h", "long_context_indexer_amd/csrc/common.h"],
        sha256="7b605c37ae27f08f2199cd7a9bfb116bbcc24e858955a4ee0f314501a9973b8c"),
    ("decode1m", "dec_score"): dict(
        fetch_kib=262428.3, write_kib=322.6, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/decode.hip", "long_context_indexer_amd/csrc/decode.h", "long_context_indexer_amd/csrc/common.h", "long_context_indexer_amd/csrc/select_row.h"],
        sha256="2dfeebdc7868aba4644b25b1ba2c4621237a458b430ca9121201a5716cf8daa9"),
    ("decode128k", "dec_score"): dict(
        fetch_kib=262549.1, write_kib=1775.4, fetch_scale=2.0, write_scale=1.0,
        sources=["long_context_indexer_amd/csrc/decode.hip", "long_context_indexer_amd/csrc/decode.h", "long_context_indexer_amd/csrc/common.h", "long_context_indexer_amd/csrc/select_row.h"],
        sha256="2dfeebdc7868aba4644b25b1ba2c4621237a458b430ca9121201a5716cf8daa9"),
}


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(workload, kernel):
    """HBM bytes per launch from the recorded counters, or None when the kernel's
    sources changed since they were taken (or none were taken)."""
    t = TRAFFIC.get((workload, kernel))
    if t is None or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- algorithmic work

def row_positions(cfg):
    """Absolute positions p of every query row (all sequences)."""
    if cfg.decode:
        return np.full(cfg.B, cfg.Tk - 1, np.int64)
    return np.tile(np.arange(cfg.Tq, dtype=np.int64), cfg.B)


def pairs_of(cfg, p):
    """Selected (query, key) pairs of rows at positions p: min(K, p+1) each."""
    return int(np.minimum(cfg.K, p + 1).sum())


def attn_flops(cfg, p):
    """4*Hq*d flops per selected (query, key) pair: q.k and p.v for every query head."""
    return 4.0 * cfg.Hq * cfg.d * pairs_of(cfg, p)


def idx_ops(cfg):
    """2*H_I*d_I int8 ops per scored (query, causal position) pair."""
    return 2.0 * cfg.H_I * cfg.d_I * float((row_positions(cfg) + 1).sum())


def decode_attn_bytes(cfg):
    """Algorithmic HBM bytes of sparse attention per decode step: the K selected
    key and value rows of every KV head, q, gate, out and the index row."""
    return cfg.B * (cfg.K * cfg.Hkv * cfg.d * 2 * 2 + 3 * cfg.Hq * cfg.d * 2 + cfg.K * 4)


def decode_step_bytes(cfg):
    """Algorithmic HBM bytes of the whole decode step: the indexer key cache of
    every history, q_idx, and the sparse-attention bytes."""
    return cfg.B * (cfg.Tk * cfg.d_I + cfg.H_I * cfg.d_I) + decode_attn_bytes(cfg)


def append_bytes(rows, Hkv, d, d_I):
    """Algorithmic HBM bytes of appending rows to the caches: every new key,
    value and indexer-key row read once and written once."""
    return 2 * rows * (2 * Hkv * d * 2 + d_I)


def kernel_work(cfg, kname, lim):
    """(bound, algorithmic work per step, unit, peak) of one kernel of a
    workload's step, or None when the kernel has no roofline of its own
    (launch-bound helpers). lim: rows with p+1 <= lim take the dense-tile path."""
    p = row_positions(cfg)
    if kname == "attn_dense":
        return "mfma", attn_flops(cfg, p[p + 1 <= lim]) / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS
    if kname == "attn_gather":
        # the selected K and V rows (Hkv*d*2 B each) of every gathered row; at
        # prefill the sequence's K and V fit the last-level cache, so this rate
        # can pass the HBM peak it is measured against
        if cfg.decode:
            return "hbm", cfg.B * cfg.K * cfg.Hkv * cfg.d * 4 / 1e9, "GB/s", PEAK_HBM_GBS
        sel = pairs_of(cfg, p[p + 1 > lim])
        return "hbm", sel * cfg.Hkv * cfg.d * 4 / 1e9, "GB/s", PEAK_HBM_GBS
    if kname in ("idx_score", "sel_scan"):
        # every causal score (the long-prefill scan computes each once in its
        # full pass, plus a 5/32 sample)
        return "mfma", idx_ops(cfg) / 1e12, "TOP/s", PEAK_INT8_TOPS
    if kname == "dec_score":
        return "hbm", cfg.B * cfg.Tk * cfg.d_I / 1e9, "GB/s", PEAK_HBM_GBS
    return None


def roofline(cfg, kern, lim, workload, prefer=None):
    """Roofline of the kernel that takes the most time per step (or `prefer`,
    when given and timed). achieved = the algorithmic work that kernel does per
    step / its summed launch durations per step (event-timed average launch
    time x launches per step)."""
    ranked = sorted(kern, key=lambda k: -kern[k]["ms_per_step"])
    dom = next((k for k in ranked if kernel_work(cfg, k, lim) is not None), ranked[0])
    if prefer in kern and kernel_work(cfg, prefer, lim) is not None:
        dom = prefer
    kw = kernel_work(cfg, dom, lim)
    ms = kern[dom]["ms_per_step"]
    if kw is None:
        return dict(kernel=dom, bound=None, achieved=None, peak=None, unit=None, frac=None,
                    traffic=None)
    bound, work, unit, peak = kw
    ach = work / (ms * 1e-3)
    return dict(kernel=dom, bound=bound, achieved=ach, peak=peak, unit=unit, frac=ach / peak,
                traffic=traffic_bytes(workload, dom),
                traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                             "copy-calibrated)",
                launches_per_step=kern[dom]["launches_per_step"],
                avg_launch_ms=kern[dom]["avg_launch_ms"])


def kernel_rooflines(cfg, kern, lim):
    """The roofline fraction of every kernel of the step that has one."""
    out = {}
    for k, v in kern.items():
        kw = kernel_work(cfg, k, lim)
        if kw is None:
            continue
        bound, work, unit, peak = kw
        ach = work / (v["ms_per_step"] * 1e-3)
        out[k] = dict(bound=bound, achieved=round(ach, 2), unit=unit, frac=round(ach / peak, 4))
    return out


# ----------------------------------------------------------------------- timing

class Timer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.t = torch

    def time(self, fn, iters):
        s = self.t.cuda.Event(enable_timing=True)
        e = self.t.cuda.Event(enable_timing=True)
        s.record(self.stream)
        for _ in range(iters):
            fn()
        e.record(self.stream)
        e.synchronize()
        return s.elapsed_time(e) / iters

    def per_step(self, fn, iters):
        """Each step bracketed by its own events (recorded back to back, read at
        the end): median, min and p90 in ms."""
        ev = [self.t.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(self.stream)
        for i in range(iters):
            fn()
            ev[i + 1].record(self.stream)
        ev[-1].synchronize()
        ts = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
        return dict(median_ms=float(np.median(ts)), min_ms=float(ts.min()),
                    p90_ms=float(np.percentile(ts, 90)))


def timed_region(timer, step, steps, lci):
    """Time `steps` steps (wall clock with a device synchronisation on both sides,
    and stream events around the whole region), then `steps` steps each between
    its own events (median/min/p90), then `steps` more with the library's
    per-kernel event log on (events around every launch, on the launch stream).
    The log's events add a few microseconds per launch, so the headline step
    time comes from the first region and only the per-kernel durations from the
    last."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_ms = timer.time(step, steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    dist = timer.per_step(step, steps)
    lci.kernel_timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name in lci.KERNELS:
        tot, n = lci.kernel_timing_read(name)
        if n:
            kern[name] = dict(launches_per_step=n / steps, ms_per_step=tot / steps,
                              avg_launch_ms=tot / n)
    lci.kernel_timing(False)
    return wall_ms, ev_ms, dist, kern


def cold_steps(step, steps, stream):
    """Each step timed alone (events on the launch stream) after the last-level
    cache has been flushed by streaming a 1 GiB buffer outside the timed span:
    inputs are in HBM but no longer in any cache. Median ms."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for _ in range(steps):
        flush.add_(1.0)  # reads and writes 1 GiB on the same stream
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        e.synchronize()
        times.append(s.elapsed_time(e))
    del flush
    times.sort()
    return times[len(times) // 2]


def time_append(lci, k_new, v_new, kI_new, k, v, kI, kv_len, reps, stream):
    """Average event-timed duration (ms) of the cache-append copy kernel and of
    its length kernel over `reps` calls, with the kernel timing log on."""
    import torch
    qo = torch.empty_like(kv_len)
    kl = torch.empty_like(kv_len)

    def call():
        lci.kv_append(k_new, v_new, kI_new, k, v, kI, kv_len, q_offset_out=qo, kv_len_out=kl,
                      stream=stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    lci.kernel_timing(True)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    cp, n_cp = lci.kernel_timing_read("kv_append")
    ln, n_ln = lci.kernel_timing_read("kv_lengths")
    lci.kernel_timing(False)
    return cp / n_cp, ln / n_ln


def copy_calibration():
    """A plain device-to-device copy of 2 GiB, five times: under rocprofv3 --pmc
    FETCH_SIZE / WRITE_SIZE it gives the factor between each counter and the bytes
    a kernel really reads and writes."""
    import torch
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)


def probe_peaks():
    """Peaks reachable on this GPU, reported beside the vendor ones: a 2 GiB
    device-to-device copy (HBM read + write bytes over time), a sum over 8 GiB
    (read bytes over time; the HBM reference is the faster of the two), and bf16 and int8
    GEMMs of 8192 x 8192 x 8192 through the installed BLAS library (the matrix
    cores' rate a tuned library reaches). Torch's own kernels on its current
    stream, timed with torch events; None where a probe is not available."""
    import torch

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out["hbm_copy_gbs"] = round(2 * n / timed(lambda: dst.copy_(src), 10) / 1e9, 1)
    del src, dst
    x = torch.ones(n, dtype=torch.float32, device="cuda")  # 8 GiB, read once per sum
    out["hbm_read_gbs"] = round(4 * n / timed(lambda: x.sum(), 5) / 1e9, 1)
    del x
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    out["bf16_gemm_tflops"] = round(2 * m ** 3 / timed(lambda: torch.matmul(a, b), 10) / 1e12, 1)
    del a, b
    try:
        a8 = torch.randint(-8, 8, (m, m), dtype=torch.int8, device="cuda")
        b8 = torch.randint(-8, 8, (m, m), dtype=torch.int8, device="cuda")
        out["int8_gemm_tops"] = round(2 * m ** 3 / timed(lambda: torch._int_mm(a8, b8), 10) / 1e12, 1)
        del a8, b8
    except (RuntimeError, AttributeError):
        out["int8_gemm_tops"] = None
    out.update(gather_probes(timed))
    torch.cuda.empty_cache()
    out["note"] = ("reachable rates measured here (copy kernel, library GEMMs, random-row "
                   "gathers); rooflines give frac against the vendor peak and frac_probe "
                   "against these (the gather kernel against the faster gather probe)")
    return out


def gather_probes(timed):
    """Random-row gather rate from a 128 MiB table (the key/value cache of the
    Prefill-64K workload: 65536 positions x 4 heads x 128 x bf16, keys and
    values), rows of 256 B (one head's key row) and 1 KiB (a position's four
    heads), by the measurement kernel in bench_probe.hip: 4 GiB gathered per
    launch from seeded uniform row numbers. None where the probe is not built."""
    import ctypes
    import torch

    path = os.path.join(ROOT, "bench_probe.so")
    if not os.path.exists(path):
        return {"gather_128mib_256b_gbs": None, "gather_128mib_1kib_gbs": None}
    fn = ctypes.CDLL(path).bench_gather_probe
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    table_bytes = 128 << 20
    table = torch.ones(table_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    res = {}
    for rb, key in ((256, "gather_128mib_256b_gbs"), (1024, "gather_128mib_1kib_gbs")):
        n = (4 << 30) // rb
        idx = torch.randint(0, table_bytes // rb, (n,), generator=gen, dtype=torch.int32,
                            device="cuda")
        stream = torch.cuda.current_stream().cuda_stream

        def go():
            rc = fn(table.data_ptr(), rb, idx.data_ptr(), n, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"bench_gather_probe failed with HIP error {rc}")

        res[key] = round(n * rb / timed(go, 5) / 1e9, 1)
        del idx
    return res


def add_probe_fracs(node, probes, kname=None):
    """frac_probe beside frac in every roofline dict under node (in place);
    kname: the kernel a roofline dict is keyed by when it names none itself."""
    hbm = max(probes.get("hbm_copy_gbs") or 0.0, probes.get("hbm_read_gbs") or 0.0) or None
    gather = max(probes.get("gather_128mib_256b_gbs") or 0.0,
                 probes.get("gather_128mib_1kib_gbs") or 0.0) or None
    ref = {"GB/s": hbm, "TFLOP/s": probes.get("bf16_gemm_tflops"),
           "TOP/s": probes.get("int8_gemm_tops")}
    if isinstance(node, dict):
        if "frac" in node and "achieved" in node and node.get("unit") in ref:
            pk = ref[node["unit"]]
            if node.get("kernel", kname) == "attn_gather" and gather:
                pk = gather
            node["frac_probe"] = round(node["achieved"] / pk, 4) if pk and node["achieved"] else None
        for k, v in node.items():
            add_probe_fracs(v, probes, k)


def host(t):
    """Host numpy copy of a device tensor (bf16 as its uint16 bit pattern)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def kernel_log_lines(kern):
    for kname, kv in kern.items():
        log(f"  {kname:12s} {kv['launches_per_step']:.0f} launch(es)/step, "
            f"{kv['ms_per_step'] * 1e3:8.1f} us/step")


def us_per_step(kern):
    return {k: round(v["ms_per_step"] * 1e3, 2) for k, v in kern.items()}


# ----------------------------------------------------------------------- oracle

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline_prefill(cfg, inp_host, budget_s):
    """The oracle as it stands, on uniformly drawn query rows of the workload
    (an unbiased sample of per-row work), whole layer per row, as tokens/s."""
    import oracle
    r = np.random.default_rng(123)
    t0 = time.perf_counter()
    n_done = 0
    batch = max(1, oracle.num_threads())
    while time.perf_counter() - t0 < budget_s:
        rows = [(0, int(i)) for i in r.integers(0, cfg.Tq, size=batch)]
        oracle.layer(inp_host, cfg.K, rows=rows)
        n_done += len(rows)
    el = time.perf_counter() - t0
    return dict(value=n_done / el, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"{n_done} query rows drawn uniformly from the {cfg.Tq} rows of the "
                       f"{cfg.name} workload, whole layer per row (scores of every causal "
                       f"position, Top-K, gated attention), {el:.1f} s")


def cpu_baseline_decode(cfg, d):
    """The oracle's decode step for every sequence of a decode workload: scores
    over the whole history, Top-K, and gated attention over the rows it selected
    (copied out of device memory by position), as queries/s."""
    import torch
    import oracle
    qI, kI, w = host(d["q_idx"]), host(d["k_idx"]), host(d["w"])
    qo, kvl, q, gate = host(d["q_offset"]), host(d["kv_len"]), host(d["q"]), host(d["gate"])
    t0 = time.perf_counter()
    S = oracle.scores(qI, kI, w, qo, kvl)
    idx, _ = oracle.topk(S, qo.astype(np.int64) + 1, cfg.K)
    t_sel = time.perf_counter() - t0
    sel = torch.from_numpy(idx.astype(np.int64)).to(d["k"].device)
    ks = host(torch.stack([d["k"][b].index_select(0, sel[b]) for b in range(cfg.B)]))
    vs = host(torch.stack([d["v"][b].index_select(0, sel[b]) for b in range(cfg.B)]))
    t1 = time.perf_counter()
    oracle.attention(q, ks, vs, gate, np.broadcast_to(np.arange(cfg.K, dtype=np.int32),
                                                      (cfg.B, cfg.K)),
                     np.full(cfg.B, cfg.K, np.int32), d["scale"])
    el = t_sel + time.perf_counter() - t1
    return dict(value=cfg.B / el, unit="queries/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"all {cfg.B} queries of {cfg.name} ({cfg.Tk}-position histories), "
                       f"{el:.1f} s (copying the selected rows out of device memory not "
                       f"counted)")


# ----------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill64k", "decode1m", "prefill8k", "decode128k",
                                       "blocks", "sets", "backward", "indexer_bwd"],
                    default=None, help="run one leg only (profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 2 GiB device buffer 5 times (HBM counter calibration runs)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU (asked for {args.gpus}); the "
              "multi-GPU split of the path is a design note, not a runnable mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_indexer_amd as lci
    import synth

    lci.load_library()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    timer = Timer(stream)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def free():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def run_prefill(name, d, cold=True):
        cfg = synth.CONFIGS[name]
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_PREFILL, geom), dtype=torch.uint8,
                         device="cuda")
        lim = lci.dense_row_limit(geom)
        out = torch.empty_like(d["q"])

        def step():
            lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                            cfg.scale, d["q_offset"], d["kv_len"], cfg.K, out=out, workspace=ws,
                            stream=stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        forks0 = lci.attn_overlap_forks()
        ms_step, ev_ms, dist, kern = timed_region(timer, step, args.steps, lci)
        forked = lci.attn_overlap_forks() > forks0
        tok_s = cfg.B * cfg.Tq / (ms_step * 1e-3)
        # with the two attention kernels at once (about equally long by the
        # split's choice), the headline is the gather: it moves the step's bytes
        res = dict(workload=name, ms_per_step=ms_step, event_ms_per_step=ev_ms, step_ms=dist,
                   tok_s=tok_s, dense_row_limit=lim,
                   roofline=roofline(cfg, kern, lim, name,
                                     prefer="attn_gather" if forked else None),
                   kernel_rooflines=kernel_rooflines(cfg, kern, lim),
                   kernels_us_per_step=us_per_step(kern))
        if forked:
            res["roofline"]["schedule"] = ("at once with attn_dense, each on its own share of "
                                           "every XCD's compute units (lci_attn_overlap)")
            both = [kern[k]["ms_per_step"] for k in ("attn_dense", "attn_gather") if k in kern]
            res["attention_overlap"] = dict(
                concurrent=True, attention_ms=max(both) if both else None,
                note="attn_dense and attn_gather ran at once on library streams with split "
                     "compute-unit masks (lci_attn_overlap): their launch durations overlap, "
                     "so each kernel's roofline is its rate on its share of the chip while "
                     "the other runs; attention_ms, the longer of the two, is about the "
                     "attention phase's wall time (both start at the fork)")
        log(f"{name} fused: {ms_step:.3f} ms/step ({ev_ms:.3f} ms by events; median "
            f"{dist['median_ms']:.3f}, min {dist['min_ms']:.3f}, p90 {dist['p90_ms']:.3f}), "
            f"{tok_s / 1e6:.2f} M tok/s")
        kernel_log_lines(kern)
        if cold:
            cold_ms = cold_steps(step, args.steps, stream)
            res["cold_cache"] = dict(ms_per_step=cold_ms, tok_s=cfg.B * cfg.Tq / (cold_ms * 1e-3),
                                     note="median of single steps, each after a 1 GiB cache "
                                          "flush")
            log(f"  cold cache {cold_ms:.3f} ms/step")
        del ws, out
        return res

    def run_decode(name):
        cfg = synth.CONFIGS[name]
        d = synth.device_inputs(cfg, seed=0)
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_DECODE, geom), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty_like(d["q"])
        idx = torch.empty((cfg.B, 1, cfg.K), dtype=torch.int32, device="cuda")

        def step(st=stream):
            lci.decode_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                           cfg.scale, d["q_offset"], d["kv_len"], cfg.K, out=out, idx_out=idx,
                           workspace=ws, stream=st)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ms_step, ev_ms, dist, kern = timed_region(timer, step, args.steps, lci)
        # the same step captured once in a HIP graph and replayed: what a serving
        # loop that replays its decode step runs (no per-launch host work)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step(side)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        gdist = Timer(torch.cuda.current_stream()).per_step(graph.replay, args.steps)
        qps, gqps = cfg.B / (ms_step * 1e-3), cfg.B / (g_ms * 1e-3)
        abytes, sbytes = decode_attn_bytes(cfg), decode_step_bytes(cfg)
        a_ms = sum(kern[k]["ms_per_step"] for k in ("attn_gather", "attn_combine") if k in kern)
        log(f"{name} fused: {ms_step:.3f} ms/step eager ({qps:.0f} queries/s), {g_ms:.3f} "
            f"ms/step graph replay ({gqps:.0f} queries/s; median {gdist['median_ms']:.3f}, "
            f"min {gdist['min_ms']:.3f}, p90 {gdist['p90_ms']:.3f}); whole step "
            f"{sbytes / g_ms / 1e6:.0f} GB/s; attention kernels {a_ms * 1e3:.1f} us = "
            f"{abytes / a_ms / 1e6:.0f} GB/s")
        kernel_log_lines(kern)
        res = dict(workload=name, queries_s=max(qps, gqps),
                   eager=dict(ms_per_step=ms_step, event_ms_per_step=ev_ms, step_ms=dist,
                              queries_s=qps),
                   graph_replay=dict(ms_per_step=g_ms, step_ms=gdist, queries_s=gqps),
                   ms_per_step=min(ms_step, g_ms),
                   step_hbm_gbs=sbytes / min(ms_step, g_ms) / 1e6,
                   step_frac_hbm=sbytes / min(ms_step, g_ms) / 1e6 / PEAK_HBM_GBS,
                   step_algorithmic_bytes=sbytes,
                   sparse_attn_us=a_ms * 1e3, sparse_attn_gbs=abytes / a_ms / 1e6,
                   sparse_attn_frac_hbm=abytes / a_ms / 1e6 / PEAK_HBM_GBS,
                   roofline=roofline(cfg, kern, 0, name),
                   kernel_rooflines=kernel_rooflines(cfg, kern, 0),
                   kernels_us_per_step=us_per_step(kern))
        del graph
        # appending one token per sequence: the new rows are each history's last
        # row, written back where it is (kv_len = Tk - 1), so the inputs stay as they are
        last = slice(cfg.Tk - 1, cfg.Tk)
        app_ms, len_ms = time_append(lci, d["k"][:, last].contiguous(),
                                     d["v"][:, last].contiguous(),
                                     d["k_idx"][:, last].contiguous(), d["k"], d["v"],
                                     d["k_idx"], torch.full_like(d["kv_len"], cfg.Tk - 1),
                                     20, stream)
        res["kv_append"] = dict(rows=cfg.B, us=app_ms * 1e3, lengths_us=len_ms * 1e3,
                                bytes=append_bytes(cfg.B, cfg.Hkv, cfg.d, cfg.d_I))
        return res, d

    def run_variant(cfg, d, block, kb, sets):
        """Prefill 8K with block-granular selection and/or index sets per KV head."""
        free()
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, kb, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I, block=block,
                             sets=sets)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_PREFILL, geom), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty_like(d["q"])

        def step():
            lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                            cfg.scale, d["q_offset"], d["kv_len"], kb, out=out, workspace=ws,
                            stream=stream, block=block, sets=sets)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ms_step, ev_ms, dist, kern = timed_region(timer, step, args.steps, lci)
        tok_s = cfg.B * cfg.Tq / (ms_step * 1e-3)
        log(f"prefill8k, blocks of {block} ({kb} kept), {sets} index set(s): {ms_step:.3f} "
            f"ms/step, {tok_s / 1e6:.2f} M tok/s")
        kernel_log_lines(kern)
        return dict(workload="prefill8k", block=block, kept=kb, index_sets=sets,
                    ms_per_step=ms_step, event_ms_per_step=ev_ms, step_ms=dist, tok_s=tok_s,
                    kernels_us_per_step=us_per_step(kern))

    def run_backward(cfg, d):
        """Gradients of attention + gate for the Prefill-8K index rows (from the
        fused forward) and a random bf16 output gradient."""
        free()
        _, idx = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                 d["gate"], cfg.scale, d["q_offset"], d["kv_len"], cfg.K,
                                 want_idx=True, stream=stream)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(7)
        dy = torch.randn(d["q"].shape, generator=gen, device="cuda").to(torch.bfloat16)
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_SPARSE_ATTN_BWD, geom), dtype=torch.uint8,
                         device="cuda")

        def step():
            lci.sparse_attn_bwd(d["q"], d["k"], d["v"], idx, d["gate"], cfg.scale, d["kv_len"],
                                dy, workspace=ws, stream=stream)

        steps = max(2, args.steps // 4)
        step()
        torch.cuda.synchronize()
        ms_step, ev_ms, dist, kern = timed_region(timer, step, steps, lci)
        pairs = pairs_of(cfg, row_positions(cfg))
        tflops = 10.0 * cfg.d * cfg.Hq * pairs / (ms_step * 1e-3) / 1e12
        log(f"prefill8k backward: {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s of backward work")
        kernel_log_lines(kern)
        return dict(workload="prefill8k", ms_per_step=ms_step, event_ms_per_step=ev_ms,
                    step_ms=dist, tok_s=cfg.B * cfg.Tq / (ms_step * 1e-3), steps=steps,
                    tflops=tflops, note="dq, dk, dv, dgate for the layer's index rows; "
                    "10*d flops per (query head, selected key); forward recomputed inside",
                    kernels_us_per_step=us_per_step(kern))

    def run_indexer_bwd(cfg, d):
        """Gradients of the scorer's distillation loss for the Prefill-8K index rows
        (from the fused forward) and seeded teacher weights (normalised per row)."""
        free()
        _, idx = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                 d["gate"], cfg.scale, d["q_offset"], d["kv_len"], cfg.K,
                                 want_idx=True, stream=stream)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(11)
        T = torch.rand(idx.shape, generator=gen, device="cuda") ** 3
        T /= T.sum(-1, keepdim=True)
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"],
                             H_I=cfg.H_I, d_I=cfg.d_I)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_INDEXER_BWD, geom), dtype=torch.uint8,
                         device="cuda")

        def step():
            lci.indexer_bwd(d["q_idx"], d["k_idx"], d["w"], idx, T, 0.002, d["q_offset"],
                            d["kv_len"], workspace=ws, stream=stream)

        steps = max(2, args.steps // 4)
        step()
        torch.cuda.synchronize()
        ms_step, ev_ms, dist, kern = timed_region(timer, step, steps, lci)
        pairs = pairs_of(cfg, row_positions(cfg))
        log(f"prefill8k indexer gradients: {ms_step:.3f} ms/step ({pairs} entries)")
        kernel_log_lines(kern)
        return dict(workload="prefill8k", ms_per_step=ms_step, event_ms_per_step=ev_ms,
                    step_ms=dist, steps=steps, entries=pairs,
                    note="loss, dq_idx, dk_idx, dw of the scorer's distillation loss over the "
                         "layer's index rows; teacher weights seeded, tau = 0.002",
                    kernels_us_per_step=us_per_step(kern))

    res = {}
    want = (lambda leg: args.only in (None, leg))
    cpu, cpu_dec = None, None

    # -------------------------------------------- Prefill 64K (the headline workload)
    if want("prefill64k"):
        cfg64 = synth.CONFIGS["prefill64k"]
        d64 = synth.device_inputs(cfg64, seed=0)
        res["prefill64k"] = run_prefill("prefill64k", d64)
        if args.only is None and not args.no_cpu:
            inp64 = {k: (host(v) if hasattr(v, "device") else v) for k, v in d64.items()}
            del d64
            free()
            cpu = cpu_baseline_prefill(cfg64, inp64, args.cpu_seconds)
            log(f"cpu oracle, prefill64k: {cpu['value']:.1f} tok/s on {cpu['cores']} threads "
                f"({cpu['cpu_model']})")
            del inp64
        else:
            del d64
        free()

    # --------------------------------------------------------------- Decode 1M
    if want("decode1m"):
        res["decode1m"], d1m = run_decode("decode1m")
        if args.only is None and not args.no_cpu:
            cpu_dec = cpu_baseline_decode(synth.CONFIGS["decode1m"], d1m)
            log(f"cpu oracle, decode1m: {cpu_dec['value']:.2f} queries/s")
        del d1m
        free()

    # ------------------------------------------------ Prefill 8K and its variants
    cfg8 = synth.CONFIGS["prefill8k"]
    if any(want(x) for x in ("prefill8k", "blocks", "sets", "backward", "indexer_bwd")):
        d8 = {k: dev(v) for k, v in synth.host_inputs(cfg8, seed=0).items()
              if isinstance(v, np.ndarray)}
        d8["scale"] = cfg8.scale
        if want("prefill8k"):
            res["prefill8k"] = run_prefill("prefill8k", d8)
            app_ms, len_ms = time_append(lci, d8["k"].clone(), d8["v"].clone(),
                                         d8["k_idx"].clone(), d8["k"], d8["v"], d8["k_idx"],
                                         torch.zeros_like(d8["kv_len"]), 20, stream)
            app_b = append_bytes(cfg8.B * cfg8.Tk, cfg8.Hkv, cfg8.d, cfg8.d_I)
            res["prefill8k"]["kv_append"] = dict(
                rows=cfg8.B * cfg8.Tk, us=app_ms * 1e3, lengths_us=len_ms * 1e3, bytes=app_b,
                gbs=app_b / app_ms / 1e6, frac_hbm=app_b / app_ms / 1e6 / PEAK_HBM_GBS,
                note="the whole prompt appended as one chunk to the key/value/indexer-key "
                     "caches (copy kernel; lengths kernel apart)")
        # blocks of 64 positions, 32 kept: the same 2048 positions per row as the
        # position Top-K, chosen as whole blocks
        if want("blocks"):
            res["blocks"] = run_variant(cfg8, d8, 64, 32, 1)
        # one index set per key/value head (4 sets of 2 indexer heads), K = 2048
        if want("sets"):
            res["sets"] = run_variant(cfg8, d8, 1, cfg8.K, cfg8.Hkv)
        if want("backward"):
            res["backward"] = run_backward(cfg8, d8)
        if want("indexer_bwd"):
            res["indexer_bwd"] = run_indexer_bwd(cfg8, d8)
        del d8
        free()

    # -------------------------------------------------------------- Decode 128K
    if want("decode128k"):
        res["decode128k"], d128 = run_decode("decode128k")
        del d128
        free()

    if args.only is not None:
        print(json.dumps(res))
        return

    # ------------------------------------------------------------------ report
    head = res["prefill64k"]
    cfg64 = synth.CONFIGS["prefill64k"]
    if cpu is not None:
        cpu = dict(cpu, decode=cpu_dec)
    line = {
        "metric": METRIC,
        "value": head["tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "indexer_dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "prefill64k", "batch": cfg64.B, "seq_len": cfg64.Tq,
                   "Hq": cfg64.Hq, "Hkv": cfg64.Hkv, "head_dim": cfg64.d, "H_I": cfg64.H_I,
                   "d_I": cfg64.d_I, "top_k": cfg64.K, "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "step_ms": head["step_ms"],
        "kernels_us_per_step": head["kernels_us_per_step"],
        "kernel_rooflines": head["kernel_rooflines"],
        "attention_overlap": head.get("attention_overlap"),
        "cold_cache": head.get("cold_cache"),
        "cpu_baseline": cpu,
        "decode_queries_s": res["decode1m"]["queries_s"],
        "workloads": {k: res[k] for k in ("decode1m", "prefill8k", "decode128k") if k in res},
    }
    for name in ("blocks", "sets", "backward", "indexer_bwd"):
        if name in res:
            line[name] = res[name]
    probes = probe_peaks()
    log(f"probe peaks: HBM copy {probes['hbm_copy_gbs']} GB/s, read {probes['hbm_read_gbs']} GB/s, bf16 GEMM "
        f"{probes['bf16_gemm_tflops']} TFLOP/s, int8 GEMM {probes['int8_gemm_tops']} TOP/s, gather from "
        f"128 MiB {probes['gather_128mib_256b_gbs']} GB/s (256 B rows), "
        f"{probes['gather_128mib_1kib_gbs']} GB/s (1 KiB rows)")
    line["probe_peaks"] = probes
    add_probe_fracs(line, probes)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
