"""Benchmark of the gated fine-grained sparse attention layer on one MI355X.

One step = one fused pass of the whole layer (indexer scoring -> Top-K ->
sparse attention -> sigmoid gate) over the Prefill-8K workload: batch 1, 8192
causal tokens, 32 query heads over 4 KV heads, head dim 128, 8 int8 indexer
heads of dim 64, K = 2048, synthetic seeded inputs already resident in HBM.
Prints ONE JSON line (rank 0). The same line carries the Decode-128K fused step
(64 single-token queries over 131072-token histories), a per-kernel breakdown,
the roofline of the dominant kernel (timed with HIP events on the stream it is
launched on) and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tok/s + decode queries/s at K=2048; % of HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# HBM traffic of the dominant kernel from rocprofv3 counter passes (one pass
# for FETCH_SIZE, one for WRITE_SIZE, KiB per dispatch, Prefill-8K step), each
# scaled by what the same counter reads for a plain 2 GiB device copy kernel
# (FETCH_SIZE reads 1 GiB for its 2 GiB of reads: x2.0; WRITE_SIZE reads
# 2 GiB for its 2 GiB of writes: x1.0). Valid only for the kernel sources the
# counters were taken on: any change to them turns the figure into null.
TRAFFIC = {
    "attn_dense": dict(fetch_kib=125491.6, fetch_scale=2.0, write_kib=65872.8, write_scale=1.0,
                       sources=("long_context_indexer_amd/csrc/attn_dense.hip",
                                "long_context_indexer_amd/csrc/attn_dense.h",
                                "long_context_indexer_amd/csrc/common.h",
                                "long_context_indexer_amd/csrc/tile.h"),
                       sha256="45fc9c45a4d3eae9a5358e73e3237d7295431079bcb32d4cfc35ae5bb2d83d0b"),
}


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """HBM bytes per launch from the recorded counters, or None when the kernel's
    sources changed since they were taken (or none were taken)."""
    t = TRAFFIC.get(kernel)
    if t is None or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def causal_pairs(cfg):
    """(query, key) pairs the layer touches: sum over rows of min(K, p+1)."""
    if cfg.decode:
        return cfg.B * min(cfg.K, cfg.Tk)
    t = np.arange(cfg.Tq, dtype=np.int64)
    return int(cfg.B * np.minimum(cfg.K, t + 1).sum())


def scored_pairs(cfg):
    """(query, history position) pairs the indexer scores: sum over rows of p+1."""
    if cfg.decode:
        return cfg.B * cfg.Tk
    return cfg.B * cfg.Tq * (cfg.Tq + 1) // 2


def attn_flops(cfg):
    return 4.0 * cfg.Hq * cfg.d * causal_pairs(cfg)


def idx_ops(cfg):
    return 2.0 * cfg.H_I * cfg.d_I * scored_pairs(cfg)


def decode_attn_bytes(cfg):
    """Algorithmic HBM bytes of sparse attention per decode query: the K selected
    key and value rows of every KV head, plus q, gate, out and the index row."""
    return cfg.B * (cfg.K * cfg.Hkv * cfg.d * 2 * 2 + 3 * cfg.Hq * cfg.d * 2 + cfg.K * 4)


def decode_step_bytes(cfg):
    """Algorithmic HBM bytes of the whole decode step per query: the indexer key
    cache of the whole history, q_idx, and the sparse-attention bytes."""
    return cfg.B * (cfg.Tk * cfg.d_I + cfg.H_I * cfg.d_I) + decode_attn_bytes(cfg)


def append_bytes(rows, Hkv, d, d_I):
    """Algorithmic HBM bytes of appending rows to the caches: every new key,
    value and indexer-key row read once and written once."""
    return 2 * rows * (2 * Hkv * d * 2 + d_I)


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


def cold_steps(step, steps, stream):
    """Each step timed alone (events on the launch stream) after the
    last-level cache has been flushed by streaming a 1 GiB buffer outside the
    timed span: inputs are in HBM but no longer in any cache. Median ms."""
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


def timed_region(timer, step, steps, lci):
    """Time `steps` steps (wall clock and stream events around the whole region),
    then run `steps` more with the library's per-kernel event log switched on
    (events around every launch, on the launch stream). The log's events add a
    few microseconds per launch, so the headline step time comes from the first
    region and only the per-kernel durations from the second."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_ms = timer.time(step, steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
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
    return wall_ms, ev_ms, kern


def roofline(cfg, kern):
    """Roofline of the kernel that takes the most time per prefill step.
    achieved = the algorithmic work that kernel does per step / its summed launch
    durations per step (its event-timed average launch time x launches/step)."""
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    ms = kern[dom]["ms_per_step"]
    if dom in ("attn_dense", "attn_gather"):
        # every Prefill-8K row keeps at least a quarter of its history, so all rows
        # take the dense-tile kernel: its work is the whole layer's attention
        ach = attn_flops(cfg) / ms / 1e9
        r = dict(kernel=dom, bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS,
                 unit="TFLOP/s", frac=ach / PEAK_BF16_TFLOPS, traffic=None)
    elif dom == "idx_score":
        ach = idx_ops(cfg) / ms / 1e9
        r = dict(kernel=dom, bound="mfma", achieved=ach, peak=PEAK_INT8_TOPS, unit="TOP/s",
                 frac=ach / PEAK_INT8_TOPS, traffic=None)
    else:
        nbytes = 4.0 * scored_pairs(cfg) + 4.0 * cfg.B * cfg.Tq * cfg.K
        ach = nbytes / ms / 1e6
        r = dict(kernel=dom, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                 frac=ach / PEAK_HBM_GBS, traffic=None)
    r["traffic"] = traffic_bytes(dom)
    r.update(traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                          "copy-calibrated)",
             launches_per_step=kern[dom]["launches_per_step"],
             avg_launch_ms=kern[dom]["avg_launch_ms"])
    return r


def cpu_baseline(cfg, inp_host, budget_s):
    """The oracle as it stands, on uniformly sampled query rows of the same
    workload (an unbiased sample of per-row work), as tokens/s."""
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
                sample=f"{n_done} query rows drawn uniformly from the {cfg.Tq} rows of the "
                       f"Prefill-8K workload, whole layer per row, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "prefill64k", "decode1m", "blocks",
                                       "sets", "backward"],
                    default=None,
                    help="run only one fused step (profiler runs; prefill64k and decode1m are "
                         "the long-context workloads, outside the default run)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 2 GiB device buffer 5 times (HBM counter calibration runs)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for {args.gpus}); the "
              "multi-GPU split of the path is a design note, not a runnable mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_indexer_amd as lci
    import synth

    lci.load_library()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    timer = Timer(stream)
    res = {}

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def run_prefill(name, inp_host):
        cfg = synth.CONFIGS[name]
        d = {k: dev(v) for k, v in inp_host.items() if isinstance(v, np.ndarray)}
        geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I)
        ws = torch.empty(lci.workspace_bytes(lci.ENTRY_PREFILL, geom), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty_like(d["q"])

        def prefill_step():
            lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                            cfg.scale, d["q_offset"], d["kv_len"], cfg.K, out=out, workspace=ws,
                            stream=stream)

        for _ in range(args.warmup):
            prefill_step()
        torch.cuda.synchronize()
        ms_step, ev_ms, kern = timed_region(timer, prefill_step, args.steps, lci)
        tok_s = cfg.B * cfg.Tq / (ms_step * 1e-3)
        cold_ms = cold_steps(prefill_step, args.steps, stream)
        # appending the whole prompt as one chunk to caches of this shape (the
        # new rows are a copy of the cache contents, so the inputs stay as they are)
        app_ms, len_ms = time_append(lci, d["k"].clone(), d["v"].clone(), d["k_idx"].clone(),
                                     d["k"], d["v"], d["k_idx"],
                                     torch.zeros_like(d["kv_len"]), 20, stream)
        app_b = append_bytes(cfg.B * cfg.Tk, cfg.Hkv, cfg.d, cfg.d_I)
        log(f"{name} fused: {ms_step:.3f} ms/step ({ev_ms:.3f} ms by events), "
            f"{tok_s / 1e6:.2f} M tok/s; cold cache {cold_ms:.3f} ms/step")
        log(f"  kv_append of the {cfg.B * cfg.Tk} prompt rows: {app_ms * 1e3:.1f} us "
            f"({app_b / app_ms / 1e6:.0f} GB/s) + lengths {len_ms * 1e3:.1f} us")
        for kname, kv in kern.items():
            log(f"  {kname:12s} {kv['launches_per_step']:.0f} launch(es)/step, "
                f"{kv['ms_per_step'] * 1e3:8.1f} us/step")
        return dict(workload=name, ms_per_step=ms_step, event_ms_per_step=ev_ms, tok_s=tok_s,
                    cold_ms_per_step=cold_ms, cold_tok_s=cfg.B * cfg.Tq / (cold_ms * 1e-3),
                    kernels=kern,
                    kv_append=dict(rows=cfg.B * cfg.Tk, us=app_ms * 1e3, lengths_us=len_ms * 1e3,
                                   bytes=app_b, gbs=app_b / app_ms / 1e6,
                                   frac_hbm=app_b / app_ms / 1e6 / PEAK_HBM_GBS))

    def run_variant(cfg, inp_host, block, kb, sets):
        """Prefill-8K with block-granular selection and/or index sets per key/value head."""
        torch.cuda.empty_cache()   # the buffers of earlier legs go back to the device
        d = {k: dev(v) for k, v in inp_host.items() if isinstance(v, np.ndarray)}
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
        ms_step, ev_ms, kern = timed_region(timer, step, args.steps, lci)
        tok_s = cfg.B * cfg.Tq / (ms_step * 1e-3)
        log(f"prefill8k, blocks of {block} ({kb} kept), {sets} index set(s): {ms_step:.3f} "
            f"ms/step, {tok_s / 1e6:.2f} M tok/s")
        for kname, kv in kern.items():
            log(f"  {kname:12s} {kv['launches_per_step']:.0f} launch(es)/step, "
                f"{kv['ms_per_step'] * 1e3:8.1f} us/step")
        return dict(workload="prefill8k", block=block, kept=kb, index_sets=sets, ms_per_step=ms_step,
                    event_ms_per_step=ev_ms, tok_s=tok_s,
                    kernels_us_per_step={k: round(v["ms_per_step"] * 1e3, 2)
                                         for k, v in kern.items()})

    def run_backward(cfg, inp_host):
        """Gradients of attention + gate for the Prefill-8K index rows (from the
        fused forward) and a random bf16 output gradient."""
        torch.cuda.empty_cache()
        d = {k: dev(v) for k, v in inp_host.items() if isinstance(v, np.ndarray)}
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
        ms_step, ev_ms, kern = timed_region(timer, step, steps, lci)
        pairs = causal_pairs(cfg)
        tflops = 10.0 * cfg.d * cfg.Hq * pairs / (ms_step * 1e-3) / 1e12
        log(f"prefill8k backward: {ms_step:.3f} ms/step, {cfg.Tq / ms_step * 1e3 / 1e6:.2f} M tok/s, "
            f"{tflops:.1f} TFLOP/s of backward work")
        for kname, kv in kern.items():
            log(f"  {kname:12s} {kv['launches_per_step']:.0f} launch(es)/step, "
                f"{kv['ms_per_step'] * 1e3:8.1f} us/step")
        return dict(workload="prefill8k", ms_per_step=ms_step, event_ms_per_step=ev_ms,
                    tok_s=cfg.B * cfg.Tq / (ms_step * 1e-3), steps=steps,
                    tflops=tflops, note="dq, dk, dv, dgate for the layer's index rows; "
                    "10*d flops per (query head, selected key); forward recomputed inside",
                    kernels_us_per_step={k: round(v["ms_per_step"] * 1e3, 2)
                                         for k, v in kern.items()})

    def run_decode(name):
        dcfg = synth.CONFIGS[name]
        dd = synth.device_inputs(dcfg, seed=0)
        dgeom = lci.make_geom(dcfg.B, dcfg.Tq, dcfg.Tk, dcfg.K, dd["q_offset"], dd["kv_len"],
                              Hq=dcfg.Hq, Hkv=dcfg.Hkv, d=dcfg.d, H_I=dcfg.H_I, d_I=dcfg.d_I)
        dws = torch.empty(lci.workspace_bytes(lci.ENTRY_DECODE, dgeom), dtype=torch.uint8,
                          device="cuda")
        dout = torch.empty_like(dd["q"])
        didx = torch.empty((dcfg.B, 1, dcfg.K), dtype=torch.int32, device="cuda")

        def decode_step():
            lci.decode_fwd(dd["q_idx"], dd["k_idx"], dd["w"], dd["q"], dd["k"], dd["v"],
                           dd["gate"], dcfg.scale, dd["q_offset"], dd["kv_len"], dcfg.K,
                           out=dout, idx_out=didx, workspace=dws, stream=stream)

        for _ in range(args.warmup):
            decode_step()
        torch.cuda.synchronize()
        dms, dev_ms, dkern = timed_region(timer, decode_step, args.steps, lci)
        qps = dcfg.B / (dms * 1e-3)
        abytes = decode_attn_bytes(dcfg)
        sbytes = decode_step_bytes(dcfg)
        a_ms = sum(dkern[k]["ms_per_step"] for k in ("attn_gather", "attn_combine") if k in dkern)
        log(f"{name} fused: {dms:.3f} ms/step, {qps:.0f} queries/s, whole step "
            f"{sbytes / dms / 1e6:.0f} GB/s; attention kernels {a_ms * 1e3:.1f} us = "
            f"{abytes / a_ms / 1e6:.0f} GB/s")
        for kname, kv in dkern.items():
            log(f"  {kname:12s} {kv['launches_per_step']:.0f} launch(es)/step, "
                f"{kv['ms_per_step'] * 1e3:8.1f} us/step")
        # appending one token per sequence: the new rows are each history's last
        # row, written back where it is (kv_len = Tk - 1), so the inputs stay as they are
        last = slice(dcfg.Tk - 1, dcfg.Tk)
        app_ms, len_ms = time_append(lci, dd["k"][:, last].contiguous(),
                                     dd["v"][:, last].contiguous(),
                                     dd["k_idx"][:, last].contiguous(), dd["k"], dd["v"],
                                     dd["k_idx"], torch.full_like(dd["kv_len"], dcfg.Tk - 1),
                                     20, stream)
        app_b = append_bytes(dcfg.B, dcfg.Hkv, dcfg.d, dcfg.d_I)
        log(f"  kv_append of one token per sequence: {app_ms * 1e3:.1f} us + lengths "
            f"{len_ms * 1e3:.1f} us")
        return dict(workload=name, ms_per_step=dms, event_ms_per_step=dev_ms, queries_s=qps,
                    step_hbm_gbs=sbytes / dms / 1e6,
                    step_frac_hbm=sbytes / dms / 1e6 / PEAK_HBM_GBS,
                    kv_append=dict(rows=dcfg.B, us=app_ms * 1e3, lengths_us=len_ms * 1e3,
                                   bytes=app_b),
                    sparse_attn_ms=a_ms, sparse_attn_gbs=abytes / a_ms / 1e6,
                    sparse_attn_frac_hbm=abytes / a_ms / 1e6 / PEAK_HBM_GBS,
                    kernels=dkern)

    if args.only in ("prefill64k", "decode1m"):
        if args.only == "prefill64k":
            res["prefill64k"] = run_prefill("prefill64k", synth.host_inputs(
                synth.CONFIGS["prefill64k"], seed=0))
        else:
            res["decode1m"] = run_decode("decode1m")
        print(json.dumps(res))
        return

    # ---------------------------------------------------------------- prefill 8K
    cfg = synth.CONFIGS["prefill8k"]
    inp_host = synth.host_inputs(cfg, seed=0)
    if args.only in (None, "prefill"):
        res["prefill"] = run_prefill("prefill8k", inp_host)

    # ------------------------------------------- Prefill 8K, block-granular selection
    # blocks of 64 positions, 32 kept: the same 2048 positions per row as the
    # position Top-K, chosen as whole blocks
    if args.only in (None, "blocks"):
        res["blocks"] = run_variant(cfg, inp_host, 64, 32, 1)
    # one index set per key/value head (4 sets of 2 indexer heads), K = 2048
    if args.only in (None, "sets"):
        res["sets"] = run_variant(cfg, inp_host, 1, cfg.K, cfg.Hkv)

    # ------------------------------------------- Prefill 8K gradients (training direction)
    if args.only in (None, "backward"):
        res["backward"] = run_backward(cfg, inp_host)

    # --------------------------------------------------------------- decode 128K
    if not args.no_decode and args.only in (None, "decode"):
        res["decode"] = run_decode("decode128k")

    if args.only is not None:
        print(json.dumps(res))
        return

    # ------------------------------------------------------------------ report
    pre = res["prefill"]
    roof = roofline(cfg, pre["kernels"])

    cpu = None
    if not args.no_cpu:
        torch.cuda.synchronize()
        cpu = cpu_baseline(cfg, inp_host, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.1f} tok/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": pre["tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "indexer_dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "prefill8k", "batch": cfg.B, "seq_len": cfg.Tq, "Hq": cfg.Hq,
                   "Hkv": cfg.Hkv, "head_dim": cfg.d, "H_I": cfg.H_I, "d_I": cfg.d_I,
                   "top_k": cfg.K, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "kernels_us_per_step": {k: round(v["ms_per_step"] * 1e3, 2)
                                for k, v in pre["kernels"].items()},
        "cold_cache": {"ms_per_step": pre["cold_ms_per_step"], "tok_s": pre["cold_tok_s"],
                       "note": "median of single steps, each after a 1 GiB cache flush"},
        "cpu_baseline": cpu,
        "kv_append": dict(pre["kv_append"], note="the whole prompt appended as one chunk to "
                          "the key/value/indexer-key caches (copy kernel; lengths kernel apart)"),
    }
    for name in ("blocks", "sets", "backward"):
        if name in res:
            line[name] = res[name]
    if "decode" in res:
        line["decode"] = res["decode"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
