"""Helpers for the GPU parity tests: host<->device conversion of the synthetic
inputs, the bf16 tolerance check, and per-row oracle sub-problems for sampled
checks at full size."""
from __future__ import annotations

import sys

import numpy as np

# Attention tolerance on bf16 outputs (max-abs and relative L2 over the compared rows)
MAX_ABS = 2e-2
REL_L2 = 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    import torch
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def to_device(inp, device="cuda"):
    return {k: (dev(v, device) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


def bf16_f64(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attn_errors(got_bits, ref):
    got = bf16_f64(got_bits).reshape(ref.shape)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_attn_close(got_bits, ref, what=""):
    max_abs, rel = attn_errors(got_bits, ref)
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= MAX_ABS and rel <= REL_L2, (what, max_abs, rel)


def row_problem(inp_dev, b, i):
    """Host inputs of one query row (b, i) as a B=1, Tq=1 problem over positions
    0..p: the oracle's answer for the row depends on nothing else."""
    qo = int(host(inp_dev["q_offset"])[b]) if not isinstance(inp_dev["q_offset"], np.ndarray) \
        else int(inp_dev["q_offset"][b])
    kvl = int(host(inp_dev["kv_len"])[b]) if not isinstance(inp_dev["kv_len"], np.ndarray) \
        else int(inp_dev["kv_len"][b])
    p = qo + i
    n = min(p + 1, kvl)

    def sl(t, *idx):
        x = t[idx]
        return host(x) if not isinstance(x, np.ndarray) else np.ascontiguousarray(x)

    w = inp_dev["w"]
    w_h = host(w) if not isinstance(w, np.ndarray) else w
    if w_h.ndim == 3:
        w_h = w_h[b, i]
    elif w_h.ndim == 2:
        w_h = w_h[i]
    return dict(
        q_idx=sl(inp_dev["q_idx"], slice(b, b + 1), slice(i, i + 1)),
        k_idx=sl(inp_dev["k_idx"], slice(b, b + 1), slice(0, n)),
        w=np.ascontiguousarray(w_h),
        q=sl(inp_dev["q"], slice(b, b + 1), slice(i, i + 1)),
        gate=None if inp_dev.get("gate") is None else sl(inp_dev["gate"], slice(b, b + 1), slice(i, i + 1)),
        k=sl(inp_dev["k"], slice(b, b + 1), slice(0, n)),
        v=sl(inp_dev["v"], slice(b, b + 1), slice(0, n)),
        q_offset=np.array([p], np.int32),
        kv_len=np.array([min(kvl, n) if p < kvl else kvl], np.int32),
        scale=inp_dev["scale"],
    )
