"""Seeded synthetic inputs for the gated fine-grained sparse attention layer.

This module only draws random inputs and plants needles. It holds none of the
layer's arithmetic (no scoring, no selection, no attention, no gate), so both
the CPU oracle's tests and the GPU path can take their inputs from it without
sharing any computation.

Workloads (shapes, value distributions, needle structure) follow the five
synthetic configurations that stand in for the pages' long-context retrieval
workloads (multi-needle haystack tests, TTFT/throughput curves across context
lengths): "Hybrid Sparse Attention for Long-Context LLMs" (Engineering and
Evaluation Recommendations) and "How Fine-Grained Sparse Attention Reshapes
Long-Context Architecture" (Evaluation Checklist).

Two generators:
  * ``host_inputs``   numpy PCG64, one SeedSequence per (seed, config, tensor,
                      sequence); used for every size the CPU can hold cheaply.
  * ``device_inputs`` torch's device generator, one seed per (config, tensor,
                      sequence), generated sequence by sequence on the GPU; used
                      for the multi-GiB decode histories. Host copies of any
                      slice the oracle needs are taken from these tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

T_Q, T_K, T_V, T_G, T_QI, T_KI, T_W, T_NEEDLE, T_MIX = range(9)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    B: int
    Tq: int          # query rows per sequence
    Tk: int          # history rows per sequence (allocated)
    decode: bool     # True: one query per sequence at position Tk-1
    Hq: int
    Hkv: int
    d: int
    H_I: int
    d_I: int
    K: int
    needles: str     # "none" | "random" | "stride4096" | "decode"
    n_needles: int = 0
    fp32_source: bool = False   # Q/K/V/G drawn in fp32 and then rounded to bf16
    q_range: int = 8            # indexer q/k uniform in [-q_range, q_range]
    w_lo: int = 1               # indexer head weights uniform in [w_lo, w_hi]
    w_hi: int = 4

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as a float32 value."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def q_offset(self, b: int) -> int:
        return self.Tk - 1 if self.decode else 0

    def kv_len(self, b: int) -> int:
        return self.Tk

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 0, B=1, Tq=256, Tk=256, decode=False, Hq=4, Hkv=1, d=64,
                   H_I=2, d_I=32, K=32, needles="none", fp32_source=True),
    "prefill8k": Config("prefill8k", 1, B=1, Tq=8192, Tk=8192, decode=False, Hq=32, Hkv=4,
                        d=128, H_I=8, d_I=64, K=2048, needles="random", n_needles=16),
    "decode128k": Config("decode128k", 2, B=64, Tq=1, Tk=131072, decode=True, Hq=32, Hkv=4,
                         d=128, H_I=8, d_I=64, K=2048, needles="none"),
    "prefill64k": Config("prefill64k", 3, B=1, Tq=65536, Tk=65536, decode=False, Hq=32,
                         Hkv=4, d=128, H_I=8, d_I=64, K=2048, needles="stride4096",
                         n_needles=16),
    "decode1m": Config("decode1m", 4, B=8, Tq=1, Tk=1048576, decode=True, Hq=32, Hkv=4,
                       d=128, H_I=8, d_I=64, K=2048, needles="decode", n_needles=32),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, cfg: Config, tensor: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg.cfg_id, tensor, b])))


def head_star(w: np.ndarray) -> int:
    """Index of the largest indexer head weight, lowest index on ties."""
    return int(np.argmax(np.asarray(w)))


def needle_plan(cfg: Config, seed: int, b: int):
    """(key position p, query row t) pairs for sequence b."""
    if cfg.needles == "none" or cfg.n_needles == 0:
        return []
    r = _rng(seed, cfg, T_NEEDLE, b)
    if cfg.needles in ("random", "stride4096"):
        # prefill: query row t sits at position t, so a needle key at p < t is causal
        T = min(cfg.Tq, cfg.Tk)
        if cfg.needles == "random":
            n = min(cfg.n_needles, T - 1)
            ps = r.choice(T - 1, size=n, replace=False) if n > 0 else []
            return [(int(p), int(r.integers(p + 1, T))) for p in ps]
        return [(4096 * j, int(r.integers(4096 * j + 1, T))) for j in range(cfg.n_needles)
                if 4096 * j + 1 < T]
    T = cfg.Tk
    if cfg.needles == "decode":
        ps = r.choice(T, size=cfg.n_needles, replace=False)
        return [(int(p), 0) for p in ps]
    raise ValueError(cfg.needles)


def host_inputs(cfg: Config, seed: int = 0) -> dict:
    """All inputs of one configuration as host numpy arrays.

    Keys: q_idx int8 [B,Tq,H_I,d_I]; k_idx int8 [B,Tk,d_I]; w int8 [H_I] (one
    weight per indexer head, broadcast over sequences and rows); q, gate uint16
    (bf16 bits) [B,Tq,Hq,d]; k, v uint16 [B,Tk,Hkv,d]; q_offset, kv_len int32 [B];
    scale float; needles list per sequence. fp32 sources are kept under
    ``*_f32`` when the configuration draws them in fp32.
    """
    B, Tq, Tk = cfg.B, cfg.Tq, cfg.Tk
    out = {}
    w = _rng(seed, cfg, T_W, 0).integers(cfg.w_lo, cfg.w_hi + 1, size=cfg.H_I, dtype=np.int8)
    hs = head_star(w)
    q_idx = np.empty((B, Tq, cfg.H_I, cfg.d_I), np.int8)
    k_idx = np.empty((B, Tk, cfg.d_I), np.int8)
    qf = np.empty((B, Tq, cfg.Hq, cfg.d), np.float32)
    kf = np.empty((B, Tk, cfg.Hkv, cfg.d), np.float32)
    vf = np.empty((B, Tk, cfg.Hkv, cfg.d), np.float32)
    gf = np.empty((B, Tq, cfg.Hq, cfg.d), np.float32)
    lo, hi = -cfg.q_range, cfg.q_range + 1
    needles = []
    for b in range(B):
        q_idx[b] = _rng(seed, cfg, T_QI, b).integers(lo, hi, size=q_idx.shape[1:], dtype=np.int8)
        k_idx[b] = _rng(seed, cfg, T_KI, b).integers(lo, hi, size=k_idx.shape[1:], dtype=np.int8)
        qf[b] = _rng(seed, cfg, T_Q, b).standard_normal(qf.shape[1:], dtype=np.float32)
        kf[b] = _rng(seed, cfg, T_K, b).standard_normal(kf.shape[1:], dtype=np.float32)
        vf[b] = _rng(seed, cfg, T_V, b).standard_normal(vf.shape[1:], dtype=np.float32)
        gf[b] = _rng(seed, cfg, T_G, b).standard_normal(gf.shape[1:], dtype=np.float32)
        plan = needle_plan(cfg, seed, b)
        for p, t in plan:
            for g in range(cfg.Hkv):
                kf[b, p, g] = qf[b, t, g * cfg.G]
            k_idx[b, p] = q_idx[b, t, hs]
        needles.append(plan)
    out.update(q_idx=q_idx, k_idx=k_idx, w=w,
               q=bf16_bits(qf), k=bf16_bits(kf), v=bf16_bits(vf), gate=bf16_bits(gf),
               q_offset=np.array([cfg.q_offset(b) for b in range(B)], np.int32),
               kv_len=np.array([cfg.kv_len(b) for b in range(B)], np.int32),
               scale=cfg.scale, needles=needles)
    if cfg.fp32_source:
        out.update(q_f32=qf, k_f32=kf, v_f32=vf, gate_f32=gf)
    return out


def host_mix(cfg: Config, seed: int = 0) -> np.ndarray:
    """The other branch's output for the gate to mix with (the linear or
    compressed attention the pages pair the sparse branch with): uint16 (bf16
    bits) [B,Tq,Hq,d] of standard normals, its own stream per sequence."""
    m = np.empty((cfg.B, cfg.Tq, cfg.Hq, cfg.d), np.float32)
    for b in range(cfg.B):
        m[b] = _rng(seed, cfg, T_MIX, b).standard_normal(m.shape[1:], dtype=np.float32)
    return bf16_bits(m)


def index_rows(q_offset: np.ndarray, kv_len: np.ndarray, Tq: int, K: int,
               seed: int = 0) -> np.ndarray:
    """Random valid index rows int32 [B,Tq,K]: row i of sequence b (position
    p = q_offset[b] + i) lists min(K, p+1) distinct positions of 0..p in
    increasing order, then -1; rows past the history (p >= kv_len[b]) are all
    -1. An input for the attention and its gradients without running a
    selection (uniform choice, no scores)."""
    B = len(q_offset)
    out = np.full((B, Tq, K), -1, np.int32)
    r = np.random.default_rng(seed)
    for b in range(B):
        for i in range(Tq):
            p = int(q_offset[b]) + i
            if p >= int(kv_len[b]):
                continue
            if p + 1 <= K:
                out[b, i, :p + 1] = np.arange(p + 1, dtype=np.int32)
            else:
                out[b, i] = np.sort(r.choice(p + 1, K, replace=False)).astype(np.int32)
    return out


def device_inputs(cfg: Config, seed: int = 0, device: str = "cuda") -> dict:
    """All inputs of one configuration as device torch tensors, drawn on the GPU.

    Same shapes and distributions as ``host_inputs`` (bf16 tensors are
    torch.bfloat16, rounded to nearest even from float32 normals); the values
    come from torch's device generator and so differ from the numpy stream.
    Generated one sequence at a time so the float32 staging stays small.
    """
    import torch

    B, Tq, Tk = cfg.B, cfg.Tq, cfg.Tk
    gen = torch.Generator(device=device)

    def seeded(tensor: int, b: int) -> "torch.Generator":
        gen.manual_seed(((seed * 1_000_003 + cfg.cfg_id) * 97 + tensor) * 1_000_003 + b)
        return gen

    w_np = _rng(seed, cfg, T_W, 0).integers(cfg.w_lo, cfg.w_hi + 1, size=cfg.H_I, dtype=np.int8)
    hs = head_star(w_np)
    w = torch.from_numpy(w_np).to(device)
    q_idx = torch.empty((B, Tq, cfg.H_I, cfg.d_I), dtype=torch.int8, device=device)
    k_idx = torch.empty((B, Tk, cfg.d_I), dtype=torch.int8, device=device)
    q = torch.empty((B, Tq, cfg.Hq, cfg.d), dtype=torch.bfloat16, device=device)
    gate = torch.empty_like(q)
    k = torch.empty((B, Tk, cfg.Hkv, cfg.d), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    lo, hi = -cfg.q_range, cfg.q_range + 1
    needles = []
    for b in range(B):
        q_idx[b] = torch.randint(lo, hi, q_idx.shape[1:], generator=seeded(T_QI, b),
                                 dtype=torch.int8, device=device)
        k_idx[b] = torch.randint(lo, hi, k_idx.shape[1:], generator=seeded(T_KI, b),
                                 dtype=torch.int8, device=device)
        for dst, tid in ((q, T_Q), (gate, T_G), (k, T_K), (v, T_V)):
            # draw in slabs of at most 2^26 values to bound the float32 staging buffer
            flat = dst[b].view(-1)
            g = seeded(tid, b)
            step = 1 << 26
            for s in range(0, flat.numel(), step):
                n = min(step, flat.numel() - s)
                flat[s:s + n] = torch.randn(n, generator=g, dtype=torch.float32,
                                            device=device).to(torch.bfloat16)
        plan = needle_plan(cfg, seed, b)
        for p, t in plan:
            for g_ in range(cfg.Hkv):
                k[b, p, g_] = q[b, t, g_ * cfg.G]
            k_idx[b, p] = q_idx[b, t, hs]
        needles.append(plan)
    q_offset = torch.tensor([cfg.q_offset(b) for b in range(B)], dtype=torch.int32, device=device)
    kv_len = torch.tensor([cfg.kv_len(b) for b in range(B)], dtype=torch.int32, device=device)
    return dict(q_idx=q_idx, k_idx=k_idx, w=w, q=q, k=k, v=v, gate=gate, q_offset=q_offset,
                kv_len=kv_len, scale=cfg.scale, needles=needles)


def scaled(cfg: Config, **kw) -> Config:
    """A reduced copy of a configuration (parity cases at sizes the oracle finishes quickly)."""
    return cfg.replace(**kw)
