"""GPU parity of the gradients of the scorer's distillation loss
(lci_indexer_bwd) against the oracle's fp64 chain rule.

Tolerance: the kernels compute the scores exactly (int8 rows, int32 sums) and
everything after them in fp32: tau*S (2^-24 relative), the softmax with the
hardware exp and log (about 1 ulp each), sums of up to 4096 terms in fp32, and
dk in 32.32 fixed point (2^-33 per contribution). Allowed: relative L2 1e-4 and
max-abs 1e-3 of the largest reference value, per gradient and for the loss.
dq, dk and dw must be bit-identical across calls."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, log, to_device

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
MAX_REL = 1e-3
TINY = synth.CONFIGS["tiny"]
MED = synth.CONFIGS["prefill8k"].replace(Tq=200, Tk=700, K=128, n_needles=0, needles="none")


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def _close(got, want, what):
    got = np.asarray(got, np.float64)
    diff = got - want
    scale = max(np.abs(want).max(), 1e-30)
    rel = np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30)
    mx = np.abs(diff).max() / scale
    log(f"  {what}: rel_l2={rel:.2e} max/ref_max={mx:.2e}")
    assert rel <= REL_L2 and mx <= MAX_REL, (what, rel, mx)


def _teacher(r, shape, normalised=True):
    T = r.random(shape) ** 3           # uneven weights
    if normalised:
        T /= T.sum(-1, keepdims=True)
    return T.astype(np.float32)


def _case(orc, name):
    r = np.random.default_rng(90)
    if name == "tiny_topk":
        cfg = TINY.replace(Tq=64, Tk=256)
        inp = synth.host_inputs(cfg, seed=90)
        inp["q_offset"] = np.array([192], np.int32)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, _teacher(r, idx.shape), 0.01
    if name == "med_rowweights_ragged":
        cfg = MED.replace(B=2)
        inp = synth.host_inputs(cfg, seed=91)
        inp["q_offset"] = np.array([0, 450], np.int32)
        inp["kv_len"] = np.array([700, 640], np.int32)
        inp["w"] = r.integers(-4, 6, size=(cfg.B, cfg.Tq, cfg.H_I)).astype(np.int8)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, _teacher(r, idx.shape), 0.003
    if name == "scrambled_padding":
        cfg = TINY.replace(Tq=40, Tk=120, K=24, H_I=4, d_I=64)
        inp = synth.host_inputs(cfg, seed=92)
        inp["q_offset"] = np.array([70], np.int32)
        inp["kv_len"] = np.array([105], np.int32)          # rows 35.. are invalid
        idx = np.stack([r.permutation(111)[:cfg.K] for _ in range(cfg.Tq)]).astype(np.int32)[None]
        idx[0, 3, 10:] = -1
        idx[0, 5, :] = 110                                   # past every row's position
        idx[0, 7, 2] = idx[0, 7, 1]                          # a repeated position
        T = _teacher(r, idx.shape, normalised=False)         # teachers not summing to 1
        return cfg, inp, idx, T, 0.02
    if name == "h16d64":
        cfg = TINY.replace(Tq=96, Tk=300, K=48, H_I=16, d_I=64)
        inp = synth.host_inputs(cfg, seed=93)
        inp["q_offset"] = np.array([204], np.int32)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, _teacher(r, idx.shape), 0.002
    if name == "h8d128_int8_extremes":
        cfg = TINY.replace(Tq=80, Tk=200, K=40, H_I=8, d_I=128)
        inp = synth.host_inputs(cfg, seed=94)
        inp["q_idx"] = r.integers(-128, 128, size=inp["q_idx"].shape).astype(np.int8)
        inp["k_idx"] = r.integers(-128, 128, size=inp["k_idx"].shape).astype(np.int8)
        inp["w"] = r.integers(-128, 128, size=cfg.H_I).astype(np.int8)
        inp["q_offset"] = np.array([120], np.int32)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, _teacher(r, idx.shape), 1e-7
    if name == "long_history_global_counts":
        # more positions than the transpose keeps per-block counters for in LDS
        # (16384): the per-entry atomic count and fill
        cfg = TINY.replace(Tq=48, Tk=20000, K=64, H_I=4, d_I=64)
        inp = synth.host_inputs(cfg, seed=98)
        inp["q_offset"] = np.array([19900], np.int32)
        inp["kv_len"] = np.array([19948], np.int32)
        idx = np.stack([r.choice(19900 + i + 1, cfg.K, replace=False) for i in range(cfg.Tq)])
        idx = idx.astype(np.int32)[None]
        idx[0, :, 0] = 7                                     # a position every row points at
        return cfg, inp, idx, _teacher(r, idx.shape), 0.01
    raise KeyError(name)


CASES = ["tiny_topk", "med_rowweights_ragged", "scrambled_padding", "h16d64",
         "h8d128_int8_extremes", "long_history_global_counts"]


def _run(lci, inp, idx, T, tau):
    import torch
    d = to_device(inp)
    res = lci.indexer_bwd(d["q_idx"], d["k_idx"], d["w"], dev(idx), dev(T), tau, d["q_offset"],
                          d["kv_len"])
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name", CASES)
def test_indexer_bwd(lci, orc, name):
    import torch
    cfg, inp, idx, T, tau = _case(orc, name)
    log(f"indexer bwd {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} H_I={cfg.H_I} d_I={cfg.d_I} "
        f"K={idx.shape[2]} tau={tau}")
    res = _run(lci, inp, idx, T, tau)
    want = orc.indexer_bwd(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"],
                           idx, T, tau)
    for key in ("loss", "dq", "dk", "dw"):
        _close(host(res[key]), want[key], f"{name} {key}")
    res2 = _run(lci, inp, idx, T, tau)
    for key in ("dq", "dk", "dw", "loss"):
        assert torch.equal(res[key], res2[key]), key


def _sets_case(orc, name):
    """(cfg, inp, idx [B,S,Tq,K], teacher, tau): index rows from the oracle's own
    per-set selection, or scrambled rows."""
    r = np.random.default_rng(97)
    if name == "sets2_h8d64":
        cfg, S = TINY.replace(Tq=64, Tk=256, H_I=8, d_I=64), 2
        inp = synth.host_inputs(cfg, seed=97)
        inp["q_offset"] = np.array([192], np.int32)
        tau = 0.01
    elif name == "sets4_rowweights_ragged":
        cfg, S = MED.replace(B=2, H_I=8), 4
        inp = synth.host_inputs(cfg, seed=98)
        inp["q_offset"] = np.array([0, 450], np.int32)
        inp["kv_len"] = np.array([700, 640], np.int32)
        inp["w"] = r.integers(-4, 6, size=(cfg.B, cfg.Tq, cfg.H_I)).astype(np.int8)
        tau = 0.004
    elif name == "sets8_one_head_each":
        cfg, S = TINY.replace(Tq=48, Tk=160, K=32, Hq=8, H_I=8, d_I=32), 8
        inp = synth.host_inputs(cfg, seed=99)
        inp["q_offset"] = np.array([112], np.int32)
        tau = 0.05
    elif name == "sets2_h16d64_scrambled":
        cfg, S = TINY.replace(Tq=40, Tk=120, K=24, H_I=16, d_I=64), 2
        inp = synth.host_inputs(cfg, seed=100)
        inp["q_offset"] = np.array([70], np.int32)
        inp["kv_len"] = np.array([105], np.int32)          # rows 35.. are invalid
        idx = np.stack([np.stack([r.permutation(111)[:cfg.K] for _ in range(cfg.Tq)])
                        for _ in range(S)]).astype(np.int32)[None]
        idx[0, 1, 3, 10:] = -1
        idx[0, 0, 5, :] = 110                               # past every row's position
        T = _teacher(r, idx.shape, normalised=False)
        return cfg, inp, idx, T, 0.002
    else:
        raise KeyError(name)
    lay = orc.layer(inp, cfg.K, sets=S)["idx"].reshape(cfg.B, cfg.Tq, S, cfg.K)
    idx = np.ascontiguousarray(lay.transpose(0, 2, 1, 3))
    return cfg, inp, idx, _teacher(r, idx.shape), tau


SETS_CASES = ["sets2_h8d64", "sets4_rowweights_ragged", "sets8_one_head_each",
              "sets2_h16d64_scrambled"]


@pytest.mark.parametrize("name", SETS_CASES)
def test_indexer_bwd_sets(lci, orc, name):
    """Index sets: set j is the scorer of its group of H_I/S indexer heads over
    its own index rows and teacher; loss per set, dq and dw per head, dk summed
    over the sets, against the oracle; repeat calls bit-identical."""
    import torch
    cfg, inp, idx, T, tau = _sets_case(orc, name)
    log(f"indexer bwd {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} H_I={cfg.H_I} d_I={cfg.d_I} "
        f"sets={idx.shape[1]} K={idx.shape[3]} tau={tau}")
    res = _run(lci, inp, idx, T, tau)
    want = orc.indexer_bwd(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"],
                           idx, T, tau)
    assert tuple(res["loss"].shape) == want["loss"].shape
    for key in ("loss", "dq", "dk", "dw"):
        _close(host(res[key]), want[key], f"{name} {key}")
    res2 = _run(lci, inp, idx, T, tau)
    for key in ("dq", "dk", "dw", "loss"):
        assert torch.equal(res[key], res2[key]), key


def test_indexer_bwd_prefill8k_sampled(lci, orc):
    """The full Prefill-8K size (8192 rows, 8 indexer heads of 64, K = 2048) on
    random valid index rows: loss, dq and dw of rows 0-63 and 8100-8191 against
    the oracle on those rows alone, and dk of positions 8100.. (only rows 8100..
    can select them, so those rows' sums are complete)."""
    import torch
    cfg = synth.CONFIGS["prefill8k"]
    inp = synth.host_inputs(cfg, seed=95)
    idx = synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K, seed=95)
    r = np.random.default_rng(96)
    T = _teacher(r, idx.shape)
    tau = 0.002
    log("indexer bwd prefill8k sampled: B=1 Tq=Tk=8192 H_I=8 d_I=64 K=2048")
    res = _run(lci, inp, idx, T, tau)
    got = {k_: host(res[k_]) for k_ in ("loss", "dq", "dk", "dw")}
    s0 = 8100
    for rows in (slice(0, 64), slice(s0, cfg.Tq)):
        sub_off = np.array([rows.start], np.int32)
        want = orc.indexer_bwd(inp["q_idx"][:, rows], inp["k_idx"], inp["w"], sub_off,
                               inp["kv_len"], idx[:, rows], T[:, rows], tau)
        tag = f"rows {rows.start}-{rows.stop - 1}"
        _close(got["loss"][:, rows], want["loss"], f"8k {tag} loss")
        _close(got["dq"][:, rows], want["dq"], f"8k {tag} dq")
        _close(got["dw"][:, rows], want["dw"], f"8k {tag} dw")
    _close(got["dk"][:, s0:], want["dk"][:, s0:], f"8k keys {s0}.. dk")
