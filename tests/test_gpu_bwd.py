"""GPU parity of the gradients of sparse attention + gate (lci_sparse_attn_bwd)
against the oracle's chain rule in fp64.

Tolerance: the kernels recompute the forward output o and round it to bf16
(2^-9 relative) before it enters delta = do.o and dgate, keep do in bf16 for
delta and the two passes over the selected pairs (2^-9 relative in dv and dP;
the same rounded do in delta and dP keeps sum_t dl_t at the rounding of o),
and accumulate in fp32; dk and dv are summed in 32.32 fixed point (2^-33 per
contribution). The comparison allows relative L2 1e-2 and max-abs 2e-2 of the
largest reference value per gradient (measured: at most 3e-3 and 1.2e-2). dq,
dk and dv must be bit-identical across runs (order-free integer sums)."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, log, to_device

pytestmark = pytest.mark.gpu

MED = synth.CONFIGS["prefill8k"].replace(Tq=300, Tk=300, K=96, n_needles=4)
TINY = synth.CONFIGS["tiny"]
REL_L2 = 1e-2
MAX_REL = 2e-2


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def _close(got, want, what):
    got = got.astype(np.float64)
    diff = got - want
    scale = max(np.abs(want).max(), 1e-30)
    rel = np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30)
    mx = np.abs(diff).max() / scale
    log(f"  {what}: rel_l2={rel:.2e} max/ref_max={mx:.2e}")
    assert rel <= REL_L2 and mx <= MAX_REL, (what, rel, mx)


def _case(orc, name):
    r = np.random.default_rng(60)
    if name == "med_gate_mix":
        cfg = MED
        inp = synth.host_inputs(cfg, seed=60)
        inp["mix"] = synth.host_mix(cfg, seed=60)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, True
    if name == "tiny_scrambled_ungated":
        cfg = TINY.replace(Tq=40, Tk=120, K=24)
        inp = synth.host_inputs(cfg, seed=61)
        inp["kv_len"] = np.array([100], np.int32)      # entries >= 100 are skipped
        idx = np.stack([r.permutation(cfg.Tk)[:cfg.K] for _ in range(cfg.Tq)]).astype(np.int32)
        idx[3, 10:] = -1
        idx[5, :] = -1                                  # a row with no entry
        idx[7, 2] = idx[7, 1]                           # a repeated position
        return cfg, inp, idx[None], False
    if name == "g16_gate":
        cfg = TINY.replace(Hq=16, Hkv=1, d=128, Tq=64, Tk=64, K=80)
        inp = synth.host_inputs(cfg, seed=62)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, True
    if name == "d64_g2_two_sequences":
        cfg = TINY.replace(B=2, Hq=4, Hkv=2, Tq=50, Tk=90, K=30)
        inp = synth.host_inputs(cfg, seed=63)
        inp["q_offset"] = np.array([40, 0], np.int32)
        inp["kv_len"] = np.array([90, 45], np.int32)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, True
    if name == "mixed_paths":
        # rows past 16K (K = 64: p >= 1024) and two out-of-order rows go to the
        # gather kernels, the other token blocks to the tile kernels
        cfg = MED.replace(Tq=1300, Tk=1300, K=64)
        inp = synth.host_inputs(cfg, seed=65)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K).copy()
        for i in (10, 130):
            idx[0, i, :i + 1] = r.permutation(idx[0, i, :i + 1])
        return cfg, inp, idx, True
    if name == "g1_d64":
        # one query head per key/value head
        cfg = TINY.replace(Hq=4, Hkv=4, d=64, Tq=150, Tk=220, K=40)
        inp = synth.host_inputs(cfg, seed=67)
        inp["q_offset"] = np.array([70], np.int32)
        idx = orc.layer(inp, cfg.K)["idx"].reshape(cfg.B, cfg.Tq, cfg.K)
        return cfg, inp, idx, True
    if name == "decode_splits":
        # eight one-row sequences with K >= 128: the forward splits each row's
        # entries, no row takes the tile path, and the gather kernels write dk,
        # dv without a tile pass before them
        cfg = MED.replace(B=8, Tq=1, Tk=4096, K=256, n_needles=0, needles="none")
        inp = synth.host_inputs(cfg, seed=68)
        inp["kv_len"] = np.array([4096, 3000, 17, 256, 257, 4000, 1, 2048], np.int32)
        inp["q_offset"] = inp["kv_len"] - 1
        idx = synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K, seed=68)
        return cfg, inp, idx, True
    if name == "one_chunk_long_history":
        # partial dk, dv of two or more row chunks would take more than 1 GiB
        # (B Tk Hkv d = 136001 * 4 * 128 floats, twice, per chunk): one chunk,
        # the tile kernel writes dk, dv itself, zeros for every key block past
        # the tile rows; rows 1024.. (p + 1 > 16 K) take the gather kernels
        cfg = MED.replace(Tq=1100, Tk=136001, K=64, n_needles=0, needles="none")
        inp = synth.host_inputs(cfg, seed=69)
        idx = synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K, seed=69)
        return cfg, inp, idx, True
    raise KeyError(name)


CASES = ["med_gate_mix", "tiny_scrambled_ungated", "g16_gate", "d64_g2_two_sequences",
         "mixed_paths", "g1_d64", "decode_splits", "one_chunk_long_history"]

# launches of (bwd_dq, bwd_dkdv) per call where the case is there to reach a
# particular arrangement: no tile dq pass (split rows), no partial-sum pass
# (one chunk)
LAUNCHES = {"decode_splits": (1, 1), "one_chunk_long_history": (2, 2), "med_gate_mix": (2, 3)}


@pytest.mark.parametrize("name", CASES)
def test_sparse_attn_bwd(lci, orc, name):
    import torch
    cfg, inp, idx, gated = _case(orc, name)
    r = np.random.default_rng(64)
    dy = synth.bf16_bits(r.standard_normal((cfg.B, cfg.Tq, cfg.Hq, cfg.d), dtype=np.float32))
    gate = inp["gate"] if gated else None
    mix = inp.get("mix") if gated else None
    log(f"bwd {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} "
        f"K={idx.shape[2]} gated={gated} mix={mix is not None}")
    d = to_device(inp)
    lci.kernel_timing(True)
    res = lci.sparse_attn_bwd(d["q"], d["k"], d["v"], dev(idx), dev(gate), inp["scale"],
                              d["kv_len"], dev(dy), mix=dev(mix))
    torch.cuda.synchronize()
    launches = (lci.kernel_timing_read("bwd_dq")[1], lci.kernel_timing_read("bwd_dkdv")[1])
    lci.kernel_timing(False)
    if name in LAUNCHES:
        assert launches == LAUNCHES[name], launches
    want = orc.attention_bwd(inp["q"], inp["k"], inp["v"], gate, idx, inp["kv_len"],
                             inp["scale"], dy, mix=mix)
    for key in ("dq", "dk", "dv", "dgate", "dmix"):
        if want[key] is None:
            assert res[key] is None
            continue
        _close(host(res[key]), want[key], f"{name} {key}")
    # deterministic: a second call gives the same bits
    res2 = lci.sparse_attn_bwd(d["q"], d["k"], d["v"], dev(idx), dev(gate), inp["scale"],
                               d["kv_len"], dev(dy), mix=dev(mix))
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert torch.equal(res[key], res2[key]), key


def test_sparse_attn_bwd_prefill8k_sampled(lci, orc):
    """The gradient call at the full Prefill-8K size of the backward benchmark
    (8192 rows, Hq = 32 over 4 key/value heads, d = 128, K = 2048, every row on
    the tile path) on random valid index rows, checked on what the oracle
    computes from a subset of the rows: dq and dgate of the first 64 and the
    last 92 rows, and dk, dv of positions 8100.. (only the last 92 rows can
    select them, so the subset's sums for them are complete)."""
    import torch
    cfg = synth.CONFIGS["prefill8k"]
    inp = synth.host_inputs(cfg, seed=66)
    idx = synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K, seed=66)
    r = np.random.default_rng(67)
    dy = synth.bf16_bits(r.standard_normal((cfg.B, cfg.Tq, cfg.Hq, cfg.d), dtype=np.float32))
    log("bwd prefill8k sampled: B=1 Tq=Tk=8192 Hq=32 Hkv=4 d=128 K=2048")
    d = to_device(inp)
    res = lci.sparse_attn_bwd(d["q"], d["k"], d["v"], dev(idx), d["gate"], inp["scale"],
                              d["kv_len"], dev(dy))
    torch.cuda.synchronize()
    got = {k_: host(res[k_]) for k_ in ("dq", "dk", "dv", "dgate")}
    s0 = 8100
    for rows in (slice(0, 64), slice(s0, cfg.Tq)):
        want = orc.attention_bwd(inp["q"][:, rows], inp["k"], inp["v"], inp["gate"][:, rows],
                                 idx[:, rows], inp["kv_len"], inp["scale"], dy[:, rows])
        tag = f"rows {rows.start}-{rows.stop - 1}"
        _close(got["dq"][:, rows], want["dq"], f"8k {tag} dq")
        _close(got["dgate"][:, rows], want["dgate"], f"8k {tag} dgate")
    _close(got["dk"][:, s0:], want["dk"][:, s0:], f"8k keys {s0}.. dk")
    _close(got["dv"][:, s0:], want["dv"][:, s0:], f"8k keys {s0}.. dv")


def test_sparse_attn_bwd_prefill8k_chunk_seams(lci, orc):
    """dk and dv summed across the row chunks of the tile kernel at the full
    Prefill-8K size: keys 64..127 are selected only by 64 rows spread over
    every chunk (the other rows drop them and pad with -1, still ascending and
    tile-eligible), so the oracle on those 64 rows gives their whole sums."""
    import torch
    cfg = synth.CONFIGS["prefill8k"]
    inp = synth.host_inputs(cfg, seed=70)
    idx = synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K, seed=70)
    lo, hi = 64, 128
    S = np.linspace(128, cfg.Tq - 1, 64).astype(np.int64)
    keep = np.zeros(cfg.Tq, bool)
    keep[S] = True
    for i in np.flatnonzero(~keep):
        row = idx[0, i]
        v = row[(row >= 0) & ((row < lo) | (row >= hi))]
        row[:] = -1
        row[:v.size] = v
    assert all(((idx[0, i] >= lo) & (idx[0, i] < hi)).any() for i in S)
    r = np.random.default_rng(71)
    dy = synth.bf16_bits(r.standard_normal((cfg.B, cfg.Tq, cfg.Hq, cfg.d), dtype=np.float32))
    log("bwd prefill8k chunk seams: keys 64..127 from 64 rows across every chunk")
    d = to_device(inp)
    res = lci.sparse_attn_bwd(d["q"], d["k"], d["v"], dev(idx), d["gate"], inp["scale"],
                              d["kv_len"], dev(dy))
    torch.cuda.synchronize()
    want = orc.attention_bwd(inp["q"][:, S], inp["k"], inp["v"], inp["gate"][:, S],
                             idx[:, S], inp["kv_len"], inp["scale"], dy[:, S])
    _close(host(res["dq"])[:, S], want["dq"], "8k seam rows dq")
    _close(host(res["dk"])[:, lo:hi], want["dk"][:, lo:hi], f"8k keys {lo}..{hi - 1} dk")
    _close(host(res["dv"])[:, lo:hi], want["dv"][:, lo:hi], f"8k keys {lo}..{hi - 1} dv")


def _random_set_rows(cfg, inp, sets, seed):
    """Random valid index rows per set: int32 [B, Tq, sets, K]."""
    return np.stack([synth.index_rows(inp["q_offset"], inp["kv_len"], cfg.Tq, cfg.K,
                                      seed=seed + j) for j in range(sets)], axis=2)


def _sets_case(orc, name):
    """(config, inputs, index rows [B, Tq, sets, K], gated) of the set cases."""
    if name == "per_kv_head_mix":
        cfg = MED.replace(Tq=200, Tk=200, K=48)
        inp = synth.host_inputs(cfg, seed=80)
        inp["mix"] = synth.host_mix(cfg, seed=80)
        idx = orc.layer(inp, cfg.K, sets=cfg.Hkv)["idx"].reshape(cfg.B, cfg.Tq, cfg.Hkv, cfg.K)
        return cfg, inp, idx, True
    if name == "per_query_head_two_sequences":
        cfg = MED.replace(B=2, Hq=8, Hkv=2, H_I=8, Tq=90, Tk=260, K=40)
        inp = synth.host_inputs(cfg, seed=81)
        inp["q_offset"] = np.array([170, 0], np.int32)
        inp["kv_len"] = np.array([260, 70], np.int32)   # sequence 1: rows past 69 are empty
        idx = orc.layer(inp, cfg.K, sets=cfg.Hq)["idx"].reshape(cfg.B, cfg.Tq, cfg.Hq, cfg.K)
        return cfg, inp, idx, True
    if name == "sets2_over_kv4_ungated":
        cfg = MED.replace(Tq=160, Tk=160, K=40)
        inp = synth.host_inputs(cfg, seed=82)
        idx = _random_set_rows(cfg, inp, 2, 82)
        return cfg, inp, idx, False
    if name == "per_query_head_splits":
        # one-row sequences with long lists: the forward recompute splits them
        cfg = MED.replace(B=4, Hq=8, Hkv=2, Tq=1, Tk=3000, K=512, n_needles=0, needles="none")
        inp = synth.host_inputs(cfg, seed=83)
        inp["kv_len"] = np.array([3000, 900, 1, 2048], np.int32)
        inp["q_offset"] = inp["kv_len"] - 1
        idx = _random_set_rows(cfg, inp, cfg.Hq, 83)
        return cfg, inp, idx, True
    if name == "per_query_head_g16_d64":
        cfg = TINY.replace(Hq=16, Hkv=1, d=64, Tq=70, Tk=150, K=30)
        inp = synth.host_inputs(cfg, seed=84)
        inp["q_offset"] = np.array([80], np.int32)
        idx = _random_set_rows(cfg, inp, cfg.Hq, 84)
        return cfg, inp, idx, True
    raise KeyError(name)


SET_CASES = ["per_kv_head_mix", "per_query_head_two_sequences", "sets2_over_kv4_ungated",
             "per_query_head_splits", "per_query_head_g16_d64"]


@pytest.mark.parametrize("name", SET_CASES)
def test_sparse_attn_bwd_sets(lci, orc, name):
    """Gradients over index sets (query head h reads set h // (Hq // sets)):
    every row takes the gather kernels, dk and dv walk each set's list of rows;
    against the oracle's chain rule, and bit-identical across two calls."""
    import torch
    cfg, inp, idx, gated = _sets_case(orc, name)
    sets = idx.shape[2]
    r = np.random.default_rng(85)
    dy = synth.bf16_bits(r.standard_normal((cfg.B, cfg.Tq, cfg.Hq, cfg.d), dtype=np.float32))
    gate = inp["gate"] if gated else None
    mix = inp.get("mix") if gated else None
    log(f"bwd sets {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hq={cfg.Hq} Hkv={cfg.Hkv} "
        f"d={cfg.d} K={cfg.K} sets={sets} gated={gated}")
    d = to_device(inp)
    idx4 = np.ascontiguousarray(idx.transpose(0, 2, 1, 3))   # [B, sets, Tq, K]
    args = (d["q"], d["k"], d["v"], dev(idx4), dev(gate), inp["scale"], d["kv_len"], dev(dy))
    res = lci.sparse_attn_bwd(*args, q_offset=d["q_offset"], mix=dev(mix))
    torch.cuda.synchronize()
    want = orc.attention_bwd(inp["q"], inp["k"], inp["v"], gate, idx, inp["kv_len"],
                             inp["scale"], dy, mix=mix)
    for key in ("dq", "dk", "dv", "dgate", "dmix"):
        if want[key] is None:
            assert res[key] is None
            continue
        _close(host(res[key]), want[key], f"{name} {key}")
    res2 = lci.sparse_attn_bwd(*args, q_offset=d["q_offset"], mix=dev(mix))
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert torch.equal(res[key], res2[key]), key
