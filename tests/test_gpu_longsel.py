"""GPU parity of the long-prefill selection (scores never written to memory):
fused prefills with histories longer than 8192 positions and at least 8192
query rows, every row against the oracle: index rows bit-exact, outputs within
the bf16 tolerance, lse within 1e-4.

The cases reach every way a row can end: rows that keep every position
(p < K), rows that list every position (p < the list capacity), sampled rows
finished from their list, and rows the list cannot finish (every score equal:
the list overflows; a planted pattern that makes the sampled threshold too
high: the list holds fewer than K) redone from their whole score row. Also:
ties at the K-th score, ragged and invalid rows, continuation rows, index sets
per key/value head and per query head, both indexer widths, K = 64 and K = 4096, one indexer
head, and the gate mix."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, host, log, to_device

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4

# small attention heads keep the oracle's attention cheap at 8192+ rows
BASE = synth.CONFIGS["prefill8k"].replace(Hq=2, Hkv=1, d=64, Tq=8192, Tk=12000, K=2048,
                                          needles="none", n_needles=0)


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def plant_stride_pattern(inp, stride=8):
    """Every position that is a multiple of `stride` scores far above the rest
    (indexer head 0 of every query is all ones, those key rows all eights):
    every sampled position is one of them, and there are fewer of them than K."""
    inp["q_idx"][:, :, 0, :] = 1
    inp["k_idx"][:, ::stride, :] = 8
    return inp


CASES = {
    # rows at positions 3807..11998: listed (p < cap) and sampled rows
    "base": (BASE, dict(q_offset=[3807]), None),
    # two sequences: rows from position 0 (every position kept, then listed,
    # then sampled) and continuation rows whose tail is past the history
    "ragged_two_seqs": (BASE.replace(B=2, Tq=4096, Tk=16384),
                        dict(q_offset=[0, 12000], kv_len=[16384, 16000]), None),
    # scores over a few values: many ties at the K-th score
    "heavy_ties": (BASE, dict(q_offset=[3807], q_range=1), None),
    # every score equal: every long row's list overflows (whole-row redo)
    "all_equal": (BASE.replace(Tk=9000), dict(q_offset=[807], q_range=0), None),
    # the sample sees only the planted high scores: lists shorter than K (redo)
    "sample_too_high": (BASE, dict(q_offset=[3807]), plant_stride_pattern),
    "sets_per_kv_head": (BASE.replace(Hq=4, Hkv=2, H_I=8), dict(q_offset=[3807], sets=2), None),
    # one set per query head (two query heads per key/value head, one indexer head each)
    "sets_per_query_head": (BASE.replace(Hq=4, Hkv=2, H_I=4), dict(q_offset=[3807], sets=4),
                            None),
    "h4_d128": (BASE.replace(H_I=4, d_I=128), dict(q_offset=[3807]), None),
    "k64": (BASE.replace(K=64), dict(q_offset=[3807]), None),
    "k4096": (BASE.replace(K=4096, Tk=20000), dict(q_offset=[11807]), None),
    "h1_mix": (BASE.replace(H_I=1), dict(q_offset=[3807], mix=True), None),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(CASES))
def test_long_prefill_select(lci, orc, name):
    import torch
    cfg, kw, plant = CASES[name]
    kw = dict(kw)
    sets = kw.pop("sets", 1)
    with_mix = kw.pop("mix", False)
    if "q_range" in kw:
        cfg = cfg.replace(q_range=kw.pop("q_range"))
    inp = synth.host_inputs(cfg, seed=71)
    if "q_offset" in kw:
        inp["q_offset"] = np.asarray(kw["q_offset"], np.int32)
    if "kv_len" in kw:
        inp["kv_len"] = np.asarray(kw["kv_len"], np.int32)
    if plant is not None:
        inp = plant(inp)
    if with_mix:
        inp["mix"] = synth.host_mix(cfg, seed=71)
    log(f"long select {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={cfg.K} H_I={cfg.H_I} "
        f"d_I={cfg.d_I} sets={sets}")
    d = to_device(inp)
    geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                         Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I, sets=sets)
    lci.kernel_timing(True)
    out, idx, lse = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                    d["gate"], inp["scale"], d["q_offset"], d["kv_len"], cfg.K,
                                    want_idx=True, want_lse=True, mix=d.get("mix"), sets=sets)
    torch.cuda.synchronize()
    _, n_scan = lci.kernel_timing_read("sel_scan")
    _, n_score = lci.kernel_timing_read("idx_score")
    lci.kernel_timing(False)
    # the call took the long-prefill selection, not the materialised scores
    assert n_scan == sets and n_score == 0, (n_scan, n_score)
    assert lci.workspace_bytes(lci.ENTRY_PREFILL, geom) > 0
    res = orc.layer(inp, cfg.K, sets=sets)
    nr = cfg.B * cfg.Tq
    if sets == 1:
        got_idx = host(idx).reshape(nr, -1)
    else:
        got_idx = host(idx).reshape(cfg.B, sets, cfg.Tq, -1).transpose(0, 2, 1, 3).reshape(
            nr, sets, -1)
    want_idx = res["idx"].reshape(got_idx.shape)
    bad = np.flatnonzero((got_idx != want_idx).reshape(nr, -1).any(1))
    assert bad.size == 0, (name, f"{bad.size} rows differ, first {bad[0]}",
                           got_idx.reshape(nr, -1)[bad[0]][:12],
                           want_idx.reshape(nr, -1)[bad[0]][:12])
    assert_attn_close(host(out).reshape(nr, cfg.Hq, cfg.d), res["out"], f"long select {name}")
    lse = host(lse).reshape(nr, cfg.Hq)
    fin = np.isfinite(res["lse"])
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - res["lse"][fin]).max() < LSE_TOL
    log(f"long select {name}: {nr} rows bit-exact")
