"""The tile and gather attention kernels at once on two library streams with
split compute-unit masks (lci_attn_overlap): a schedule only, so the results
must be bit-identical to the two kernels one after the other, and equal to the
oracle. Prompts whose rows split between the paths (K = 64: the tile path takes
rows p + 1 <= 1024), with two index sets and the gate mix, caller-given index
rows (the unfused entry builds the tile masks itself), continuation rows
(Tq < Tk: the automatic mode keeps one stream, the forced one splits), and a
captured graph (under capture the call keeps to the caller's stream)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, host, log, to_device

pytestmark = pytest.mark.gpu

BASE = synth.CONFIGS["prefill8k"].replace(B=2, Hq=8, Hkv=2, d=128, Tq=3000, Tk=3000, K=64,
                                          needles="none", n_needles=0)


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    yield m
    m.attn_overlap(m.OVERLAP_AUTO)


def _fused(lci, cfg, inp, d, sets, mode):
    import torch
    lci.attn_overlap(mode)
    forks0 = lci.attn_overlap_forks()
    out, idx, lse = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                    d["gate"], inp["scale"], d["q_offset"], d["kv_len"], cfg.K,
                                    want_idx=True, want_lse=True, mix=d.get("mix"), sets=sets)
    torch.cuda.synchronize()
    return dict(out=host(out), idx=host(idx), lse=host(lse)), lci.attn_overlap_forks() - forks0


CASES = {
    "prompt": (BASE, dict()),
    "prompt_sets2_mix": (BASE.replace(H_I=8), dict(sets=2, mix=True)),
    "continuation": (BASE.replace(Tq=1500), dict(q_offset=[1200, 1500])),
}


@pytest.mark.parametrize("name", list(CASES))
def test_overlap_fused_prefill(lci, orc, name):
    cfg, kw = CASES[name]
    sets = kw.get("sets", 1)
    inp = synth.host_inputs(cfg, seed=120)
    if "q_offset" in kw:
        inp["q_offset"] = np.asarray(kw["q_offset"], np.int32)
    if kw.get("mix"):
        inp["mix"] = synth.host_mix(cfg, seed=120)
    d = to_device(inp)
    log(f"overlap {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={cfg.K} sets={sets}")
    off, n_off = _fused(lci, cfg, inp, d, sets, lci.OVERLAP_OFF)
    on, n_on = _fused(lci, cfg, inp, d, sets, lci.OVERLAP_ON)
    auto, n_auto = _fused(lci, cfg, inp, d, sets, lci.OVERLAP_AUTO)
    assert n_off == 0 and n_on == 1, (n_off, n_on)
    log(f"overlap {name}: forced split forked, automatic mode forked {n_auto}")
    for key in ("out", "idx", "lse"):
        assert np.array_equal(off[key], on[key]), key
        assert np.array_equal(off[key], auto[key]), key
    res = orc.layer(inp, cfg.K, sets=sets)
    nr = cfg.B * cfg.Tq
    if sets == 1:
        got_idx = off["idx"].reshape(nr, -1)
    else:
        got_idx = off["idx"].reshape(cfg.B, sets, cfg.Tq, -1).transpose(0, 2, 1, 3).reshape(nr, sets, -1)
    assert np.array_equal(got_idx, res["idx"].reshape(got_idx.shape))
    assert_attn_close(off["out"].reshape(nr, cfg.Hq, cfg.d), res["out"], f"overlap {name}")


def test_overlap_unfused_caller_rows(lci, orc):
    """lci_sparse_attn_fwd on caller-given index rows (the oracle's): the split
    builds the tile masks and done bytes on the caller's stream before it
    forks."""
    import torch
    cfg = BASE
    inp = synth.host_inputs(cfg, seed=121)
    res = orc.layer(inp, cfg.K)
    d = to_device(inp)
    didx = torch.from_numpy(np.ascontiguousarray(res["idx"].reshape(cfg.B, cfg.Tq, cfg.K))).cuda()
    outs = []
    for mode in (lci.OVERLAP_OFF, lci.OVERLAP_ON):
        lci.attn_overlap(mode)
        forks0 = lci.attn_overlap_forks()
        out, lse = lci.sparse_attn_fwd(d["q"], d["k"], d["v"], didx, d["gate"], inp["scale"],
                                       d["kv_len"], want_lse=True)
        torch.cuda.synchronize()
        assert lci.attn_overlap_forks() - forks0 == (1 if mode == lci.OVERLAP_ON else 0)
        outs.append((host(out), host(lse)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert_attn_close(outs[1][0].reshape(cfg.B * cfg.Tq, cfg.Hq, cfg.d), res["out"],
                      "overlap unfused")


def test_overlap_graph_capture_keeps_one_stream(lci):
    """A prefill captured into a graph with the split forced runs on the
    captured stream alone; replays (with eager work between them) equal the
    eager result."""
    import torch
    cfg = BASE.replace(B=1)
    inp = synth.host_inputs(cfg, seed=122)
    d = to_device(inp)
    geom = lci.make_geom(cfg.B, cfg.Tq, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                         Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I)
    ws = torch.empty(lci.workspace_bytes(lci.ENTRY_PREFILL, geom), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    lci.attn_overlap(lci.OVERLAP_ON)

    def step():
        lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                        inp["scale"], d["q_offset"], d["kv_len"], cfg.K, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = host(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    forks0 = lci.attn_overlap_forks()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    assert lci.attn_overlap_forks() == forks0
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), eager)
