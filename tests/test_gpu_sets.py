"""GPU parity of one index set per key/value head (the per-head index rows of
the pages' pseudocode: "Hybrid Sparse Attention for Long-Context LLMs", Indexer
+ Top-K section). Each set is scored by its group of indexer heads; the index
rows [B, Hkv, Tq, K] must equal the oracle's bit for bit and the attention
outputs must be within the bf16 tolerance."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, dev, host, log, to_device

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4
MED = synth.CONFIGS["prefill8k"].replace(Tq=640, Tk=640, K=128, n_needles=8)
TINY = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def _check(lci, orc, cfg, inp, block, entry, name):
    import torch
    d = to_device(inp)
    fn = lci.prefill_fwd if entry == "prefill" else lci.decode_fwd
    out, idx, lse = fn(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                       inp["scale"], d["q_offset"], d["kv_len"], cfg.K, want_idx=True,
                       want_lse=True, mix=d.get("mix"), block=block, sets=cfg.Hkv)
    torch.cuda.synchronize()
    res = orc.layer(inp, cfg.K, block=block, sets=cfg.Hkv)
    # [B, sets, Tq, KI] -> [B*Tq, sets, KI]
    got = host(idx).transpose(0, 2, 1, 3).reshape(res["idx"].shape)
    assert np.array_equal(got, res["idx"]), name
    assert_attn_close(host(out).reshape(res["out"].shape), res["out"], name)
    lse = host(lse).reshape(-1, cfg.Hq)
    fin = np.isfinite(res["lse"])
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - res["lse"][fin]).max() < LSE_TOL
    return res


PREFILL_CASES = {
    # 4 sets of 2 indexer heads each (the one-weight-row MFMA scorer)
    "h8_sets4": (MED, 1, dict(), False),
    # continuation rows and an invalid row, with the gate mix
    "ragged_mix": (MED.replace(B=2, Tq=96, Tk=700, K=200), 1,
                   dict(q_offset=[604, 300], kv_len=[700, 396]), True),
    # sets with blocks of 16
    "blocks16": (MED.replace(K=8), 16, dict(), False),
    # 2 sets of one indexer head, d = 64 (the per-row scorer)
    "d64_sets2_h1": (TINY.replace(Hq=4, Hkv=2, H_I=2, d_I=32, Tq=77, Tk=200, K=40), 1, dict(),
                     False),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_sets(lci, orc, name):
    cfg, block, kw, mix = PREFILL_CASES[name]
    inp = synth.host_inputs(cfg, seed=40)
    for k_, v_ in kw.items():
        inp[k_] = np.asarray(v_, np.int32)
    if mix:
        inp["mix"] = synth.host_mix(cfg, seed=40)
    log(f"prefill sets {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hkv={cfg.Hkv} H_I={cfg.H_I} "
        f"K={cfg.K} block={block}")
    res = _check(lci, orc, cfg, inp, block, "prefill", name)
    # the sets really differ from one another
    assert not all((res["idx"][:, g] == res["idx"][:, 0]).all() for g in range(cfg.Hkv))


def test_decode_sets(lci, orc):
    L = 20000
    cfg = MED.replace(B=3, Tq=1, Tk=L, decode=True, K=2048, needles="decode", n_needles=6)
    inp = synth.host_inputs(cfg, seed=41)
    inp["kv_len"] = np.array([L, 1500, 900], np.int32)
    inp["q_offset"] = np.array([L - 1, 1499, 900], np.int32)   # sequence 2 is invalid
    log("decode sets: B=3 L=20000 K=2048 sets=4")
    _check(lci, orc, cfg, inp, 1, "decode", "decode sets")


def test_sparse_attn_per_head_rows(lci, orc):
    """lci_sparse_attn_fwd on the oracle's per-head index rows, scrambled (the
    gather kernel reads each wave's own row)."""
    import torch
    cfg = MED.replace(Tq=300, Tk=300, K=96)
    inp = synth.host_inputs(cfg, seed=42)
    res = orc.layer(inp, cfg.K, sets=cfg.Hkv)
    r = np.random.default_rng(2)
    idx = np.stack([[r.permutation(row) for row in rows] for rows in res["idx"]]).astype(np.int32)
    idx4 = idx.reshape(cfg.B, cfg.Tq, cfg.Hkv, cfg.K).transpose(0, 2, 1, 3).copy()
    d = to_device(inp)
    out, lse = lci.sparse_attn_fwd(d["q"], d["k"], d["v"], dev(idx4), d["gate"], inp["scale"],
                                   d["kv_len"], want_lse=True)
    torch.cuda.synchronize()
    log("sparse_attn per-head rows: Tq=300 K=96 sets=4")
    assert_attn_close(host(out).reshape(res["out"].shape), res["out"], "per-head rows")
    assert np.abs(host(lse).reshape(-1, cfg.Hq) - res["lse"]).max() < LSE_TOL
