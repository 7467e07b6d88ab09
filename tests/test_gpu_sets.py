"""GPU parity of index sets (the per-head index rows of the pages' pseudocode:
"Hybrid Sparse Attention for Long-Context LLMs", Indexer + Top-K section; "How
Fine-Grained Sparse Attention Reshapes ...", runtime section). Query head h
attends over set h // (Hq // sets): one set per key/value head (sets = Hkv),
one per query head (sets = Hq), or a set spanning several key/value heads. Each
set is scored by its group of indexer heads; the index rows [B, sets, Tq, K]
must equal the oracle's bit for bit and the attention outputs must be within
the bf16 tolerance."""
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


def _check(lci, orc, cfg, inp, block, entry, name, sets=None):
    import torch
    sets = cfg.Hkv if sets is None else sets
    d = to_device(inp)
    fn = lci.prefill_fwd if entry == "prefill" else lci.decode_fwd
    out, idx, lse = fn(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                       inp["scale"], d["q_offset"], d["kv_len"], cfg.K, want_idx=True,
                       want_lse=True, mix=d.get("mix"), block=block, sets=sets)
    torch.cuda.synchronize()
    res = orc.layer(inp, cfg.K, block=block, sets=sets)
    # [B, sets, Tq, KI] -> [B*Tq, sets, KI]
    got = host(idx).transpose(0, 2, 1, 3).reshape(res["idx"].shape)
    assert np.array_equal(got, res["idx"]), name
    assert_attn_close(host(out).reshape(res["out"].shape), res["out"], name)
    lse = host(lse).reshape(-1, cfg.Hq)
    fin = np.isfinite(res["lse"])
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - res["lse"][fin]).max() < LSE_TOL
    return res


# per-query-head sets: 8 query heads on 2 key/value heads, one indexer head each
PQH = MED.replace(Hq=8, Hkv=2, H_I=8)

PREFILL_CASES = {
    # name: (config, block, overrides, mix, sets (None: Hkv))
    # 4 sets of 2 indexer heads each (the one-weight-row MFMA scorer)
    "h8_sets4": (MED, 1, dict(), False, None),
    # continuation rows and an invalid row, with the gate mix
    "ragged_mix": (MED.replace(B=2, Tq=96, Tk=700, K=200), 1,
                   dict(q_offset=[604, 300], kv_len=[700, 396]), True, None),
    # sets with blocks of 16
    "blocks16": (MED.replace(K=8), 16, dict(), False, None),
    # 2 sets of one indexer head, d = 64 (the per-row scorer)
    "d64_sets2_h1": (TINY.replace(Hq=4, Hkv=2, H_I=2, d_I=32, Tq=77, Tk=200, K=40), 1, dict(),
                     False, None),
    # one set per query head; K = 24 puts rows past position 383 on the gather
    # path, the rest on the tile path (each tile workgroup spans 4 sets)
    "per_query_head": (PQH.replace(K=24), 1, dict(), False, 8),
    # one set per query head, 16 heads on one key/value head: two groups of 8
    # waves per gathered row, 16 sets per tile workgroup; d = 64
    "per_query_head_h16": (TINY.replace(Hq=16, Hkv=1, H_I=16, d_I=32, Tq=200, Tk=200, K=10), 1,
                           dict(), False, 16),
    # one set per query head with continuation rows, an invalid row and the mix
    "per_query_head_ragged_mix": (PQH.replace(B=2, Tq=96, Tk=700, K=20), 1,
                                  dict(q_offset=[604, 300], kv_len=[700, 396]), True, 8),
    # one set per query head, blocks of 16
    "per_query_head_blocks16": (PQH.replace(K=4), 16, dict(), False, 8),
    # two sets over four key/value heads (each set spans two of them)
    "sets2_over_kv4": (MED.replace(K=24), 1, dict(), False, 2),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_sets(lci, orc, name):
    cfg, block, kw, mix, sets = PREFILL_CASES[name]
    sets = cfg.Hkv if sets is None else sets
    inp = synth.host_inputs(cfg, seed=40)
    for k_, v_ in kw.items():
        inp[k_] = np.asarray(v_, np.int32)
    if mix:
        inp["mix"] = synth.host_mix(cfg, seed=40)
    log(f"prefill sets {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hq={cfg.Hq} Hkv={cfg.Hkv} "
        f"H_I={cfg.H_I} K={cfg.K} block={block} sets={sets}")
    res = _check(lci, orc, cfg, inp, block, "prefill", name, sets)
    # the sets really differ from one another
    assert not all((res["idx"][:, g] == res["idx"][:, 0]).all() for g in range(sets))


@pytest.mark.parametrize("per_query_head", [False, True], ids=["per_kv_head", "per_query_head"])
def test_decode_sets(lci, orc, per_query_head):
    L = 20000
    base = PQH if per_query_head else MED
    cfg = base.replace(B=3, Tq=1, Tk=L, decode=True, K=2048, needles="decode", n_needles=6)
    sets = cfg.Hq if per_query_head else cfg.Hkv
    inp = synth.host_inputs(cfg, seed=41)
    inp["kv_len"] = np.array([L, 1500, 900], np.int32)
    inp["q_offset"] = np.array([L - 1, 1499, 900], np.int32)   # sequence 2 is invalid
    log(f"decode sets: B=3 L=20000 K=2048 Hq={cfg.Hq} Hkv={cfg.Hkv} sets={sets}")
    _check(lci, orc, cfg, inp, 1, "decode", "decode sets", sets)


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


def _random_sets(r, cfg, q_offset, sets, K, order):
    """Index rows [B*Tq, sets, K] of distinct causal positions per set, -1
    padded at the end; ascending (tile path when dense enough) or scrambled
    (gather path)."""
    rows = np.full((cfg.B * cfg.Tq, sets, K), -1, np.int32)
    for row in range(cfg.B * cfg.Tq):
        p = int(q_offset[row // cfg.Tq]) + row % cfg.Tq
        for g in range(sets):
            n = min(p + 1, int(r.integers(1, K + 1)))
            pos = np.sort(r.choice(p + 1, size=n, replace=False)).astype(np.int32)
            if order == "scrambled":
                pos = r.permutation(pos)
            rows[row, g, :n] = pos
    return rows


SPARSE_SETS_CASES = {
    # name: (config, K, sets)
    "per_query_head_g4": (PQH.replace(Tq=300, Tk=300), 96, 8),
    "per_query_head_h16_d64": (TINY.replace(Hq=16, Hkv=1, Tq=120, Tk=120), 40, 16),
    "sets2_over_kv4": (MED.replace(Tq=300, Tk=300), 96, 2),
    # few rows at the end of a long history, long lists: split-K partials and
    # the combine kernel
    "per_query_head_splits": (PQH.replace(B=2, Tq=3, Tk=3000), 1024, 8),
}


@pytest.mark.parametrize("order", ["sorted", "scrambled"])
@pytest.mark.parametrize("name", list(SPARSE_SETS_CASES))
def test_sparse_attn_sets(lci, orc, name, order):
    """lci_sparse_attn_fwd on index rows [B, sets, Tq, K] against the oracle's
    attention over the same rows; sorted rows may take the tile path."""
    import torch
    cfg, K, sets = SPARSE_SETS_CASES[name]
    inp = synth.host_inputs(cfg, seed=43)
    inp["q_offset"] = np.full(cfg.B, cfg.Tk - cfg.Tq, np.int32)
    r = np.random.default_rng(3)
    rows = _random_sets(r, cfg, inp["q_offset"], sets, K, order)
    ref, ref_lse = orc.attention(inp["q"], inp["k"], inp["v"], inp["gate"], rows, inp["kv_len"],
                                 inp["scale"])
    idx4 = rows.reshape(cfg.B, cfg.Tq, sets, K).transpose(0, 2, 1, 3).copy()
    d = to_device(inp)
    log(f"sparse_attn sets {name} {order}: B={cfg.B} Tq={cfg.Tq} Hq={cfg.Hq} Hkv={cfg.Hkv} "
        f"K={K} sets={sets}")
    out, lse = lci.sparse_attn_fwd(d["q"], d["k"], d["v"], dev(idx4), d["gate"], inp["scale"],
                                   d["kv_len"], q_offset=d["q_offset"], want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(host(out).reshape(ref.shape), ref, name)
    lse = host(lse).reshape(-1, cfg.Hq)
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - ref_lse[fin]).max() < LSE_TOL


UNFUSED_CASES = {
    # name: (config, K, block, sets, overrides)
    "per_query_head": (PQH.replace(Tq=200, Tk=260), 32, 1, 8, dict(q_offset=[60])),
    "sets4_h2_ragged": (MED.replace(B=2, Tq=70, Tk=300), 48, 1, 4,
                        dict(q_offset=[230, 0], kv_len=[300, 50])),
    "sets2_blocks8": (MED.replace(Tq=64, Tk=400), 6, 8, 2, dict(q_offset=[336])),
    # rows longer than the one-wave form (workgroup-per-row kernel)
    "sets2_long_rows": (MED.replace(Tq=4, Tk=9000), 512, 1, 2, dict(q_offset=[8996])),
}


@pytest.mark.parametrize("name", list(UNFUSED_CASES))
def test_unfused_score_topk_sets(lci, orc, name):
    """lci_idx_score and lci_topk_select with a set axis: set g's scores are
    the oracle's scores of indexer-head group g (bit-exact, nothing written
    past p), its index rows the oracle's Top-K of them."""
    import torch
    cfg, K, block, sets, kw = UNFUSED_CASES[name]
    inp = synth.host_inputs(cfg, seed=44)
    for k_, v_ in kw.items():
        inp[k_] = np.asarray(v_, np.int32)
    B, Tq, Tk, H_I = cfg.B, cfg.Tq, cfg.Tk, cfg.H_I
    Hg = H_I // sets
    d = to_device(inp)
    log(f"unfused sets {name}: B={B} Tq={Tq} Tk={Tk} H_I={H_I} K={K} block={block} sets={sets}")
    sentinel = torch.full((B, sets, Tq, Tk), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    S = lci.idx_score(d["q_idx"], d["k_idx"], d["w"], d["q_offset"], d["kv_len"],
                      scores=sentinel, sets=sets)
    idx, sel = lci.topk_select(S, K, d["q_offset"], d["kv_len"], want_scores=True, block=block)
    torch.cuda.synchronize()
    S, idx, sel = host(S), host(idx), host(sel)
    assert idx.shape == (B, sets, Tq, K * block) and sel.shape == (B, sets, Tq, K)
    n = np.array([int(inp["q_offset"][b]) + i + 1 if int(inp["q_offset"][b]) + i < inp["kv_len"][b]
                  else 0 for b in range(B) for i in range(Tq)])
    for g in range(sets):
        qg = np.ascontiguousarray(inp["q_idx"][:, :, g * Hg:(g + 1) * Hg])
        wg = np.ascontiguousarray(inp["w"][g * Hg:(g + 1) * Hg])
        ref = orc.scores(qg, inp["k_idx"], wg, inp["q_offset"], inp["kv_len"])
        got = S[:, g].reshape(B * Tq, Tk)
        for row in range(B * Tq):
            assert (got[row, :n[row]] == ref[row, :n[row]]).all(), (name, g, row)
            assert (got[row, n[row]:] == 0x5A5A5A5A).all(), (name, g, row, "wrote past p")
        if block > 1:
            want_idx, _, want_sel = orc.block_topk(ref, n, K, block)
        else:
            want_idx, want_sel = orc.topk(ref, n, K)
        gi = idx[:, g].reshape(B * Tq, -1)
        gs = sel[:, g].reshape(B * Tq, -1)
        bad = np.flatnonzero((gi != want_idx).any(1))
        assert len(bad) == 0, (name, g, bad[:5])
        assert (gs == want_sel).all(), (name, g)
