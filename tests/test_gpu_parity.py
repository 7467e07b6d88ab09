"""GPU parity: every entry point of the HIP library against the CPU oracle on the
same seeded inputs. Indexer scores and Top-K index sets must match bit for bit;
attention outputs within max-abs 2e-2 and relative L2 5e-3 (bf16).

Small cases cover every row; they span several tiles of every kernel and end in
ragged tails. Edge cases: ragged sequences, continuation rows (q_offset > 0),
invalid rows, K = 1, K larger than the history, heavy ties, all-zero scores,
negative per-row weights, a null gate, every supported indexer shape, and the
gate mixing the output with another branch's (tile, gather and split-K
epilogues, empty and invalid rows)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, dev, host, log, to_device

pytestmark = pytest.mark.gpu

I32_MIN = np.iinfo(np.int32).min
# lse is fp32 arithmetic on exact bf16 products: a few fp32 ulps of |lse| <= ~20,
# plus v_exp_f32/v_log_f32 (about 1 ulp each) summed over <= 4096 terms
LSE_TOL = 1e-4


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def make(cfg, seed=0, q_offset=None, kv_len=None, w=None, q_range=None):
    if q_range is not None:
        cfg = cfg.replace(q_range=q_range)
    inp = synth.host_inputs(cfg, seed=seed)
    if q_offset is not None:
        inp["q_offset"] = np.asarray(q_offset, np.int32)
    if kv_len is not None:
        inp["kv_len"] = np.asarray(kv_len, np.int32)
    if w is not None:
        inp["w"] = np.asarray(w, np.int8)
    return inp


TINY = synth.CONFIGS["tiny"]
MED = synth.CONFIGS["prefill8k"].replace(Tq=640, Tk=640, K=128, n_needles=8)

SCORE_CASES = {
    "tiny": (TINY, {}),
    "h8d64_ragged": (MED.replace(B=2, Tq=200, Tk=700),
                     dict(q_offset=[0, 450], kv_len=[700, 640])),
    "h1d32": (TINY.replace(H_I=1, d_I=32, Tq=97, Tk=300), dict(q_offset=[180])),
    "h4d128": (TINY.replace(H_I=4, d_I=128, Tq=130, Tk=130), {}),
    "h16d64_rowweights": (TINY.replace(H_I=16, d_I=64, B=2, Tq=70, Tk=333),
                          dict(q_offset=[0, 263], kv_len=[333, 333])),
    "decode_shape": (MED.replace(B=3, Tq=1, Tk=5000, decode=True), {}),
    # int32 extremes: every int8 input at -128 and every weight at 127, at the
    # largest indexer size (H_I*d_I = 1024: S = 16*127*64*128^2 = 2 130 706 432)
    # and on the shared-weight MFMA layout (H_I*d_I = 512, 64+ rows)
    "extreme_h16d64": (TINY.replace(H_I=16, d_I=64, Tq=64, Tk=200), {}),
    "extreme_h8d128": (TINY.replace(H_I=8, d_I=128, Tq=40, Tk=100), {}),
    "extreme_q16": (MED.replace(Tq=128, Tk=300), {}),
}


@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_idx_score_bit_exact(lci, orc, name):
    import torch
    cfg, kw = SCORE_CASES[name]
    inp = make(cfg, seed=1, **kw)
    if name == "h16d64_rowweights":
        r = np.random.default_rng(5)
        inp["w"] = r.integers(-128, 128, size=(cfg.B, cfg.Tq, cfg.H_I)).astype(np.int8)
        inp["q_idx"] = r.integers(-128, 128, size=inp["q_idx"].shape).astype(np.int8)
        inp["k_idx"] = r.integers(-128, 128, size=inp["k_idx"].shape).astype(np.int8)
    if name.startswith("extreme"):
        inp["q_idx"][:] = -128
        inp["k_idx"][:] = -128
        inp["w"] = np.full(cfg.H_I, 127, np.int8)
    log(f"idx_score {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} H_I={cfg.H_I} d_I={cfg.d_I}")
    d = to_device(inp)
    sentinel = torch.full((cfg.B, cfg.Tq, cfg.Tk), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    got = host(lci.idx_score(d["q_idx"], d["k_idx"], d["w"], d["q_offset"], d["kv_len"],
                             scores=sentinel)).reshape(cfg.B * cfg.Tq, cfg.Tk)
    torch.cuda.synchronize()
    ref = orc.scores(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"])
    for r in range(cfg.B * cfg.Tq):
        b, i = divmod(r, cfg.Tq)
        p = int(inp["q_offset"][b]) + i
        if p < inp["kv_len"][b]:
            assert (got[r, :p + 1] == ref[r, :p + 1]).all(), (name, b, i)
            assert (got[r, p + 1:] == 0x5A5A5A5A).all(), (name, b, i, "wrote beyond p")
        else:
            assert (got[r] == 0x5A5A5A5A).all(), (name, b, i, "wrote an invalid row")


TOPK_CASES = {
    "tiny": (TINY, 32, {}),
    "k1": (TINY.replace(Tq=64, Tk=64), 1, {}),
    "k_over_t": (TINY.replace(Tq=50, Tk=50), 77, {}),
    "ties": (MED.replace(Tq=300, Tk=300), 64, dict(q_range=1)),
    "all_zero": (TINY.replace(Tq=80, Tk=80), 16, dict(q_range=0)),
    "ragged_invalid": (MED.replace(B=3, Tq=40, Tk=900), 100,
                       dict(q_offset=[0, 850, 400], kv_len=[900, 870, 420])),
    "long_rows": (MED.replace(B=2, Tq=1, Tk=40000, decode=True), 2048, {}),
    # one-wave kernel at its limit: rows of 8184..8191 positions, row starts not
    # 16-byte aligned (Tk % 4 == 3), a partial last chunk
    "wave_unaligned": (MED.replace(Tq=8, Tk=8191), 2048, dict(q_offset=[8183])),
    # rows of exactly 8192 positions (every chunk full) and a few shorter ones
    "wave_full": (MED.replace(Tq=12, Tk=8192), 3000, dict(q_offset=[8180])),
}


@pytest.mark.parametrize("name", list(TOPK_CASES))
def test_topk_bit_exact(lci, orc, name):
    cfg, K, kw = TOPK_CASES[name]
    inp = make(cfg.replace(K=K), seed=2, **kw)
    log(f"topk {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={K}")
    S = orc.scores(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"])
    n = np.array([int(inp["q_offset"][b]) + i + 1 if int(inp["q_offset"][b]) + i < inp["kv_len"][b]
                  else 0 for b in range(cfg.B) for i in range(cfg.Tq)])
    want_idx, want_sel = orc.topk(S, n, K)
    d = to_device(inp)
    Sd = dev(S.reshape(cfg.B, cfg.Tq, cfg.Tk))
    idx, sel = lci.topk_select(Sd, K, d["q_offset"], d["kv_len"], want_scores=True)
    idx = host(idx).reshape(-1, K)
    sel = host(sel).reshape(-1, K)
    bad = np.flatnonzero((idx != want_idx).any(1))
    assert len(bad) == 0, (name, bad[:5], idx[bad[0]][:16], want_idx[bad[0]][:16])
    assert (sel == want_sel).all()


ATTN_CASES = {
    "tiny": (TINY, 32, True),
    "gqa8_d128": (MED.replace(Tq=300, Tk=300), 96, True),
    "ungated": (MED.replace(Tq=100, Tk=400), 64, False),
    "d64_g2": (TINY.replace(Hq=4, Hkv=2, Tq=77, Tk=200), 40, True),
    "h16_kv1": (TINY.replace(Hq=16, Hkv=1, Tq=40, Tk=128), 24, True),
    "decode_split": (MED.replace(B=3, Tq=1, Tk=9000, decode=True), 2048, True),
}


@pytest.mark.parametrize("order", ["sorted", "scrambled"])
@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_sparse_attn_on_oracle_idx(lci, orc, name, order):
    """Sorted index rows (the Top-K output form) may take the dense-tile path;
    scrambled rows must take the gather path; both must match the oracle."""
    import torch
    cfg, K, gated = ATTN_CASES[name]
    inp = make(cfg.replace(K=K), seed=3)
    log(f"sparse_attn {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hq={cfg.Hq} Hkv={cfg.Hkv} "
        f"d={cfg.d} K={K}")
    res = orc.layer(inp, K, gated=gated)
    idx = res["idx"]
    if order == "scrambled":
        r = np.random.default_rng(0)
        idx = np.stack([r.permutation(row) for row in idx]).astype(np.int32)
    d = to_device(inp)
    out, lse = lci.sparse_attn_fwd(d["q"], d["k"], d["v"], dev(idx.reshape(cfg.B, cfg.Tq, K)),
                                   d["gate"] if gated else None, inp["scale"], d["kv_len"],
                                   want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(host(out), res["out"].reshape(cfg.B, cfg.Tq, cfg.Hq, cfg.d), name)
    lse = host(lse).reshape(-1, cfg.Hq)
    assert np.abs(lse - res["lse"]).max() < LSE_TOL


def _fused_check(lci, orc, cfg, inp, K, rows=None, entry="prefill"):
    import torch
    d = to_device(inp)
    fn = lci.prefill_fwd if entry == "prefill" else lci.decode_fwd
    out, idx, lse = fn(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                       inp["scale"], d["q_offset"], d["kv_len"], K, want_idx=True, want_lse=True,
                       mix=d.get("mix"))
    torch.cuda.synchronize()
    res = orc.layer(inp, K, rows=rows)
    out = host(out).reshape(cfg.B * cfg.Tq, cfg.Hq, cfg.d)
    idx = host(idx).reshape(cfg.B * cfg.Tq, K)
    lse = host(lse).reshape(-1, cfg.Hq)
    sel = np.arange(cfg.B * cfg.Tq) if rows is None else np.array([b * cfg.Tq + i for b, i in rows])
    assert (idx[sel] == res["idx"]).all()
    assert_attn_close(out[sel], res["out"], f"{entry} B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk}")
    fin = np.isfinite(res["lse"])
    assert (np.isfinite(lse[sel]) == fin).all()
    assert np.abs(lse[sel][fin] - res["lse"][fin]).max() < LSE_TOL


def test_tiny_fp32_source(lci, orc):
    """The Tiny configuration draws Q, K, V and the gate logits in fp32. The
    library computes from their bf16 roundings (to nearest even): parity is
    checked against the oracle on those bf16 inputs, and the same output is also
    reported against the oracle on the fp32 sources (the rounding of the inputs
    shows there, at about 3e-3 relative L2), within the same bounds."""
    import torch
    from gpu_util import attn_errors
    cfg = TINY
    inp = synth.host_inputs(cfg, seed=0)
    assert "q_f32" in inp
    d = to_device(inp)
    out, idx = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                               inp["scale"], d["q_offset"], d["kv_len"], cfg.K, want_idx=True)
    torch.cuda.synchronize()
    res = orc.layer(inp, cfg.K)
    out = host(out).reshape(cfg.Tq, cfg.Hq, cfg.d)
    assert (host(idx).reshape(cfg.Tq, cfg.K) == res["idx"]).all()
    ref32, _ = orc.attention_f32(inp["q_f32"], inp["k_f32"], inp["v_f32"], inp["gate_f32"],
                                 res["idx"], inp["kv_len"], inp["scale"])
    a16 = attn_errors(out, res["out"])
    a32 = attn_errors(out, ref32)
    o16 = np.abs(res["out"] - ref32)
    log(f"tiny: GPU vs bf16-input oracle max_abs={a16[0]:.3e} rel_l2={a16[1]:.3e}; "
        f"GPU vs fp32-source oracle max_abs={a32[0]:.3e} rel_l2={a32[1]:.3e}; "
        f"bf16-input oracle vs fp32-source oracle max_abs={o16.max():.3e} "
        f"rel_l2={np.linalg.norm(o16) / np.linalg.norm(ref32):.3e}")
    assert_attn_close(out, res["out"], "tiny fp32 source, bf16 parity")
    assert_attn_close(out, ref32, "tiny fp32 source, against the fp32 sources")


FUSED_CASES = {
    "tiny": (TINY, {}),
    "med_needles": (MED, {}),
    "ragged_continuation": (MED.replace(B=2, Tq=96, Tk=700, K=200),
                            dict(q_offset=[604, 300], kv_len=[700, 396])),
    "invalid_rows": (TINY.replace(B=2, Tq=20, Tk=100, K=8), dict(q_offset=[90, 0],
                                                                  kv_len=[100, 10])),
    # one split: the Top-K kernel writes the tile path's flags and masks; rows
    # p < 64 keep everything, 64 <= p < 1024 take masked tiles (histories of at
    # most 16 K), the rest gather
    "tile_masks_from_topk": (MED.replace(Tq=2048, Tk=2048, K=64), {}),
    # histories no longer than 4K: every row, the empty ones included, is written
    # by the tile kernel and the gather kernel is not launched
    # the largest K, on rows that keep 68-72% of their history (tile path)
    "k_max": (MED.replace(Tq=300, Tk=6000, K=4096), dict(q_offset=[5700])),
    "tile_only_with_empty_rows": (MED.replace(B=2, Tq=64, Tk=128, K=32),
                                  dict(q_offset=[64, 0], kv_len=[100, 50])),
}


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_prefill_fused(lci, orc, name):
    cfg, kw = FUSED_CASES[name]
    inp = make(cfg, seed=4, **kw)
    log(f"prefill {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={cfg.K}")
    _fused_check(lci, orc, cfg, inp, cfg.K)


def test_decode_fused(lci, orc):
    cfg = MED.replace(B=5, Tq=1, Tk=20000, decode=True, K=2048, needles="decode", n_needles=12)
    inp = make(cfg, seed=6, kv_len=[20000, 19999, 4000, 2048, 1500],
               q_offset=[19999, 19998, 3999, 2047, 1499])
    log("decode B=5 ragged")
    _fused_check(lci, orc, cfg, inp, cfg.K, entry="decode")


DECODE_EDGE = {
    # every score equal: one histogram bin holds the whole history (capacity fallback)
    "all_equal": (dict(q_range=0), 12000),
    # scores in a narrow range: many ties inside the threshold bin
    "heavy_ties": (dict(q_range=1), 30000),
    # another indexer shape, K larger than some histories
    "h2d32": (dict(H_I=2, d_I=32, K=300), 9000),
    # the largest K
    "k_max": (dict(K=4096), 20000),
    # a long history (66 chunks, a ragged last chunk)
    "long_history": (dict(), 270000),
    # the same with every score equal: the whole-row fallback over a long row
    "long_history_all_equal": (dict(q_range=0), 270000),
}


@pytest.mark.parametrize("name", list(DECODE_EDGE))
def test_decode_fused_edges(lci, orc, name):
    kw, L = DECODE_EDGE[name]
    q_range = kw.pop("q_range", None)
    cfg = MED.replace(B=3, Tq=1, Tk=L, decode=True, K=kw.pop("K", 2048), needles="none", **kw)
    inp = make(cfg, seed=8, q_range=q_range, kv_len=[L, L - 77, 250],
               q_offset=[L - 1, L - 78, 249])
    log(f"decode edge {name}: L={L} K={cfg.K} H_I={cfg.H_I} d_I={cfg.d_I}")
    _fused_check(lci, orc, cfg, inp, cfg.K, entry="decode")


def test_decode_sample_too_high(lci, orc):
    """Every 32nd position (each sampled one) scores far above the rest and
    there are fewer of them than K: the threshold from the sample sits above
    the K-th score, the candidate list falls short of K, and the row is
    selected again from its whole score row. One sequence stays on the list
    path (unplanted) beside it, one takes every position."""
    L = 40000
    cfg = MED.replace(B=3, Tq=1, Tk=L, decode=True, K=2048, needles="none")
    inp = make(cfg, seed=9, kv_len=[L, L - 5, 3000], q_offset=[L - 1, L - 6, 2999],
               w=[1] * cfg.H_I)
    inp["q_idx"][0] = 1
    inp["k_idx"][0, ::32, :] = 8
    log(f"decode sample too high: L={L} K={cfg.K} (1250 planted positions < K)")
    _fused_check(lci, orc, cfg, inp, cfg.K, entry="decode")


def test_deterministic(lci):
    import torch
    cfg = MED.replace(Tq=256, Tk=256, K=64)
    d = to_device(make(cfg, seed=7))
    outs = []
    for _ in range(2):
        o, i = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"],
                               cfg.scale, d["q_offset"], d["kv_len"], cfg.K, want_idx=True)
        outs.append((host(o).copy(), host(i).copy()))
    torch.cuda.synchronize()
    assert (outs[0][0] == outs[1][0]).all() and (outs[0][1] == outs[1][1]).all()


# ---- the gate mixing the sparse output o with another branch's output x:
# s*o + (1-s)*x, s = sigmoid(gate); rows without entries give (1-s)*x

MIX_ATTN_CASES = {
    # sorted rows: dense-tile epilogue; scrambled rows: gather epilogue
    "tile": (MED.replace(Tq=300, Tk=300), 96, "sorted"),
    "gather": (MED.replace(Tq=300, Tk=300), 96, "scrambled"),
    "gather_d64": (TINY.replace(Hq=4, Hkv=2, Tq=77, Tk=200), 40, "scrambled"),
    # few long rows: split-K, the combine kernel applies the gate
    "split": (MED.replace(B=3, Tq=1, Tk=9000, decode=True), 2048, "sorted"),
}


@pytest.mark.parametrize("name", list(MIX_ATTN_CASES))
def test_sparse_attn_mix(lci, orc, name):
    import torch
    cfg, K, order = MIX_ATTN_CASES[name]
    cfg = cfg.replace(K=K)
    inp = make(cfg, seed=9)
    inp["mix"] = synth.host_mix(cfg, seed=9)
    log(f"sparse_attn mix {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} Hq={cfg.Hq} K={K} {order}")
    res = orc.layer(inp, K)
    idx = res["idx"]
    if order == "scrambled":
        r = np.random.default_rng(1)
        idx = np.stack([r.permutation(row) for row in idx]).astype(np.int32)
    d = to_device(inp)
    out, lse = lci.sparse_attn_fwd(d["q"], d["k"], d["v"], dev(idx.reshape(cfg.B, cfg.Tq, K)),
                                   d["gate"], inp["scale"], d["kv_len"], want_lse=True,
                                   mix=d["mix"])
    torch.cuda.synchronize()
    assert_attn_close(host(out), res["out"].reshape(cfg.B, cfg.Tq, cfg.Hq, cfg.d), name)
    assert np.abs(host(lse).reshape(-1, cfg.Hq) - res["lse"]).max() < LSE_TOL


MIX_FUSED_CASES = {
    # invalid rows (positions past the history) on the gather path
    "invalid_rows": (TINY.replace(B=2, Tq=20, Tk=100, K=8), dict(q_offset=[90, 0],
                                                                  kv_len=[100, 10])),
    # empty rows written by the tile kernel
    "tile_only_with_empty_rows": (MED.replace(B=2, Tq=64, Tk=128, K=32),
                                  dict(q_offset=[64, 0], kv_len=[100, 50])),
    "tile_masks_from_topk": (MED.replace(Tq=2048, Tk=2048, K=256), {}),
}


@pytest.mark.parametrize("name", list(MIX_FUSED_CASES))
def test_prefill_fused_mix(lci, orc, name):
    cfg, kw = MIX_FUSED_CASES[name]
    inp = make(cfg, seed=10, **kw)
    inp["mix"] = synth.host_mix(cfg, seed=10)
    log(f"prefill mix {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={cfg.K}")
    _fused_check(lci, orc, cfg, inp, cfg.K)


def test_decode_fused_mix(lci, orc):
    # sequence 1 is invalid (its position is past its history): its output is (1-s)*x
    cfg = MED.replace(B=3, Tq=1, Tk=20000, decode=True, K=2048, needles="none")
    inp = make(cfg, seed=11, kv_len=[20000, 3000, 5000], q_offset=[19999, 3000, 4999])
    inp["mix"] = synth.host_mix(cfg, seed=11)
    log("decode mix B=3 with an invalid sequence")
    _fused_check(lci, orc, cfg, inp, cfg.K, entry="decode")
