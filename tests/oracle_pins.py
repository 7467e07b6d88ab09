"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, each
checked against an oracle build (the real one, or a deliberately mutated copy).

Every pin raises AssertionError when the oracle disagrees. None of them retypes
the oracle's general formula: they use hand-worked values (tests/golden/),
closed forms of special cases, library routines (torch's SDPA, numpy matmul,
scipy's expit / logsumexp) and brute-force definitions that differ from the
oracle's own algorithm (the O(n^2) rank definition of Top-K, the masked dense
formulation of attention).
"""
from __future__ import annotations

import json
import os

import numpy as np

from synth import bf16_bits, bf16_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
I32_MIN = np.iinfo(np.int32).min


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf(x):
    return bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------ indexer

def pin_indexer_hand(orc):
    g = _golden("indexer_hand.json")
    S, ovf = orc.score_row(np.array(g["q_idx"]), np.array(g["k_idx"]), np.array(g["w"]), 5)
    assert not ovf
    assert S.tolist() == g["scores"], (S.tolist(), g["scores"])


def pin_indexer_unit_keys(orc):
    """k_s = c_s * e_{j_s} reduces each head's dot to c_s * q[h, j_s]."""
    r = np.random.default_rng(11)
    H_I, d_I = 4, 8
    q = r.integers(-8, 9, size=(H_I, d_I))
    w = np.array([1, 2, 3, 5])
    n = 40
    js = r.integers(0, d_I, size=n)
    cs = r.integers(-5, 6, size=n)
    k = np.zeros((n, d_I), np.int64)
    k[np.arange(n), js] = cs
    S, _ = orc.score_row(q, k, w, n)
    want = [(w * np.maximum(0, cs[s] * q[:, js[s]])).sum() for s in range(n)]
    assert S.tolist() == want


def pin_indexer_zero_query(orc):
    r = np.random.default_rng(12)
    k = r.integers(-8, 9, size=(30, 16))
    S, _ = orc.score_row(np.zeros((3, 16), np.int8), k, np.array([1, -2, 4]), 30)
    assert (S == 0).all()


def pin_indexer_one_hot_weights(orc):
    """With w = e_h the score is ReLU of a textbook dot product (numpy matmul),
    and doubling w doubles the score exactly."""
    r = np.random.default_rng(13)
    H_I, d_I, n = 3, 32, 50
    q = r.integers(-8, 9, size=(H_I, d_I))
    k = r.integers(-8, 9, size=(n, d_I))
    dots = k.astype(np.int64) @ q.T.astype(np.int64)        # [n, H_I]
    for h in range(H_I):
        w = np.zeros(H_I, np.int64)
        w[h] = 1
        S, _ = orc.score_row(q, k, w, n)
        assert S.tolist() == np.maximum(dots[:, h], 0).tolist()
    w = np.array([3, 1, 4])
    S1, _ = orc.score_row(q, k, w, n)
    S2, _ = orc.score_row(q, k, 2 * w, n)
    assert (S2 == 2 * S1.astype(np.int64)).all()
    assert (S1 >= 0).all()


def pin_indexer_head_permutation(orc):
    r = np.random.default_rng(14)
    q = r.integers(-8, 9, size=(8, 16))
    w = r.integers(1, 5, size=8)
    k = r.integers(-8, 9, size=(25, 16))
    perm = r.permutation(8)
    S1, _ = orc.score_row(q, k, w, 25)
    S2, _ = orc.score_row(q[perm], k, w[perm], 25)
    assert (S1 == S2).all()


def pin_indexer_causal_rows(orc):
    """Row i of sequence b covers positions 0..q_offset[b]+i (its own included)
    and leaves the rest undefined; ragged sequences."""
    r = np.random.default_rng(15)
    B, Tq, Tk, H_I, d_I = 2, 5, 12, 2, 8
    q_idx = r.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.int8)
    k_idx = r.integers(-8, 9, size=(B, Tk, d_I)).astype(np.int8)
    w = np.array([1, 2], np.int8)
    q_offset = np.array([0, 6], np.int32)
    kv_len = np.array([5, 11], np.int32)
    S = orc.scores(q_idx, k_idx, w, q_offset, kv_len)
    for b in range(B):
        for i in range(Tq):
            p = q_offset[b] + i
            row = S[b * Tq + i]
            if p < kv_len[b]:
                assert (row[p + 1:] == I32_MIN).all()
                ref, _ = orc.score_row(q_idx[b, i], k_idx[b], w, p + 1)
                assert (row[:p + 1] == ref).all()
            else:
                assert (row == I32_MIN).all()
    # the row's own key: put a needle at position p and nowhere else
    q1 = np.zeros((1, 3, 1, 4), np.int8)
    q1[0, :, 0, 0] = 1
    k1 = np.zeros((1, 3, 4), np.int8)
    k1[0, 2, 0] = 7
    S = orc.scores(q1, k1, np.array([1], np.int8), np.array([0], np.int32),
                   np.array([3], np.int32))
    assert S[2, 2] == 7 and S[1, :2].tolist() == [0, 0]


def pin_indexer_overflow(orc):
    """H_I*d_I <= 1024 never leaves int32: the extreme value fits exactly; twice
    as many heads overflow and are reported."""
    q = np.full((16, 64), -128, np.int8)
    k = np.full((2, 64), -128, np.int8)
    S, ovf = orc.score_row(q, k, np.full(16, 127, np.int8), 2)
    assert not ovf and S.tolist() == [16 * 127 * 64 * 128 * 128] * 2
    q = np.full((32, 64), -128, np.int8)
    _, ovf = orc.score_row(q, k, np.full(32, 127, np.int8), 2)
    assert ovf


# ------------------------------------------------------------------- Top-K

def _rank_topk(S, K):
    """O(n^2) definition: s is kept iff fewer than K positions rank ahead of it."""
    n = len(S)
    keep = [s for s in range(n)
            if sum(1 for t in range(n) if S[t] > S[s] or (S[t] == S[s] and t < s)) < K]
    return keep + [-1] * (K - len(keep))


def pin_topk_hand(orc):
    g = _golden("indexer_hand.json")
    S = np.array(g["scores"], np.int32)
    for K, want in g["topk"].items():
        K = int(K)
        idx, sel = orc.topk(S, 5, K)
        if K == 1:
            assert idx[0, 0] == want[0]
        else:
            assert idx[0].tolist() == want, (K, idx[0].tolist(), want)


def pin_topk_rank_definition(orc):
    r = np.random.default_rng(21)
    for trial in range(60):
        n = int(r.integers(1, 60))
        hi = int(r.choice([2, 4, 1000]))
        S = r.integers(-hi, hi, size=n).astype(np.int32)
        for K in sorted({1, max(1, n // 3), n, n + 5}):
            idx, sel = orc.topk(S, n, K)
            want = _rank_topk(S.tolist(), K)
            assert idx[0].tolist() == want, (S.tolist(), K)
            m = min(K, n)
            assert sel[0, :m].tolist() == S[idx[0, :m]].tolist()
            assert (sel[0, m:] == I32_MIN).all()


def pin_topk_closed_forms(orc):
    n, K = 100, 17
    idx, _ = orc.topk(np.arange(n, dtype=np.int32), n, K)
    assert idx[0].tolist() == list(range(n - K, n))
    idx, _ = orc.topk(-np.arange(n, dtype=np.int32), n, K)
    assert idx[0].tolist() == list(range(K))
    idx, _ = orc.topk(np.full(n, 5, np.int32), n, K)
    assert idx[0].tolist() == list(range(K))
    S = np.full(n, I32_MIN, np.int32)
    S[[3, 50, 99]] = np.iinfo(np.int32).max
    idx, _ = orc.topk(S, n, 5)
    assert idx[0].tolist() == [0, 1, 3, 50, 99]
    # only the first n entries of a row are candidates
    idx, _ = orc.topk(np.arange(n, dtype=np.int32), 10, 4)
    assert idx[0].tolist() == [6, 7, 8, 9]


def pin_topk_invariants(orc):
    r = np.random.default_rng(22)
    n, K = 5000, 300
    S = (r.integers(0, 400, size=n) * r.integers(0, 2, size=n)).astype(np.int32)
    idx, sel = orc.topk(S, n, K)
    idx = idx[0]
    assert (np.diff(idx) > 0).all() and idx[0] >= 0 and idx[-1] < n
    mask = np.zeros(n, bool)
    mask[idx] = True
    v = S[mask].min()
    assert v >= S[~mask].max()
    ties_in = np.flatnonzero(mask & (S == v))
    ties_out = np.flatnonzero(~mask & (S == v))
    if len(ties_out):
        assert ties_in.max() < ties_out.min()


def pin_topk_split_merge(orc):
    """Exact two-level selection (used by history-split decode): the Top-K of the
    union of each chunk's Top-K equals the Top-K of the whole row."""
    r = np.random.default_rng(23)
    n, K = 3000, 64
    S = r.integers(0, 50, size=n).astype(np.int32)
    want, _ = orc.topk(S, n, K)
    for chunks in (1, 2, 7, 32):
        bounds = np.linspace(0, n, chunks + 1).astype(int)
        cand = []
        for c in range(chunks):
            lo, hi = bounds[c], bounds[c + 1]
            loc, _ = orc.topk(S[lo:hi], hi - lo, K)
            cand += [lo + s for s in loc[0] if s >= 0]
        cand = np.array(sorted(cand))
        sub, _ = orc.topk(S[cand], len(cand), K)
        got = cand[sub[0][sub[0] >= 0]]
        assert got.tolist() == want[0].tolist()


# --------------------------------------------------------------- attention

def _rand_bf16(r, shape):
    return _bf(r.standard_normal(shape).astype(np.float32))


def _sdpa_dense(q, k, v, scale):
    """Dense causal attention from torch's SDPA in fp64 (library routine); GQA
    by repeating each KV head over its group of query heads."""
    import torch
    qf = torch.from_numpy(bf16_to_f32(q).astype(np.float64)).permute(0, 2, 1, 3)
    kf = torch.from_numpy(bf16_to_f32(k).astype(np.float64)).permute(0, 2, 1, 3)
    vf = torch.from_numpy(bf16_to_f32(v).astype(np.float64)).permute(0, 2, 1, 3)
    G = qf.shape[1] // kf.shape[1]
    kf = kf.repeat_interleave(G, dim=1)
    vf = vf.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True,
                                                         scale=scale)
    logits = (qf @ kf.transpose(-1, -2)) * scale
    T = qf.shape[2]
    logits = logits.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def pin_attn_hand(orc):
    g = _golden("attention_hand.json")
    q = _bf(g["q"])[None, None]
    k = _bf(g["k"])[None, :, None]
    v = _bf(g["v"])[None, :, None]
    gate = _bf(g["gate"])[None, None]
    idx = np.array([g["idx"]], np.int32)
    out, lse = orc.attention(q, k, v, gate, idx, np.array([3]), g["scale"], rows=[[0, 0]])
    assert np.allclose(out[0], g["out"], rtol=0, atol=1e-14)
    assert np.allclose(lse[0], g["lse"], rtol=0, atol=1e-14)
    out, _ = orc.attention(q, k, v, None, idx, np.array([3]), g["scale"], rows=[[0, 0]])
    assert np.allclose(out[0], g["out_ungated"], rtol=0, atol=1e-14)
    out, lse = orc.attention(q, k, v, gate, idx, np.array([3]), g["scale"], rows=[[0, 0]],
                             mix=_bf(g["mix"])[None, None])
    assert np.allclose(out[0], g["out_mixed"], rtol=0, atol=1e-14)
    assert np.allclose(lse[0], g["lse"], rtol=0, atol=1e-14)


def pin_attn_dense_equivalence(orc):
    """K >= p+1 selects every causal position, so the layer is dense causal attention."""
    r = np.random.default_rng(31)
    B, T, Hq, Hkv, d = 2, 24, 4, 2, 16
    q = _rand_bf16(r, (B, T, Hq, d))
    k = _rand_bf16(r, (B, T, Hkv, d))
    v = _rand_bf16(r, (B, T, Hkv, d))
    scale = float(np.float32(0.3))
    K = T + 3
    idx = np.full((B * T, K), -1, np.int32)
    for b in range(B):
        for i in range(T):
            idx[b * T + i, :i + 1] = np.arange(i + 1)
    out, lse = orc.attention(q, k, v, None, idx, np.array([T, T]), scale)
    ref, ref_lse = _sdpa_dense(q, k, v, scale)
    assert np.abs(out.reshape(B, T, Hq, d) - ref).max() < 1e-12
    assert np.abs(lse.reshape(B, T, Hq) - ref_lse).max() < 1e-12


def pin_attn_f32_dense_equivalence(orc):
    """The fp32-source form: K >= p+1 on fp32 inputs (not bf16-representable)
    is dense causal attention, from torch's SDPA in fp64 on the same fp32
    values; with the gate, sigmoid(G) times it (scipy expit)."""
    import torch
    from scipy.special import expit
    r = np.random.default_rng(36)
    B, T, Hq, Hkv, d = 2, 20, 4, 1, 16
    q = r.standard_normal((B, T, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, T, Hkv, d)).astype(np.float32)
    v = r.standard_normal((B, T, Hkv, d)).astype(np.float32)
    g = r.standard_normal((B, T, Hq, d)).astype(np.float32)
    scale = 0.125
    idx = np.full((B * T, T), -1, np.int32)
    for b in range(B):
        for i in range(T):
            idx[b * T + i, :i + 1] = np.arange(i + 1)
    out, lse = orc.attention_f32(q, k, v, g, idx, np.array([T, T]), scale)
    qf = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kf = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
    vf = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy() * expit(g.astype(np.float64))
    assert np.abs(out.reshape(B, T, Hq, d) - ref).max() < 1e-12
    assert np.isfinite(lse).all()


def pin_attn_f32_matches_bf16_form(orc):
    """On values that bf16 represents exactly, the fp32-source form and the bf16
    form read the same numbers and must agree bit for bit (ragged index rows,
    padding, an entry past the history, two index sets)."""
    r = np.random.default_rng(37)
    B, Tq, Tk, Hq, Hkv, d, K = 2, 6, 30, 4, 2, 8, 7
    q, gate = _rand_bf16(r, (B, Tq, Hq, d)), _rand_bf16(r, (B, Tq, Hq, d))
    k, v = _rand_bf16(r, (B, Tk, Hkv, d)), _rand_bf16(r, (B, Tk, Hkv, d))
    kv_len = np.array([30, 21], np.int32)
    idx = r.integers(-1, 30, size=(B * Tq, Hkv, K)).astype(np.int32)
    a, la = orc.attention(q, k, v, gate, idx, kv_len, 0.3)
    f = [bf16_to_f32(x).astype(np.float32) for x in (q, k, v, gate)]
    b, lb = orc.attention_f32(f[0], f[1], f[2], f[3], idx, kv_len, 0.3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    a, _ = orc.attention(q, k, v, None, idx[:, 0], kv_len, 0.3)
    b, _ = orc.attention_f32(f[0], f[1], f[2], None, idx[:, 0], kv_len, 0.3)
    assert np.array_equal(a, b)


def pin_attn_single_key(orc):
    """K = 1: softmax of one logit is 1, so y = sigmoid(G) * V[s] (scipy expit)."""
    from scipy.special import expit
    r = np.random.default_rng(32)
    Tk, Hq, Hkv, d = 9, 4, 2, 8
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    v = _rand_bf16(r, (1, Tk, Hkv, d))
    gate = _rand_bf16(r, (1, 1, Hq, d))
    out, _ = orc.attention(q, k, v, gate, np.array([[5]], np.int32), np.array([Tk]), 0.7)
    vv = bf16_to_f32(v[0, 5]).astype(np.float64)
    want = np.stack([vv[h // 2] for h in range(Hq)]) * expit(bf16_to_f32(gate[0, 0]).astype(
        np.float64))
    assert np.abs(out[0] - want).max() < 1e-14


def pin_attn_constant_values(orc):
    """Every selected V row of KV head g equal to c_g gives o = c_g for its query heads."""
    r = np.random.default_rng(33)
    Tk, Hq, Hkv, d = 40, 6, 3, 8
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    c = _rand_bf16(r, (Hkv, d))
    v = np.broadcast_to(c, (1, Tk, Hkv, d)).copy()
    idx = np.array([r.choice(Tk, 15, replace=False)], np.int32)
    out, _ = orc.attention(q, k, v, None, idx, np.array([Tk]), 0.25)
    cf = bf16_to_f32(c).astype(np.float64)
    for h in range(Hq):
        assert np.abs(out[0, h] - cf[h // 2]).max() < 1e-14


def pin_attn_two_keys(orc):
    """Two selected keys: the weights are the logistic function of the logit gap."""
    r = np.random.default_rng(34)
    d = 8
    q = _rand_bf16(r, (1, 1, 1, d))
    k = _rand_bf16(r, (1, 2, 1, d))
    v = _rand_bf16(r, (1, 2, 1, d))
    scale = 0.5
    out, _ = orc.attention(q, k, v, None, np.array([[0, 1]], np.int32), np.array([2]), scale)
    qf, kf, vf = (bf16_to_f32(x).astype(np.float64) for x in (q, k, v))
    gap = scale * (float(qf[0, 0, 0] @ kf[0, 0, 0]) - float(qf[0, 0, 0] @ kf[0, 1, 0]))
    a0 = 1.0 / (1.0 + np.exp(-gap))
    want = a0 * vf[0, 0, 0] + (1 - a0) * vf[0, 1, 0]
    assert np.abs(out[0, 0] - want).max() < 1e-14


def pin_attn_permutation_and_padding(orc):
    r = np.random.default_rng(35)
    Tk, Hq, Hkv, d = 64, 4, 1, 16
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    v = _rand_bf16(r, (1, Tk, Hkv, d))
    sel = np.sort(r.choice(Tk, 20, replace=False)).astype(np.int32)
    o1, l1 = orc.attention(q, k, v, None, sel[None], np.array([Tk]), 0.25)
    o2, l2 = orc.attention(q, k, v, None, r.permutation(sel)[None], np.array([Tk]), 0.25)
    padded = np.concatenate([sel, np.full(7, -1, np.int32)])
    o3, l3 = orc.attention(q, k, v, None, r.permutation(padded)[None], np.array([Tk]), 0.25)
    assert np.abs(o1 - o2).max() < 1e-14 and np.abs(o1 - o3).max() < 1e-14
    assert np.abs(l1 - l3).max() < 1e-14


def pin_attn_history_past_allocation(orc):
    """A history length beyond the allocated rows (kv_len > Tk) is not a valid
    history (the library's validity rule: 0 <= p < kv_len <= Tk): attention over
    it reads no entry, so the output is 0 (the gate's mix alone with a mix),
    lse is -inf, and every gradient is 0, while the same rows with kv_len = Tk
    give ordinary results."""
    r = np.random.default_rng(36)
    B, Tq, Tk, Hq, Hkv, d, K = 1, 3, 16, 2, 1, 8, 6
    q = _rand_bf16(r, (B, Tq, Hq, d))
    k, v = (_rand_bf16(r, (B, Tk, Hkv, d)) for _ in range(2))
    G, x, dy = (_rand_bf16(r, (B, Tq, Hq, d)) for _ in range(3))
    idx = np.stack([np.sort(r.choice(Tk, K, replace=False)) for _ in range(Tq)])[None]
    idx = idx.astype(np.int32)
    o, lse = orc.attention(q, k, v, None, idx.reshape(Tq, K), np.array([Tk + 1]), 0.3)
    assert (o == 0).all() and np.isneginf(lse).all()
    o_ok, lse_ok = orc.attention(q, k, v, None, idx.reshape(Tq, K), np.array([Tk]), 0.3)
    assert np.isfinite(lse_ok).all() and np.abs(o_ok).max() > 0
    om, _ = orc.attention(q, k, v, G, idx.reshape(Tq, K), np.array([Tk + 1]), 0.3, mix=x)
    from scipy.special import expit
    want = expit(-bf16_to_f32(G).astype(np.float64)) * bf16_to_f32(x).astype(np.float64)
    assert np.abs(om - want.reshape(om.shape)).max() < 1e-12
    g = orc.attention_bwd(q, k, v, G, idx, np.array([Tk + 1]), 0.3, dy, mix=x)
    for name in ("dq", "dk", "dv"):
        assert (g[name] == 0).all(), name
    # o = 0: dgate = dy*(0 - x)*s*(1 - s), dmix = (1 - s)*dy
    sg = expit(bf16_to_f32(G).astype(np.float64))
    xf, dyf = (bf16_to_f32(a).astype(np.float64) for a in (x, dy))
    assert np.abs(g["dgate"] - (-dyf * xf * sg * (1 - sg))).max() < 1e-12
    assert np.abs(g["dmix"] - (1 - sg) * dyf).max() < 1e-12
    g_ok = orc.attention_bwd(q, k, v, G, idx, np.array([Tk]), 0.3, dy, mix=x)
    assert np.abs(g_ok["dq"]).max() > 0


def pin_attn_mask_formulation(orc):
    """Page 5's form (scores over the whole cache, a sparse mask, masked softmax via
    torch) equals attention over the gathered rows."""
    import torch
    r = np.random.default_rng(36)
    Tk, Hq, Hkv, d = 50, 4, 2, 16
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    v = _rand_bf16(r, (1, Tk, Hkv, d))
    gate = _rand_bf16(r, (1, 1, Hq, d))
    sel = np.sort(r.choice(Tk, 12, replace=False)).astype(np.int32)
    out, lse = orc.attention(q, k, v, gate, sel[None], np.array([Tk]), 0.3)
    qt = torch.from_numpy(bf16_to_f32(q[0, 0]).astype(np.float64))
    kt = torch.from_numpy(bf16_to_f32(k[0]).astype(np.float64))
    vt = torch.from_numpy(bf16_to_f32(v[0]).astype(np.float64))
    gt = torch.from_numpy(bf16_to_f32(gate[0, 0]).astype(np.float64))
    mask = torch.full((Tk,), float("-inf"), dtype=torch.float64)
    mask[torch.from_numpy(sel).long()] = 0.0
    for h in range(Hq):
        g = h // (Hq // Hkv)
        logits = (kt[:, g] @ qt[h]) * 0.3 + mask
        a = torch.softmax(logits, dim=0)
        o = (a[:, None] * vt[:, g]).sum(0) * torch.sigmoid(gt[h])
        assert (o.numpy() - out[0, h]).__abs__().max() < 1e-13
        assert abs(torch.logsumexp(logits, 0).item() - lse[0, h]) < 1e-13


# -------------------------------------------------------------------- gate

def pin_gate_limits(orc):
    """G = 0 halves the output; G = +30 leaves it (to 1e-13 relative); the
    gated/ungated ratio is scipy's expit of G."""
    from scipy.special import expit
    r = np.random.default_rng(41)
    Tk, Hq, Hkv, d = 30, 2, 1, 8
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    v = _rand_bf16(r, (1, Tk, Hkv, d))
    idx = np.arange(Tk, dtype=np.int32)[None]
    o, _ = orc.attention(q, k, v, None, idx, np.array([Tk]), 0.3)
    z, _ = orc.attention(q, k, v, _bf(np.zeros((1, 1, Hq, d))), idx, np.array([Tk]), 0.3)
    assert np.abs(z - o / 2).max() < 1e-15
    big, _ = orc.attention(q, k, v, _bf(np.full((1, 1, Hq, d), 30.0)), idx, np.array([Tk]), 0.3)
    assert np.abs(big - o).max() <= 1e-12 * np.abs(o).max()
    G = _rand_bf16(r, (1, 1, Hq, d))
    y, _ = orc.attention(q, k, v, G, idx, np.array([Tk]), 0.3)
    ratio = expit(bf16_to_f32(G[0, 0]).astype(np.float64))
    assert np.abs(y[0] - o[0] * ratio).max() < 1e-14


def pin_gate_mix(orc):
    """Mixing with another branch's output x: G = 0 gives (o + x)/2, G = +30
    gives o and G = -30 gives x (to 1e-12 relative), x = o gives o for any G,
    a row with no selected entry gives sigmoid(-G) * x, and the random-G case
    weighs the ungated output by scipy's expit(G) and x by expit(-G)."""
    from scipy.special import expit
    r = np.random.default_rng(43)
    Tk, Hq, Hkv, d = 30, 4, 2, 8
    q = _rand_bf16(r, (1, 1, Hq, d))
    k = _rand_bf16(r, (1, Tk, Hkv, d))
    v = _rand_bf16(r, (1, Tk, Hkv, d))
    x = _rand_bf16(r, (1, 1, Hq, d))
    xf = bf16_to_f32(x[0]).astype(np.float64)
    idx = np.arange(Tk, dtype=np.int32)[None]
    kv = np.array([Tk])
    o, lse0 = orc.attention(q, k, v, None, idx, kv, 0.3)

    def run(G, mix=x, sel=idx):
        return orc.attention(q, k, v, G, sel, kv, 0.3, mix=mix)

    z, lse = run(_bf(np.zeros((1, 1, Hq, d))))
    assert np.abs(z - (o + xf) / 2).max() < 1e-15
    assert (lse == lse0).all()
    big, _ = run(_bf(np.full((1, 1, Hq, d), 30.0)))
    assert np.abs(big - o).max() <= 1e-12 * np.abs(o).max()
    small, _ = run(_bf(np.full((1, 1, Hq, d), -30.0)))
    assert np.abs(small - xf).max() <= 1e-12 * np.abs(xf).max()
    G = _rand_bf16(r, (1, 1, Hq, d))
    s = expit(bf16_to_f32(G[0]).astype(np.float64))
    y, _ = run(G)
    assert np.abs(y - (s * o + expit(-bf16_to_f32(G[0]).astype(np.float64)) * xf)).max() < 1e-14
    # x equal to the (bf16-exact) sparse output itself leaves it unchanged
    k1 = np.array([[7]], np.int32)
    o1, _ = orc.attention(q, k, v, None, k1, kv, 0.3)
    same, _ = run(G, mix=bf16_bits(o1.astype(np.float32))[None], sel=k1)
    assert np.abs(same - o1).max() < 1e-14
    empty, lse_e = run(G, sel=np.full((1, 5), -1, np.int32))
    assert np.abs(empty - (1 - s) * xf).max() < 1e-15
    assert np.isneginf(lse_e).all()


# ------------------------------------------------------------------- layer

def pin_layer_dense_rows(orc):
    """Through the whole layer, rows with K >= p+1 equal gated dense causal attention."""
    from scipy.special import expit
    import synth
    cfg = synth.CONFIGS["tiny"].replace(Tq=40, Tk=40)
    inp = synth.host_inputs(cfg, seed=3)
    res = orc.layer(inp, K=64)
    ref, ref_lse = _sdpa_dense(inp["q"], inp["k"], inp["v"], inp["scale"])
    gate = expit(bf16_to_f32(inp["gate"]).astype(np.float64))
    want = ref * gate
    got = res["out"].reshape(want.shape)
    assert np.abs(got - want).max() < 1e-12
    assert np.abs(res["lse"].reshape(ref_lse.shape) - ref_lse).max() < 1e-12
    for i in range(cfg.Tq):
        assert res["idx"][i].tolist() == list(range(i + 1)) + [-1] * (64 - i - 1)


def pin_layer_composition(orc):
    """The whole-layer entry equals score -> Top-K -> attention run step by step,
    including an invalid row (position beyond the history) and ragged sequences."""
    import synth
    cfg = synth.CONFIGS["tiny"].replace(B=2, Tq=6, Tk=70, K=9, decode=False)
    inp = synth.host_inputs(cfg, seed=5)
    inp["q_offset"] = np.array([10, 63], np.int32)
    inp["kv_len"] = np.array([40, 68], np.int32)
    res = orc.layer(inp, K=9)
    S = orc.scores(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"])
    n = np.array([inp["q_offset"][b] + i + 1 for b in range(2) for i in range(6)])
    valid = np.array([inp["q_offset"][b] + i < inp["kv_len"][b] for b in range(2)
                      for i in range(6)])
    idx, sel = orc.topk(S, np.where(valid, n, 0), 9)
    out, lse = orc.attention(inp["q"], inp["k"], inp["v"], inp["gate"], idx, inp["kv_len"],
                             inp["scale"])
    assert (res["idx"] == idx).all() and (res["sel"] == sel).all()
    assert np.abs(res["out"] - out).max() == 0.0
    assert (~valid).sum() == 1 and (res["idx"][~valid] == -1).all()
    assert (res["out"][~valid] == 0).all() and np.isneginf(res["lse"][~valid]).all()


def pin_layer_mix(orc):
    """With another branch's output x in the input, the whole layer equals the
    unmixed layer's selection followed by the mixed attention step, and an
    invalid row (no history to select from) gives sigmoid(-G) * x."""
    from scipy.special import expit
    import synth
    cfg = synth.CONFIGS["tiny"].replace(B=2, Tq=6, Tk=70, K=9, decode=False)
    inp = synth.host_inputs(cfg, seed=6)
    inp["q_offset"] = np.array([10, 63], np.int32)
    inp["kv_len"] = np.array([40, 68], np.int32)
    base = orc.layer(inp, K=9)
    inp["mix"] = synth.host_mix(cfg, seed=6)
    res = orc.layer(inp, K=9)
    assert (res["idx"] == base["idx"]).all() and (res["sel"] == base["sel"]).all()
    assert np.array_equal(res["lse"], base["lse"])
    out, _ = orc.attention(inp["q"], inp["k"], inp["v"], inp["gate"], base["idx"],
                           inp["kv_len"], inp["scale"], mix=inp["mix"])
    valid = ~np.isneginf(base["lse"][:, 0])
    assert (~valid).sum() == 1
    assert np.abs(res["out"][valid] - out[valid]).max() == 0.0
    G = bf16_to_f32(inp["gate"]).astype(np.float64).reshape(res["out"].shape)
    x = bf16_to_f32(inp["mix"]).astype(np.float64).reshape(res["out"].shape)
    assert np.abs(res["out"][~valid] - expit(-G[~valid]) * x[~valid]).max() < 1e-15


# ------------------------------------------------------------------ append

def pin_append_hand(orc):
    """Hand-worked append: rows go right after each history, the ones past the
    capacity are dropped, lengths outside 0..Tk are taken at the nearest end."""
    new = np.arange(1, 2 * 3 * 2 + 1, dtype=np.uint8).reshape(2, 3, 2)  # rows (1,2) (3,4) (5,6) | (7,8) (9,10) (11,12)
    cache = np.full((2, 5, 2), 0xEE, np.uint8)
    out, qo, kl = orc.kv_append(new, cache, np.array([1, 4], np.int32), np.array([3, 2], np.int32))
    E = 0xEE
    want = np.array([[[E, E], [1, 2], [3, 4], [5, 6], [E, E]],
                     [[E, E], [E, E], [E, E], [E, E], [7, 8]]], np.uint8)
    assert (out == want).all()
    assert qo.tolist() == [1, 4] and kl.tolist() == [4, 5]
    assert (cache == E).all()                      # the input is not modified
    out, qo, kl = orc.kv_append(new, cache, np.array([-3, 9], np.int32))
    assert qo.tolist() == [0, 5] and kl.tolist() == [3, 5]
    assert (out[0, :3] == new[0]).all() and (out[0, 3:] == E).all() and (out[1] == E).all()
    out, qo, kl = orc.kv_append(new, cache, np.array([0, 2], np.int32), np.array([0, 9], np.int32))
    assert (out[0] == E).all() and (out[1, 2:] == new[1]).all() and kl.tolist() == [0, 5]


def pin_append_chunked_layer(orc):
    """Chunked prefill: caches built by appending chunks of 7, 13 and 20 rows
    (the second sequence appends fewer rows to each chunk) hold the full history,
    and the layer run on each chunk's rows at the returned q_offset / kv_len
    equals the same rows of the layer run once on the whole history."""
    import synth
    cfg = synth.CONFIGS["tiny"].replace(B=2, Tq=40, Tk=40, K=9)
    inp = synth.host_inputs(cfg, seed=12)
    full = orc.layer(inp, K=9)
    caches = {n: np.zeros_like(inp[n]) for n in ("k", "v", "k_idx")}
    kv_len = np.zeros(2, np.int32)
    start = np.zeros(2, np.int64)
    for c in (7, 13, 20):
        n_new = np.array([c, c - 3], np.int32)
        for n in caches:
            chunk = np.zeros((2, c) + inp[n].shape[2:], inp[n].dtype)
            for b in range(2):
                chunk[b, :n_new[b]] = inp[n][b, start[b]:start[b] + n_new[b]]
            caches[n], qo, kl = orc.kv_append(chunk, caches[n], kv_len, n_new)
        assert qo.tolist() == kv_len.tolist() and kl.tolist() == (kv_len + n_new).tolist()
        sub = dict(inp, k=caches["k"], v=caches["v"], k_idx=caches["k_idx"], q_offset=qo,
                   kv_len=kl)
        for n in ("q_idx", "q", "gate"):
            sub[n] = np.zeros((2, c) + inp[n].shape[2:], inp[n].dtype)
            for b in range(2):
                sub[n][b, :n_new[b]] = inp[n][b, start[b]:start[b] + n_new[b]]
        res = orc.layer(sub, K=9)
        for b in range(2):
            rows = slice(b * c, b * c + n_new[b])
            frows = slice(b * 40 + start[b], b * 40 + start[b] + n_new[b])
            assert (res["idx"][rows] == full["idx"][frows]).all()
            assert np.array_equal(res["out"][rows], full["out"][frows])
            # rows past the appended ones lie beyond the history: invalid
            assert (res["idx"][b * c + n_new[b]:(b + 1) * c] == -1).all()
        kv_len = kl
        start += n_new
    for n in caches:
        for b in range(2):
            assert (caches[n][b, :start[b]] == inp[n][b, :start[b]]).all()


# ------------------------------------------------------------ block Top-K

def pin_block_topk_hand(orc):
    """Hand-worked blocks of 2: scores 5 1 | 9 9 | 2 7 | 3 score 5, 9, 7, 3."""
    S = np.array([5, 1, 9, 9, 2, 7, 3], np.int32)
    idx, blk, sel = orc.block_topk(S, 7, 2, 2)
    assert blk[0].tolist() == [1, 2] and sel[0].tolist() == [9, 7]
    assert idx[0].tolist() == [2, 3, 4, 5]
    idx, blk, sel = orc.block_topk(S, 7, 5, 2)   # more blocks asked than exist
    assert blk[0].tolist() == [0, 1, 2, 3, -1] and sel[0].tolist() == [5, 9, 7, 3, I32_MIN]
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5, 6, -1, -1, -1]
    # only the first 5 candidates: the last block is position 4 alone (score 2)
    idx, blk, sel = orc.block_topk(S, 5, 2, 2)
    assert blk[0].tolist() == [0, 1] and idx[0].tolist() == [0, 1, 2, 3]
    idx, blk, sel = orc.block_topk(S, 5, 3, 2)
    assert idx[0].tolist() == [0, 1, 2, 3, 4, -1] and sel[0].tolist() == [5, 9, 2]
    # equal block scores: the lower block wins
    T = np.array([4, 4, 1, 4, 4], np.int32)
    idx, blk, sel = orc.block_topk(T, 5, 2, 2)
    assert blk[0].tolist() == [0, 1] and idx[0].tolist() == [0, 1, 2, 3]


def pin_block_topk_definition(orc):
    """Against a brute-force reading of the definition (numpy block maxima, a
    Python sort by (score desc, block asc)) on rows with heavy ties; block 1 is
    the position Top-K."""
    r = np.random.default_rng(44)
    for trial in range(40):
        n = int(r.integers(1, 200))
        block = int(r.choice([1, 2, 3, 8, 16, 64]))
        K = int(r.integers(1, 12))
        S = r.integers(-3, 4, n).astype(np.int32) * 1000
        idx, blk, sel = orc.block_topk(S, n, K, block)
        nb = -(-n // block)
        pad = np.full(nb * block, np.iinfo(np.int32).min, np.int64)
        pad[:n] = S
        bs = pad.reshape(nb, block).max(axis=1)
        keep = sorted(sorted(range(nb), key=lambda j: (-bs[j], j))[:K])
        want_blk = keep + [-1] * (K - len(keep))
        assert blk[0].tolist() == want_blk, (trial, n, block, K)
        assert sel[0].tolist() == [int(bs[j]) for j in keep] + [I32_MIN] * (K - len(keep))
        pos = [s for j in keep for s in range(j * block, min((j + 1) * block, n))]
        assert idx[0].tolist() == pos + [-1] * (K * block - len(pos))
        if block == 1:
            pidx, psel = orc.topk(S, n, K)
            assert (pidx == idx).all() and (psel == sel).all()


def pin_layer_block_dense_and_composition(orc):
    """Through the whole layer with blocks of 16: K >= ceil((p+1)/16) keeps every
    position (gated dense causal attention, torch SDPA); with fewer blocks the
    layer equals scores -> block Top-K -> attention over the expanded rows."""
    from scipy.special import expit
    import synth
    cfg = synth.CONFIGS["tiny"].replace(Tq=40, Tk=40)
    inp = synth.host_inputs(cfg, seed=13)
    res = orc.layer(inp, K=3, block=16)
    ref, ref_lse = _sdpa_dense(inp["q"], inp["k"], inp["v"], inp["scale"])
    want = ref * expit(bf16_to_f32(inp["gate"]).astype(np.float64))
    assert np.abs(res["out"].reshape(want.shape) - want).max() < 1e-12
    assert np.abs(res["lse"].reshape(ref_lse.shape) - ref_lse).max() < 1e-12
    for i in range(cfg.Tq):
        assert res["idx"][i].tolist() == list(range(i + 1)) + [-1] * (48 - i - 1)
    cfg = synth.CONFIGS["tiny"].replace(B=2, Tq=6, Tk=70, decode=False)
    inp = synth.host_inputs(cfg, seed=14)
    inp["q_offset"] = np.array([10, 60], np.int32)
    inp["kv_len"] = np.array([40, 68], np.int32)
    res = orc.layer(inp, K=2, block=8)
    S = orc.scores(inp["q_idx"], inp["k_idx"], inp["w"], inp["q_offset"], inp["kv_len"])
    n = np.array([inp["q_offset"][b] + i + 1 if inp["q_offset"][b] + i < inp["kv_len"][b] else 0
                  for b in range(2) for i in range(6)])
    idx, blk, sel = orc.block_topk(S, n, 2, 8)
    out, lse = orc.attention(inp["q"], inp["k"], inp["v"], inp["gate"], idx, inp["kv_len"],
                             inp["scale"])
    assert (res["idx"] == idx).all() and (res["sel"] == sel).all()
    assert np.array_equal(res["out"], out) and np.array_equal(res["lse"], lse)


# ------------------------------------------------------------ index sets

def _set_sub_problem(inp, sets, s):
    """Set s's own shared-set problem, sliced with numpy: its group of indexer
    heads and their weights, its query heads (and gates), and the key/value
    heads those query heads read."""
    Hq, Hkv, H_I = inp["q"].shape[2], inp["k"].shape[2], inp["q_idx"].shape[2]
    hps, Hg, G = Hq // sets, H_I // sets, Hq // Hkv
    k0, k1 = s * hps // G, ((s + 1) * hps - 1) // G + 1
    sub = dict(inp)
    sub["q_idx"] = np.ascontiguousarray(inp["q_idx"][:, :, s * Hg:(s + 1) * Hg])
    sub["w"] = np.ascontiguousarray(inp["w"][s * Hg:(s + 1) * Hg])
    for n in ("q", "gate"):
        sub[n] = np.ascontiguousarray(inp[n][:, :, s * hps:(s + 1) * hps])
    for n in ("k", "v"):
        sub[n] = np.ascontiguousarray(inp[n][:, :, k0:k1])
    return sub


def pin_sets_sub_problems(orc):
    """Index sets (query head h reads set h // (Hq/sets), set g scored by its
    group of indexer heads) equal, set by set, the shared-set layer run on that
    set's own sub-problem: one set per key/value head, one per query head (two
    query heads on one key/value head then read different sets), and two sets
    over four key/value heads. Identical indexer groups give every head the
    shared-set selection."""
    import synth
    base = synth.CONFIGS["tiny"].replace(B=2, Tq=12, Tk=60, K=7, decode=False)
    cases = [  # (Hq, Hkv, H_I, sets)
        (4, 2, 4, 2),    # one set per key/value head
        (4, 2, 4, 4),    # one set per query head
        (8, 4, 4, 2),    # a set spans two key/value heads
    ]
    for Hq, Hkv, H_I, sets in cases:
        cfg = base.replace(Hq=Hq, Hkv=Hkv, H_I=H_I)
        inp = synth.host_inputs(cfg, seed=15)
        inp["w"] = np.array([1, 3, 4, 2], np.int8)[:H_I]
        inp["q_offset"] = np.array([40, 50], np.int32)
        inp["kv_len"] = np.array([52, 55], np.int32)   # sequence 1 ends in invalid rows
        hps = Hq // sets
        for block in (1, 4):
            K = 3 if block > 1 else cfg.K
            res = orc.layer(inp, K=K, block=block, sets=sets)
            for g in range(sets):
                one = orc.layer(_set_sub_problem(inp, sets, g), K=K, block=block)
                assert (res["idx"][:, g] == one["idx"]).all()
                assert (res["sel"][:, g] == one["sel"]).all()
                assert np.array_equal(res["out"][:, g * hps:(g + 1) * hps], one["out"])
                assert np.array_equal(res["lse"][:, g * hps:(g + 1) * hps], one["lse"])
            assert not (res["idx"][:, 0] == res["idx"][:, 1]).all()
    # every group a copy of group 0: every head keeps the shared-set selection
    cfg = base.replace(Hq=4, Hkv=2, H_I=4)
    inp = synth.host_inputs(cfg, seed=15)
    inp["q_offset"] = np.array([40, 50], np.int32)
    inp["kv_len"] = np.array([52, 55], np.int32)
    for sets in (2, 4):
        Hg = 4 // sets
        dup = dict(inp)
        dup["q_idx"] = np.ascontiguousarray(np.concatenate([inp["q_idx"][:, :, :Hg]] * sets, axis=2))
        dup["w"] = np.tile(np.array([1, 3], np.int8)[:Hg], sets)
        res = orc.layer(dup, K=cfg.K, sets=sets)
        one = dict(dup, q_idx=np.ascontiguousarray(inp["q_idx"][:, :, :Hg]),
                   w=np.array([1, 3], np.int8)[:Hg])
        shared = orc.layer(one, K=cfg.K)
        for g in range(sets):
            assert (res["idx"][:, g] == shared["idx"]).all()
        assert np.array_equal(res["out"], shared["out"])


# ------------------------------------------------------------------ backward

def _torch_sparse_forward(q, k, v, G, x, idx, kv_len, scale):
    """The gated sparse attention written with torch ops on float64 tensors (an
    independent statement of the forward, for autograd)."""
    import torch
    B, Tq, Hq, d = q.shape
    Hkv = k.shape[2]
    it = torch.from_numpy(idx.astype(np.int64))                       # [B,Tq,K]
    valid = (it >= 0) & (it < torch.from_numpy(kv_len.astype(np.int64))[:, None, None])
    safe = torch.where(valid, it, torch.zeros_like(it))
    bi = torch.arange(B)[:, None, None]
    ks = k[bi, safe].repeat_interleave(Hq // Hkv, dim=3)             # [B,Tq,K,Hq,d]
    vs = v[bi, safe].repeat_interleave(Hq // Hkv, dim=3)
    logits = (ks * q[:, :, None]).sum(-1) * scale                      # [B,Tq,K,Hq]
    logits = logits.masked_fill(~valid[..., None], float("-inf"))
    any_valid = valid.any(-1)[..., None, None]                         # [B,Tq,1,1]
    P = torch.softmax(torch.where(any_valid, logits, torch.zeros_like(logits)), dim=2)
    P = torch.where(any_valid & valid[..., None], P, torch.zeros_like(P))
    o = (P[..., None] * vs).sum(2)                                     # [B,Tq,Hq,d]
    if G is None:
        return o
    s = torch.sigmoid(G)
    return s * o + (1 - s) * x if x is not None else s * o


def _bwd_against_autograd(orc, q, k, v, G, x, idx, kv_len, scale, dy, tol):
    import torch
    t = lambda a: torch.from_numpy(bf16_to_f32(a).astype(np.float64)).requires_grad_(True)
    tq, tk, tv = t(q), t(k), t(v)
    tg = t(G) if G is not None else None
    tx = t(x) if x is not None else None
    y = _torch_sparse_forward(tq, tk, tv, tg, tx, idx, kv_len, scale)
    (y * torch.from_numpy(bf16_to_f32(dy).astype(np.float64))).sum().backward()
    res = orc.attention_bwd(q, k, v, G, idx, kv_len, scale, dy, mix=x)
    pairs = [("dq", tq), ("dk", tk), ("dv", tv)]
    if G is not None:
        pairs.append(("dgate", tg))
    if x is not None:
        pairs.append(("dmix", tx))
    for name, leaf in pairs:
        want = leaf.grad.numpy()
        assert np.abs(res[name] - want).max() <= tol * max(1.0, np.abs(want).max()), name


def _torch_sparse_forward_sets(q, k, v, G, x, idx, kv_len, scale):
    """The gated sparse attention with index sets, written with torch ops on
    float64 tensors (an independent statement of the forward, for autograd):
    idx [B,Tq,S,K]; query head h attends over set h // (Hq // S) and reads
    key/value head h // (Hq // Hkv)."""
    import torch
    B, Tq, Hq, d = q.shape
    Hkv, S = k.shape[2], idx.shape[2]
    it = torch.from_numpy(idx.astype(np.int64)).repeat_interleave(Hq // S, dim=2)  # [B,Tq,Hq,K]
    valid = (it >= 0) & (it < torch.from_numpy(kv_len.astype(np.int64))[:, None, None, None])
    safe = torch.where(valid, it, torch.zeros_like(it))
    bi = torch.arange(B)[:, None, None, None]
    hk = (torch.arange(Hq) // (Hq // Hkv))[None, None, :, None]
    ks, vs = k[bi, safe, hk], v[bi, safe, hk]                          # [B,Tq,Hq,K,d]
    logits = (ks * q[:, :, :, None]).sum(-1) * scale                   # [B,Tq,Hq,K]
    logits = logits.masked_fill(~valid, float("-inf"))
    any_valid = valid.any(-1, keepdim=True)
    P = torch.softmax(torch.where(any_valid, logits, torch.zeros_like(logits)), dim=-1)
    P = torch.where(any_valid & valid, P, torch.zeros_like(P))
    o = (P[..., None] * vs).sum(3)                                     # [B,Tq,Hq,d]
    if G is None:
        return o
    s = torch.sigmoid(G)
    return s * o + (1 - s) * x if x is not None else s * o


def pin_bwd_sets_autograd(orc):
    """Index sets (query head h reads set h // (Hq/S)): one per key/value head, one
    per query head, two over four key/value heads; sparse rows in any order with
    -1 padding, a repeated position, a row without entries and a short history:
    the oracle's gradients equal torch autograd through a per-head gather
    written independently, gated with the mix and ungated."""
    import torch
    r = np.random.default_rng(57)
    for Hq, Hkv, S, gated in ((4, 2, 2, True), (4, 2, 4, True), (8, 4, 2, False)):
        B, Tq, Tk, d, K = 2, 5, 30, 16, 9
        q = _rand_bf16(r, (B, Tq, Hq, d))
        k, v = (_rand_bf16(r, (B, Tk, Hkv, d)) for _ in range(2))
        G, x, dy = (_rand_bf16(r, (B, Tq, Hq, d)) for _ in range(3))
        idx = r.integers(0, Tk, size=(B, Tq, S, K)).astype(np.int32)
        idx[0, 0, :, 0] = idx[0, 0, :, 1]          # a repeated position
        idx[:, :, :, -2:] = -1                       # padding
        idx[1, 3, 0] = -1                            # a row (set 0) without entries
        kv_len = np.array([Tk, 20], np.int32)        # sequence 1: entries past 20 dropped
        t = lambda a: torch.from_numpy(bf16_to_f32(a).astype(np.float64)).requires_grad_(True)
        tq, tk, tv = t(q), t(k), t(v)
        tg, tx = (t(G), t(x)) if gated else (None, None)
        y = _torch_sparse_forward_sets(tq, tk, tv, tg, tx, idx, kv_len, 0.3)
        (y * torch.from_numpy(bf16_to_f32(dy).astype(np.float64))).sum().backward()
        res = orc.attention_bwd(q, k, v, G if gated else None, idx, kv_len, 0.3, dy,
                                mix=x if gated else None)
        pairs = [("dq", tq), ("dk", tk), ("dv", tv)] + ([("dgate", tg), ("dmix", tx)] if gated else [])
        for name, leaf in pairs:
            want = leaf.grad.numpy()
            assert np.abs(res[name] - want).max() <= 1e-10 * max(1.0, np.abs(want).max()), (Hq, S, name)


def pin_bwd_dense_sdpa(orc):
    """K >= p+1 (every causal position): the gradients equal torch autograd through
    its SDPA (causal, fp64, GQA by head repetition) with the gate and the mix."""
    import torch
    r = np.random.default_rng(50)
    B, T, Hq, Hkv, d = 2, 20, 4, 2, 16
    q, k, v = (_rand_bf16(r, (B, T, h, d)) for h in (Hq, Hkv, Hkv))
    G, x, dy = (_rand_bf16(r, (B, T, Hq, d)) for _ in range(3))
    scale = 0.35
    idx = np.full((B, T, T + 2), -1, np.int32)
    for i in range(T):
        idx[:, i, :i + 1] = np.arange(i + 1)
    t = lambda a: torch.from_numpy(bf16_to_f32(a).astype(np.float64)).requires_grad_(True)
    tq, tk, tv, tg, tx = t(q), t(k), t(v), t(G), t(x)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(2, dim=2).transpose(1, 2),
        tv.repeat_interleave(2, dim=2).transpose(1, 2), is_causal=True, scale=scale).transpose(1, 2)
    s = torch.sigmoid(tg)
    y = s * o + (1 - s) * tx
    (y * torch.from_numpy(bf16_to_f32(dy).astype(np.float64))).sum().backward()
    res = orc.attention_bwd(q, k, v, G, idx, np.array([T, T]), scale, dy, mix=x)
    for name, leaf in (("dq", tq), ("dk", tk), ("dv", tv), ("dgate", tg), ("dmix", tx)):
        assert np.abs(res[name] - leaf.grad.numpy()).max() < 1e-12, name


def pin_bwd_sparse_autograd(orc):
    """Sparse index rows in any order, with -1 padding, a repeated position, a row
    with no entry and a history shorter than the allocation: the gradients equal
    torch autograd through an independent torch statement of the forward, gated
    and mixed, gated only, and ungated."""
    r = np.random.default_rng(51)
    B, Tq, Tk, Hq, Hkv, d, K = 2, 5, 30, 4, 1, 8, 9
    q = _rand_bf16(r, (B, Tq, Hq, d))
    k, v = (_rand_bf16(r, (B, Tk, Hkv, d)) for _ in range(2))
    G, x, dy = (_rand_bf16(r, (B, Tq, Hq, d)) for _ in range(3))
    idx = np.stack([np.stack([r.permutation(Tk)[:K] for _ in range(Tq)]) for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[0, 1, 3:] = -1
    idx[0, 2, 4] = idx[0, 2, 0]            # a repeated position counts twice
    idx[1, 3, :] = -1                      # no entry at all
    kv_len = np.array([Tk, 22])            # entries >= 22 of sequence 1 are skipped
    _bwd_against_autograd(orc, q, k, v, G, x, idx, kv_len, 0.5, dy, 1e-12)
    _bwd_against_autograd(orc, q, k, v, G, None, idx, kv_len, 0.5, dy, 1e-12)
    _bwd_against_autograd(orc, q, k, v, None, None, idx, kv_len, 0.5, dy, 1e-12)


def pin_bwd_constant_values(orc):
    """Constant value rows make the output independent of the weights: dq and dk
    vanish, dv spreads the head's output gradient over the selected rows."""
    r = np.random.default_rng(52)
    B, Tq, Tk, Hq, Hkv, d, K = 1, 3, 12, 2, 1, 8, 5
    q = _rand_bf16(r, (B, Tq, Hq, d))
    k = _rand_bf16(r, (B, Tk, Hkv, d))
    v = np.broadcast_to(_rand_bf16(r, (1, 1, 1, d)), (B, Tk, Hkv, d)).copy()
    dy = _rand_bf16(r, (B, Tq, Hq, d))
    idx = np.array([[[0, 3, 5, 7, 11], [1, 2, -1, -1, -1], [4, 4, 6, 8, 9]]], np.int32)
    res = orc.attention_bwd(q, k, v, None, idx, np.array([Tk]), 0.7, dy)
    assert np.abs(res["dq"]).max() < 1e-14 and np.abs(res["dk"]).max() < 1e-14
    # dv summed over all rows = sum over rows and heads of dy (softmax weights sum to 1)
    tot = bf16_to_f32(dy).astype(np.float64).sum(axis=(0, 1, 2))
    assert np.abs(res["dv"].sum(axis=(0, 1, 2)) - tot).max() < 1e-12




# ------------------------------------------------------- indexer gradients

def _torch_indexer_loss(q, k, w, idx, T, q_offset, kv_len, tau):
    """The distillation loss of the scorer written with torch ops on float64
    tensors (independent of the oracle, for autograd): per row, log-softmax of
    tau * sum_h w_h relu(q_h . k_s) over the row's valid entries, and
    sum_t T_t (log T_t - log p_t)."""
    import torch
    B, Tq, H_I, d_I = q.shape
    K = idx.shape[2]
    total = torch.zeros((), dtype=torch.float64)
    losses = torch.zeros((B, Tq), dtype=torch.float64)
    for b in range(B):
        for i in range(Tq):
            p = int(q_offset[b]) + i
            if not (0 <= p < int(kv_len[b]) <= k.shape[1]):
                continue
            ent = [t for t in range(K) if 0 <= int(idx[b, i, t]) <= p]
            if not ent:
                continue
            pos = torch.tensor([int(idx[b, i, t]) for t in ent])
            kk = k[b, pos]                                       # [n, d_I]
            wr = w[b, i] if w.dim() == 3 else w
            d = kk @ q[b, i].T                                   # [n, H_I]
            S = (torch.relu(d) * wr).sum(-1)
            logp = torch.log_softmax(tau * S, dim=0)
            Tt = torch.tensor([float(T[b, i, t]) for t in ent], dtype=torch.float64)
            logT = torch.where(Tt > 0, torch.log(torch.where(Tt > 0, Tt, torch.ones_like(Tt))),
                               torch.zeros_like(Tt))
            L = (Tt * (logT - logp)).sum()
            losses[b, i] = L.detach()
            total = total + L
    return total, losses


def pin_indexer_bwd_autograd(orc):
    """The oracle's gradients of the scorer's distillation loss equal torch
    autograd (fp64) through an independent statement of the loss: per-row
    weights with negative values, -1 padding, entries past the row's position,
    a repeated position, a row with no valid entry, an invalid row, and a
    teacher that does not sum to 1."""
    import torch
    r = np.random.default_rng(80)
    B, Tq, Tk, H_I, d_I, K = 2, 6, 40, 3, 8, 7
    q = r.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.int8)
    k = r.integers(-8, 9, size=(B, Tk, d_I)).astype(np.int8)
    w = r.integers(-3, 5, size=(B, Tq, H_I)).astype(np.int8)
    q_offset = np.array([20, 5], np.int32)
    kv_len = np.array([40, 9], np.int32)               # sequence 1: rows 4, 5 invalid
    idx = np.stack([np.stack([r.choice(Tk, K, replace=False) for _ in range(Tq)])
                    for _ in range(B)]).astype(np.int32)
    idx[0, 1, 4:] = -1
    idx[0, 2, 3] = idx[0, 2, 0]                         # a repeated position: two entries
    idx[0, 3, :] = 39                                   # past the row's position: none valid
    T = r.random((B, Tq, K))
    T /= T.sum(-1, keepdims=True)
    T[0, 4] *= 1.7                                      # a teacher row that sums to 1.7
    T[1, 0, 2] = 0.0                                    # a zero weight (0 log 0 = 0)
    tau = 0.01
    tq = torch.tensor(q.astype(np.float64), requires_grad=True)
    tk = torch.tensor(k.astype(np.float64), requires_grad=True)
    tw = torch.tensor(w.astype(np.float64), requires_grad=True)
    total, losses = _torch_indexer_loss(tq, tk, tw, idx, T, q_offset, kv_len, tau)
    total.backward()
    res = orc.indexer_bwd(q, k, w, q_offset, kv_len, idx, T, tau)
    assert np.abs(res["loss"] - losses.numpy()).max() < 1e-10
    for name, leaf in (("dq", tq), ("dk", tk), ("dw", tw)):
        want = leaf.grad.numpy()
        assert np.abs(res[name] - want).max() <= 1e-10 * max(1.0, np.abs(want).max()), name


def pin_indexer_bwd_closed_forms(orc):
    """A teacher equal to the scorer's own distribution (softmax of tau*S from
    numpy's scores and scipy's logsumexp) gives loss 0 and no gradient; a row
    whose single entry holds all the teacher's weight likewise; shared [H_I]
    weights give the same per-row dw as the same weights written out per row."""
    from scipy.special import logsumexp
    r = np.random.default_rng(81)
    B, Tq, Tk, H_I, d_I, K = 1, 4, 30, 2, 8, 6
    q = r.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.int8)
    k = r.integers(-8, 9, size=(B, Tk, d_I)).astype(np.int8)
    w = np.array([2, 3], np.int8)
    q_offset, kv_len = np.array([25], np.int32), np.array([30], np.int32)
    idx = np.stack([np.sort(r.choice(26, K, replace=False)) for _ in range(Tq)])[None]
    idx = idx.astype(np.int32)
    tau = 0.02
    kk = k[0][idx[0]].astype(np.int64)                           # [Tq, K, d_I]
    d = np.einsum("tkj,thj->tkh", kk, q[0].astype(np.int64))
    S = (np.maximum(d, 0) * w.astype(np.int64)).sum(-1)          # [Tq, K]
    z = tau * S
    p = np.exp(z - logsumexp(z, axis=1, keepdims=True))
    res = orc.indexer_bwd(q, k, w, q_offset, kv_len, idx, p[None], tau)
    assert np.abs(res["loss"]).max() < 1e-12
    for name in ("dq", "dk", "dw"):
        assert np.abs(res[name]).max() < 1e-9, name
    one = np.full((B, Tq, K), -1, np.int32)
    one[..., 0] = idx[..., 0]
    T1 = np.zeros((B, Tq, K))
    T1[..., 0] = 1.0
    res1 = orc.indexer_bwd(q, k, w, q_offset, kv_len, one, T1, tau)
    for name in ("loss", "dq", "dk", "dw"):
        assert np.abs(res1[name]).max() < 1e-15, name
    T = r.random((B, Tq, K))
    shared = orc.indexer_bwd(q, k, w, q_offset, kv_len, idx, T, tau)
    per_row = orc.indexer_bwd(q, k, np.broadcast_to(w, (B, Tq, H_I)).copy(), q_offset, kv_len,
                              idx, T, tau)
    for name in ("loss", "dq", "dk", "dw"):
        assert np.abs(shared[name] - per_row[name]).max() < 1e-12, name


def _ibwd_sets_problem(seed):
    r = np.random.default_rng(seed)
    B, Tq, Tk, H_I, d_I, K, S = 2, 5, 36, 6, 8, 6, 3
    q = r.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.int8)
    k = r.integers(-8, 9, size=(B, Tk, d_I)).astype(np.int8)
    w = r.integers(-3, 5, size=(B, Tq, H_I)).astype(np.int8)
    q_offset = np.array([30, 2], np.int32)
    kv_len = np.array([36, 6], np.int32)                # sequence 1: rows 4 invalid
    idx = np.stack([np.stack([np.stack([r.choice(Tk, K, replace=False) for _ in range(Tq)])
                              for _ in range(S)]) for _ in range(B)]).astype(np.int32)
    idx[0, 1, 2, 3:] = -1
    idx[1, 2, 0, :] = 35                                # past the row's position: none valid
    T = r.random((B, S, Tq, K))
    T /= T.sum(-1, keepdims=True)
    return q, k, w, q_offset, kv_len, idx, T, S


def pin_indexer_bwd_sets_autograd(orc):
    """With three index sets of two indexer heads each, the oracle's loss per
    set and its gradients equal torch autograd (fp64) of the sum of the sets'
    losses, each stated independently on its heads, weights, index rows and
    teacher (dk summed over the sets)."""
    import torch
    q, k, w, q_offset, kv_len, idx, T, S = _ibwd_sets_problem(82)
    Hs = q.shape[2] // S
    tau = 0.015
    tq = torch.tensor(q.astype(np.float64), requires_grad=True)
    tk = torch.tensor(k.astype(np.float64), requires_grad=True)
    tw = torch.tensor(w.astype(np.float64), requires_grad=True)
    total = torch.zeros((), dtype=torch.float64)
    losses = []
    for g in range(S):
        hs = slice(g * Hs, (g + 1) * Hs)
        t, l = _torch_indexer_loss(tq[:, :, hs], tk, tw[:, :, hs], idx[:, g], T[:, g], q_offset,
                                   kv_len, tau)
        total = total + t
        losses.append(l.numpy())
    total.backward()
    res = orc.indexer_bwd(q, k, w, q_offset, kv_len, idx, T, tau)
    assert res["loss"].shape == (q.shape[0], S, q.shape[1])
    assert np.abs(res["loss"] - np.stack(losses, axis=1)).max() < 1e-10
    for name, leaf in (("dq", tq), ("dk", tk), ("dw", tw)):
        want = leaf.grad.numpy()
        assert np.abs(res[name] - want).max() <= 1e-10 * max(1.0, np.abs(want).max()), name


def pin_indexer_bwd_sets_sub_problems(orc):
    """Each index set's gradients are those of its own one-set problem (its
    heads' slice of q_idx and w, its index rows and teacher): dq and dw of the
    set's heads equal that problem's, and dk is the sum of the problems' dk."""
    q, k, w, q_offset, kv_len, idx, T, S = _ibwd_sets_problem(83)
    Hs = q.shape[2] // S
    tau = 0.02
    res = orc.indexer_bwd(q, k, w, q_offset, kv_len, idx, T, tau)
    dk = np.zeros_like(res["dk"])
    for g in range(S):
        hs = slice(g * Hs, (g + 1) * Hs)
        one = orc.indexer_bwd(np.ascontiguousarray(q[:, :, hs]), k, np.ascontiguousarray(w[:, :, hs]),
                              q_offset, kv_len, np.ascontiguousarray(idx[:, g]),
                              np.ascontiguousarray(T[:, g]), tau)
        assert np.array_equal(res["loss"][:, g], one["loss"])
        assert np.array_equal(res["dq"][:, :, hs], one["dq"])
        assert np.array_equal(res["dw"][:, :, hs], one["dw"])
        dk += one["dk"]
    assert np.abs(res["dk"] - dk).max() <= 1e-12 * max(1.0, np.abs(dk).max())


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
