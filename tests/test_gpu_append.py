"""GPU parity of the cache append and of the two flows it serves: chunked
prefill and a decode loop over a growing cache (the chunked prefill that reuses
the cached scorer inputs in "Hybrid Sparse Attention for Long-Context LLMs",
Engineering and Evaluation Recommendations).

The appended caches must equal the oracle's byte for byte; index rows of every
chunk and decode step must equal the oracle's one-shot layer bit for bit, and
outputs must be within the bf16 attention tolerance. The decode step is also
captured in a HIP graph (the library allocates nothing and sets no memory from
the host) and replayed against eager steps."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, dev, host, log

pytestmark = pytest.mark.gpu

MED = synth.CONFIGS["prefill8k"].replace(K=128, n_needles=0, needles="none")


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def _rows_of(a, starts, counts, C):
    """[B, C, ...] holding rows starts[b] .. starts[b] + counts[b] - 1 of a, zero padded."""
    out = np.zeros((a.shape[0], C) + a.shape[2:], a.dtype)
    for b in range(a.shape[0]):
        out[b, :counts[b]] = a[b, starts[b]:starts[b] + counts[b]]
    return out


@pytest.mark.parametrize("Hkv,d,d_I", [(4, 128, 64), (1, 64, 32), (8, 128, 128)])
def test_kv_append_matches_oracle(lci, orc, Hkv, d, d_I):
    import torch
    B, Tn, Tk = 4, 50, 300
    r = np.random.default_rng(20)
    kn = r.integers(0, 1 << 16, (B, Tn, Hkv, d), dtype=np.uint16)
    vn = r.integers(0, 1 << 16, (B, Tn, Hkv, d), dtype=np.uint16)
    kin = r.integers(-128, 128, (B, Tn, d_I), dtype=np.int8)
    kc = r.integers(0, 1 << 16, (B, Tk, Hkv, d), dtype=np.uint16)
    vc = r.integers(0, 1 << 16, (B, Tk, Hkv, d), dtype=np.uint16)
    kic = r.integers(-128, 128, (B, Tk, d_I), dtype=np.int8)
    # empty history, room for only part of the rows, a full cache, lengths outside 0..Tk
    for kv_len, n_new in (([0, 270, 300, 13], [50, 40, 7, 0]),
                          ([-5, 400, 299, 250], None),
                          ([3, 3, 3, 3], [-2, 60, 1, 50])):
        log(f"kv_append Hkv={Hkv} d={d} d_I={d_I} kv_len={kv_len} n_new={n_new}")
        kv_len = np.array(kv_len, np.int32)
        nn = None if n_new is None else np.array(n_new, np.int32)
        d_k, d_v, d_ki = dev(kc), dev(vc), dev(kic)
        qo, kl = lci.kv_append(dev(kn), dev(vn), dev(kin), d_k, d_v, d_ki, dev(kv_len),
                               n_new=dev(nn))
        torch.cuda.synchronize()
        for got, new, cache in ((d_k, kn, kc), (d_v, vn, vc), (d_ki, kin, kic)):
            want, wqo, wkl = orc.kv_append(new, cache, kv_len, nn)
            assert np.array_equal(host(got), want)
        assert host(qo).tolist() == wqo.tolist() and host(kl).tolist() == wkl.tolist()


def test_kv_append_lengths_in_place(lci, orc):
    import torch
    B, Tn, Tk, Hkv, d, d_I = 2, 3, 10, 2, 64, 32
    r = np.random.default_rng(21)
    kc = np.zeros((B, Tk, Hkv, d), np.uint16)
    kic = np.zeros((B, Tk, d_I), np.int8)
    d_k, d_v, d_ki = dev(kc), dev(kc), dev(kic)
    kv = dev(np.array([0, 5], np.int32))
    want_k, want_len = kc, np.array([0, 5], np.int32)
    for step in range(4):   # both sequences fill up (the second one first) and stop growing
        kn = r.integers(0, 1 << 16, (B, Tn, Hkv, d), dtype=np.uint16)
        kin = r.integers(-128, 128, (B, Tn, d_I), dtype=np.int8)
        qo, kl = lci.kv_append(dev(kn), dev(kn), dev(kin), d_k, d_v, d_ki, kv, kv_len_out=kv)
        torch.cuda.synchronize()
        want_k, wqo, wkl = orc.kv_append(kn, want_k, want_len)
        want_len = wkl
        assert kl.data_ptr() == kv.data_ptr()
        assert host(kv).tolist() == wkl.tolist() and host(qo).tolist() == wqo.tolist()
        assert np.array_equal(host(d_k), want_k) and np.array_equal(host(d_v), want_k)
    assert host(kv).tolist() == [10, 10]


def test_chunked_prefill(lci, orc):
    """Prefill in three chunks through append + prefill_fwd equals the one-shot
    layer; the second sequence appends fewer rows per chunk, so each of its
    chunks ends in rows past its history (invalid rows)."""
    import torch
    T = 900
    cfg = MED.replace(B=2, Tq=T, Tk=T)
    inp = synth.host_inputs(cfg, seed=22)
    inp["mix"] = synth.host_mix(cfg, seed=22)
    full = orc.layer(inp, cfg.K)
    d_k = dev(np.zeros_like(inp["k"]))
    d_v = dev(np.zeros_like(inp["v"]))
    d_ki = dev(np.zeros_like(inp["k_idx"]))
    kv = dev(np.zeros(2, np.int32))
    w = dev(inp["w"])
    start = np.zeros(2, np.int64)
    for C, n1 in ((300, 300), (350, 200), (250, 250)):
        n = np.array([C, n1], np.int32)
        log(f"chunked prefill: chunk of {C} rows, n_new={n.tolist()}")
        qo, kl = lci.kv_append(dev(_rows_of(inp["k"], start, n, C)),
                               dev(_rows_of(inp["v"], start, n, C)),
                               dev(_rows_of(inp["k_idx"], start, n, C)), d_k, d_v, d_ki, kv,
                               n_new=dev(n), kv_len_out=kv)
        out, idx = lci.prefill_fwd(dev(_rows_of(inp["q_idx"], start, n, C)), d_ki, w,
                                   dev(_rows_of(inp["q"], start, n, C)), d_k, d_v,
                                   dev(_rows_of(inp["gate"], start, n, C)), cfg.scale, qo, kl,
                                   cfg.K, want_idx=True,
                                   mix=dev(_rows_of(inp["mix"], start, n, C)))
        torch.cuda.synchronize()
        assert host(qo).tolist() == start.tolist()
        idx = host(idx)
        out = host(out)
        got_i, want_i, got_o, want_o = [], [], [], []
        for b in range(2):
            frows = slice(b * T + start[b], b * T + start[b] + n[b])
            got_i.append(idx[b, :n[b]])
            want_i.append(full["idx"][frows])
            got_o.append(out[b, :n[b]])
            want_o.append(full["out"][frows])
            assert (idx[b, n[b]:] == -1).all()
        assert np.array_equal(np.concatenate(got_i), np.concatenate(want_i))
        assert_attn_close(np.concatenate(got_o), np.concatenate(want_o), f"chunk {C}")
        start += n
    assert host(kv).tolist() == start.tolist()
    for got, name in ((d_k, "k"), (d_v, "v"), (d_ki, "k_idx")):
        h = host(got)
        for b in range(2):
            assert np.array_equal(h[b, :start[b]], inp[name][b, :start[b]])


def _decode_setup(lci, seed):
    """Three sequences with prompts of 2500, 1800 and 4000 rows already appended
    to caches of 4100 rows; returns the inputs, device caches and lengths."""
    T = 4100
    cfg = MED.replace(B=3, Tq=T, Tk=T, K=2048)
    inp = synth.host_inputs(cfg, seed=seed)
    P = np.array([2500, 1800, 4000], np.int32)
    caches = [dev(np.zeros_like(inp[n])) for n in ("k", "v", "k_idx")]
    kv = dev(np.zeros(3, np.int32))
    z = np.zeros(3, np.int64)
    lci.kv_append(dev(_rows_of(inp["k"], z, P, int(P.max()))),
                  dev(_rows_of(inp["v"], z, P, int(P.max()))),
                  dev(_rows_of(inp["k_idx"], z, P, int(P.max()))), *caches, kv, n_new=dev(P),
                  kv_len_out=kv)
    return cfg, inp, P, caches, kv


def test_decode_loop(lci, orc):
    """Six decode steps, each appending one token to the caches and decoding it,
    equal the one-shot layer's rows at those positions."""
    import torch
    cfg, inp, P, (d_k, d_v, d_ki), kv = _decode_setup(lci, seed=23)
    w = dev(inp["w"])
    qo = dev(np.zeros(3, np.int32))
    steps = 6
    got_i, got_o = [], []
    for s in range(steps):
        pos = P + s
        tok = lambda n: dev(_rows_of(inp[n], pos, np.ones(3, np.int32), 1))
        lci.kv_append(tok("k"), tok("v"), tok("k_idx"), d_k, d_v, d_ki, kv, q_offset_out=qo,
                      kv_len_out=kv)
        out, idx = lci.decode_fwd(tok("q_idx"), d_ki, w, tok("q"), d_k, d_v, tok("gate"),
                                  cfg.scale, qo, kv, cfg.K, want_idx=True)
        torch.cuda.synchronize()
        got_i.append(host(idx).reshape(3, cfg.K))
        got_o.append(host(out).reshape(3, cfg.Hq, cfg.d))
    log(f"decode loop: {steps} steps over prompts {P.tolist()}")
    rows = [[b, int(P[b]) + s] for s in range(steps) for b in range(3)]
    ref = orc.layer(inp, cfg.K, rows=rows)
    assert np.array_equal(np.concatenate(got_i), ref["idx"])
    assert_attn_close(np.concatenate(got_o), ref["out"], "decode loop")
    assert host(kv).tolist() == (P + steps).tolist()


def test_decode_step_graph_replay(lci):
    """One decode step (append the token, decode it) captured in a HIP graph and
    replayed for five tokens, with eager work and synchronisation between the
    replays, equals the same steps run eagerly on a second copy of the caches."""
    import torch
    cfg, inp, P, eager_c, eager_kv = _decode_setup(lci, seed=24)
    _, _, _, graph_c, graph_kv = _decode_setup(lci, seed=24)
    w = dev(inp["w"])
    one = np.ones(3, np.int32)
    names = ("k", "v", "k_idx", "q_idx", "q", "gate")
    static = {n: dev(_rows_of(inp[n], P, one, 1)) for n in names}
    qo = dev(np.zeros(3, np.int32))
    out = torch.empty_like(static["q"])
    idx = torch.empty((3, 1, cfg.K), dtype=torch.int32, device="cuda")
    geom = lci.make_geom(3, 1, cfg.Tk, cfg.K, qo, graph_kv, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
                         H_I=cfg.H_I, d_I=cfg.d_I)
    ws = torch.empty(lci.workspace_bytes(lci.ENTRY_DECODE, geom), dtype=torch.uint8,
                     device="cuda")

    def step(c, kv, tok, o, i, qoff, wsp, stream=None):
        lci.kv_append(tok["k"], tok["v"], tok["k_idx"], *c, kv, q_offset_out=qoff,
                      kv_len_out=kv, stream=stream)
        lci.decode_fwd(tok["q_idx"], c[2], w, tok["q"], c[0], c[1], tok["gate"], cfg.scale,
                       qoff, kv, cfg.K, out=o, idx_out=i, workspace=wsp, stream=stream)

    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(graph_c, graph_kv, static, out, idx, qo, ws, stream=side)
    torch.cuda.synchronize()
    # capturing launches nothing: the graph caches still hold the prompt only
    assert host(graph_kv).tolist() == P.tolist()
    for s in range(5):
        pos = P + s
        tok = {n: dev(_rows_of(inp[n], pos, one, 1)) for n in names}
        for n in names:
            static[n].copy_(tok[n])
        g.replay()
        torch.cuda.synchronize()
        eo = torch.empty_like(out)
        ei = torch.empty_like(idx)
        eqo = torch.empty_like(qo)
        step(eager_c, eager_kv, tok, eo, ei, eqo, None)
        torch.cuda.synchronize()
        log(f"graph replay {s}: kv_len {host(graph_kv).tolist()}")
        assert host(graph_kv).tolist() == host(eager_kv).tolist() == (pos + 1).tolist()
        assert np.array_equal(host(idx), host(ei))
        assert np.array_equal(host(out), host(eo))
    for a, b in zip(graph_c, eager_c):
        assert torch.equal(a, b)
