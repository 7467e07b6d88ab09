"""Full-size parity on the five workload configurations, through the fused entry
points exactly as the benchmark launches them.

Every row of every workload is checked against properties that hold at any
size (index rows ascending, inside 0..p, min(K, p+1) entries, rows with p < K
equal 0..p). Beyond that the oracle recomputes, and the test compares element
by element (index rows bit-exact, outputs within the bf16 tolerance over all
compared rows):

  * Prefill 8K: all 8192 rows.
  * Decode 128K: all 64 sequences; Decode 1M: all 8 sequences. The oracle
    scores each whole history and selects on the host; the attention is then
    recomputed on the key/value rows the oracle itself selected (copied out of
    device memory by position: attention does not depend on where a row sits).
  * Prefill 64K: two whole blocks of 4096 rows (rows 4096..12287: rows the
    long-prefill selection finishes from their candidate lists, sampled and
    listed-whole rows alike), plus 32 rows of every other block (its first
    and last rows and 30 drawn at random), 8640 rows in all. The first and
    last rows of the blocks include rows 32767 and 32768, the last row the
    dense-tile path takes (p + 1 <= 16 K) and the first the gather path takes.

Planted needle recall is reported."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, host, log

pytestmark = pytest.mark.gpu

# query rows per score block of the fused prefill at Prefill 64K (1 GiB of int32 rows)
BLOCK_ROWS_64K = 4096


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def check_index_rows(idx, q_offset, kv_len, K):
    """Properties every index row has: ascending valid positions, then -1 padding."""
    import torch
    B, Tq, _ = idx.shape
    pos = q_offset.view(B, 1).long() + torch.arange(Tq, device=idx.device).view(1, Tq)
    n_valid = torch.clamp(pos + 1, max=K)
    j = torch.arange(K, device=idx.device).view(1, 1, K)
    valid = j < n_valid.unsqueeze(-1)
    assert ((idx >= 0) == valid).all()
    assert (idx <= pos.unsqueeze(-1)).all()
    d = idx[:, :, 1:] - idx[:, :, :-1]
    assert ((d > 0) | ~valid[:, :, 1:]).all()
    dense = pos < K                                    # every position kept
    if dense.any():
        want = torch.where(valid, j.expand_as(idx), torch.full_like(idx, -1))
        assert (idx[dense] == want[dense]).all()


def run_fused(lci, cfg, d, entry):
    import torch
    fn = lci.prefill_fwd if entry == "prefill" else lci.decode_fwd
    log(f"{cfg.name}: launching {entry}_fwd B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk}")
    out, idx = fn(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"], d["scale"],
                  d["q_offset"], d["kv_len"], cfg.K, want_idx=True)
    torch.cuda.synchronize()
    check_index_rows(idx, d["q_offset"], d["kv_len"], cfg.K)
    log(f"{cfg.name}: index-row properties hold on all {cfg.B * cfg.Tq} rows")
    return out, idx


def compare_rows(name, got_idx, want_idx, got_out, want_out):
    """Element-by-element comparison of the compared rows: index rows bit-exact
    (the first differing row is named), outputs within the bf16 tolerance."""
    bad = np.nonzero((got_idx != want_idx).any(axis=-1))[0]
    assert bad.size == 0, (name, f"{bad.size} index rows differ, first at compared row {bad[0]}")
    assert_attn_close(got_out, want_out, f"{name}: {got_idx.shape[0]} rows")
    log(f"{name}: index rows bit-exact and outputs within tolerance on "
        f"{got_idx.shape[0]} compared rows")


def needle_recall(idx_host_rows, needles):
    """idx_host_rows(b, t) -> host index row of query row t of sequence b."""
    hit = tot = 0
    for b, plan in enumerate(needles):
        for p, t in plan:
            tot += 1
            hit += int((idx_host_rows(b, t) == p).any())
    return hit, tot


def host_inputs_of(d):
    return {k: (host(v) if hasattr(v, "device") else v) for k, v in d.items()}


def test_prefill8k_all_rows(lci, orc):
    cfg = synth.CONFIGS["prefill8k"]
    inp = synth.host_inputs(cfg, seed=0)
    from gpu_util import to_device
    d = to_device(inp)
    out, idx = run_fused(lci, cfg, d, "prefill")
    ref = orc.layer(inp, cfg.K)
    gi = host(idx).reshape(-1, cfg.K)
    compare_rows("prefill8k", gi, ref["idx"], host(out).reshape(ref["out"].shape[0], -1),
                 ref["out"].reshape(ref["out"].shape[0], -1))
    hit, tot = needle_recall(lambda b, t: gi[t], inp["needles"])
    log(f"prefill8k needle recall {hit}/{tot}")


def prefill64k_rows(Tq, seed=1):
    """Rows 4096..12287 whole, and 32 rows of every other 4096-row block."""
    r = np.random.default_rng(seed)
    rows = set(range(BLOCK_ROWS_64K, 3 * BLOCK_ROWS_64K))
    for blk in range(Tq // BLOCK_ROWS_64K):
        lo, hi = blk * BLOCK_ROWS_64K, (blk + 1) * BLOCK_ROWS_64K
        if lo >= BLOCK_ROWS_64K and hi <= 3 * BLOCK_ROWS_64K:
            continue
        inner = r.choice(np.arange(lo + 1, hi - 1), 30, replace=False)
        rows.update([lo, hi - 1, *inner.tolist()])
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_prefill64k_blocks(lci, orc):
    cfg = synth.CONFIGS["prefill64k"]
    d = synth.device_inputs(cfg, seed=0)
    out, idx = run_fused(lci, cfg, d, "prefill")
    rows = prefill64k_rows(cfg.Tq)
    inp = host_inputs_of(d)
    log(f"prefill64k: oracle on {len(rows)} rows")
    ref = orc.layer(inp, cfg.K, rows=[(0, int(i)) for i in rows])
    gi_all = host(idx)[0]
    gi = gi_all[rows]
    go = host(out)[0][rows].reshape(len(rows), -1)
    compare_rows("prefill64k", gi, ref["idx"], go, ref["out"].reshape(len(rows), -1))
    hit, tot = needle_recall(lambda b, t: gi_all[t], d["needles"])
    log(f"prefill64k needle recall {hit}/{tot}")


def decode_all_sequences(lci, orc, cfg, d):
    """Every sequence of a decode workload against the oracle: the oracle scores
    each whole history and selects; the attention is recomputed by the oracle on
    the key/value rows at the positions the oracle selected."""
    import torch
    out, idx = run_fused(lci, cfg, d, "decode")
    B, K = cfg.B, cfg.K
    qo = host(d["q_offset"]).astype(np.int64)
    S = orc.scores(host(d["q_idx"]), host(d["k_idx"]), host(d["w"]), host(d["q_offset"]),
                   host(d["kv_len"]))
    want_idx, _ = orc.topk(S, qo + 1, K)
    del S
    got_idx = host(idx).reshape(B, K)
    bad = np.nonzero((got_idx != want_idx).any(axis=-1))[0]
    assert bad.size == 0, (cfg.name, f"{bad.size} sequences' index rows differ, first {bad[0]}")
    n_sel = np.minimum(qo + 1, K)
    assert (n_sel == K).all()
    sel = torch.from_numpy(want_idx.astype(np.int64)).to(d["k"].device)
    ks = torch.stack([d["k"][b].index_select(0, sel[b]) for b in range(B)])
    vs = torch.stack([d["v"][b].index_select(0, sel[b]) for b in range(B)])
    local = np.broadcast_to(np.arange(K, dtype=np.int32), (B, K))
    ref_out, _ = orc.attention(host(d["q"]), host(ks), host(vs), host(d["gate"]), local,
                               np.full(B, K, np.int32), d["scale"])
    compare_rows(cfg.name, got_idx, want_idx, host(out).reshape(B, -1), ref_out.reshape(B, -1))
    return got_idx


@pytest.mark.timeout(600)
def test_decode128k_all_sequences(lci, orc):
    cfg = synth.CONFIGS["decode128k"]
    d = synth.device_inputs(cfg, seed=0)
    decode_all_sequences(lci, orc, cfg, d)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_decode1m_all_sequences(lci, orc):
    cfg = synth.CONFIGS["decode1m"]
    d = synth.device_inputs(cfg, seed=0)
    gi = decode_all_sequences(lci, orc, cfg, d)
    hit, tot = needle_recall(lambda b, t: gi[b], d["needles"])
    log(f"decode1m needle recall {hit}/{tot}")
