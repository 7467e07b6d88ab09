"""GPU parity of block-granular selection (the pages' "positions or blocks":
"Hybrid Sparse Attention for Long-Context LLMs", Indexer + Top-K section, steps
1-2). The kept blocks, their scores and the expanded index rows must equal the
oracle's bit for bit; attention outputs through the fused entries must be
within the bf16 tolerance."""
import numpy as np
import pytest

import synth
from gpu_util import assert_attn_close, dev, host, log, to_device

pytestmark = pytest.mark.gpu

I32_MIN = np.iinfo(np.int32).min
LSE_TOL = 1e-4
MED = synth.CONFIGS["prefill8k"].replace(Tq=640, Tk=640, K=16, n_needles=8)


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


# (B, Tq, Tk, q_offset, kv_len, K blocks, block, score range)
SELECT_CASES = {
    "b2_ties": (2, 40, 300, [0, 250], [300, 290], 20, 2, 3),
    "b16_ragged_invalid": (3, 30, 900, [0, 880, 400], [900, 890, 410], 8, 16, 1000),
    "b64_all_equal": (1, 20, 5000, [4980], [5000], 10, 64, 0),
    "b64_more_blocks_than_exist": (2, 16, 700, [0, 600], [700, 616], 64, 64, 50),
    "b256_long": (1, 8, 40000, [39990], [40000], 16, 256, 100000),
    "b16_max_blocks": (1, 4, 16 * 8192, [16 * 8192 - 4], [16 * 8192], 128, 16, 7),
    "b8_k512": (1, 12, 6000, [5988], [6000], 512, 8, 2),
    # rows not 16-byte aligned (Tk not a multiple of 4): the scalar load path
    "b8_unaligned_rows": (2, 10, 1001, [991, 500], [1001, 700], 16, 8, 20),
    "b2_unaligned_rows": (1, 9, 333, [324], [333], 40, 2, 5),
}


@pytest.mark.parametrize("name", list(SELECT_CASES))
def test_block_topk_bit_exact(lci, orc, name):
    import torch
    B, Tq, Tk, qo, kl, K, block, rng = SELECT_CASES[name]
    log(f"block topk {name}: B={B} Tq={Tq} Tk={Tk} K={K} block={block}")
    r = np.random.default_rng(30)
    S = (r.integers(-rng, rng + 1, (B, Tq, Tk)) * 3).astype(np.int32)
    qo = np.array(qo, np.int32)
    kl = np.array(kl, np.int32)
    idx, sel = lci.topk_select(dev(S), K, dev(qo), dev(kl), want_scores=True, block=block)
    torch.cuda.synchronize()
    n = np.array([qo[b] + i + 1 if qo[b] + i < kl[b] else 0 for b in range(B) for i in range(Tq)])
    widx, wblk, wsel = orc.block_topk(S.reshape(B * Tq, Tk), n, K, block)
    assert np.array_equal(host(idx).reshape(B * Tq, K * block), widx)
    assert np.array_equal(host(sel).reshape(B * Tq, K), wsel)


FUSED_CASES = {
    # blocks of 16, 16 kept (256 positions) on 640-row sequences, with the gate mix
    "b16_prefill_mix": (MED, 16, dict(), True),
    # continuation rows and an invalid row, blocks of 64
    "b64_ragged": (MED.replace(B=2, Tq=96, Tk=700, K=4), 64,
                   dict(q_offset=[604, 300], kv_len=[700, 396]), False),
    # every causal position kept (K*block >= p+1): dense-equivalent rows
    "b256_dense": (MED.replace(Tq=300, Tk=300, K=2), 256, dict(), False),
}


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_block_prefill_fused(lci, orc, name):
    import torch
    cfg, block, kw, mix = FUSED_CASES[name]
    inp = synth.host_inputs(cfg, seed=31)
    for k_, v_ in kw.items():
        inp[k_] = np.asarray(v_, np.int32)
    if mix:
        inp["mix"] = synth.host_mix(cfg, seed=31)
    log(f"block prefill {name}: B={cfg.B} Tq={cfg.Tq} Tk={cfg.Tk} K={cfg.K} block={block}")
    d = to_device(inp)
    out, idx, lse = lci.prefill_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                    d["gate"], inp["scale"], d["q_offset"], d["kv_len"], cfg.K,
                                    want_idx=True, want_lse=True, mix=d.get("mix"), block=block)
    torch.cuda.synchronize()
    res = orc.layer(inp, cfg.K, block=block)
    assert np.array_equal(host(idx).reshape(cfg.B * cfg.Tq, -1), res["idx"])
    assert_attn_close(host(out).reshape(res["out"].shape), res["out"], name)
    lse = host(lse).reshape(-1, cfg.Hq)
    fin = np.isfinite(res["lse"])
    assert (np.isfinite(lse) == fin).all()
    assert np.abs(lse[fin] - res["lse"][fin]).max() < LSE_TOL


def test_block_decode_fused(lci, orc):
    """Decode rows with blocks of 64 (the prefill path on one row per sequence):
    ragged histories, one shorter than K blocks, one invalid."""
    import torch
    L = 20000
    cfg = MED.replace(B=4, Tq=1, Tk=L, decode=True, K=32, needles="decode", n_needles=6)
    inp = synth.host_inputs(cfg, seed=32)
    inp["kv_len"] = np.array([L, L - 77, 1500, 900], np.int32)
    inp["q_offset"] = np.array([L - 1, L - 78, 1499, 900], np.int32)
    log("block decode B=4 L=20000 K=32 block=64")
    d = to_device(inp)
    out, idx, lse = lci.decode_fwd(d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"],
                                   d["gate"], inp["scale"], d["q_offset"], d["kv_len"], cfg.K,
                                   want_idx=True, want_lse=True, block=64)
    torch.cuda.synchronize()
    res = orc.layer(inp, cfg.K, block=64)
    assert np.array_equal(host(idx).reshape(cfg.B, -1), res["idx"])
    assert_attn_close(host(out).reshape(res["out"].shape), res["out"], "block decode")
    assert (res["idx"][3] == -1).all()
