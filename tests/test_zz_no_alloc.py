"""The allocation-free fused decode (lci_decode_fwd_noalloc, workspace in the
library's static per-device scratch array) against the fused decode with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller geometry (so its workspace regions overlap what the first left in the
scratch array), index rows, outputs and lse bit-identical. The caller
workspace of the reference call is filled with a byte pattern first, so a
kernel that read a workspace byte it had not written would show up as a
difference."""
import numpy as np
import pytest

import synth
from gpu_util import host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lci():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_indexer_amd as m
    m.load_library()
    return m


def ragged(cfg, d, step):
    """History lengths Tk, Tk - step, Tk - 2*step, ...; the query at the last position."""
    import torch
    kvl = np.array([cfg.Tk - step * b for b in range(cfg.B)], np.int32)
    d["kv_len"] = torch.from_numpy(kvl).cuda()
    d["q_offset"] = torch.from_numpy(kvl - 1).cuda()
    return d


def test_decode_noalloc_matches_decode(lci):
    import torch
    base = synth.CONFIGS["decode128k"]
    cases = [(base.replace(B=64), 0, 37, False), (base.replace(B=3, Tk=20000), 1, 1111, True)]
    for call, (cfg, seed, step, with_mix) in enumerate(cases):
        d = ragged(cfg, synth.device_inputs(cfg, seed=seed), step)
        mix = torch.randn(d["q"].shape, device="cuda").to(torch.bfloat16) if with_mix else None
        geom = lci.make_geom(cfg.B, 1, cfg.Tk, cfg.K, d["q_offset"], d["kv_len"], Hq=cfg.Hq,
                             Hkv=cfg.Hkv, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I)
        need = lci.workspace_bytes(lci.ENTRY_DECODE, geom)
        assert 0 < need <= lci.noalloc_scratch_bytes()
        log(f"noalloc call {call}: B={cfg.B} Tk={cfg.Tk} workspace {need / 2**20:.1f} MiB, "
            f"mix={with_mix}")
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
        args = (d["q_idx"], d["k_idx"], d["w"], d["q"], d["k"], d["v"], d["gate"], d["scale"],
                d["q_offset"], d["kv_len"], cfg.K)
        ref_out, ref_idx, ref_lse = lci.decode_fwd(*args, want_idx=True, want_lse=True,
                                                   workspace=ws, mix=mix)
        out, idx, lse = lci.decode_fwd_noalloc(*args, want_idx=True, want_lse=True, mix=mix)
        torch.cuda.synchronize()
        assert (host(idx) == host(ref_idx)).all(), call
        assert (host(out) == host(ref_out)).all(), call
        assert (host(lse).view(np.uint32) == host(ref_lse).view(np.uint32)).all(), call
        assert (host(idx)[:, 0, :] >= 0).all()
        log(f"noalloc call {call}: index rows, outputs and lse bit-identical")
        del d, ws
        torch.cuda.empty_cache()
