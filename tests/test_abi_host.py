"""The C-ABI library on the host: it loads, exports every symbol include/lci.h
declares, and rejects invalid arguments before touching a device. No kernel is
launched here (CPU only)."""
import ctypes
import os
import re

import pytest

import long_context_indexer_amd as lci

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lci.h")

OK, NULL, SHAPE, UNSUP, OVF, WS, HIP, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lci.LIB_PATH):
        from long_context_indexer_amd import build
        build.build()
    return lci.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lci_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lci_idx_score", "lci_topk_select", "lci_sparse_attn_fwd", "lci_prefill_fwd",
              "lci_decode_fwd", "lci_kv_append", "lci_sparse_attn_bwd", "lci_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(lci.EXPORTS) <= set(declared_functions())


def test_abi_version_and_status_strings(lib):
    assert lib.lci_abi_version() == lci.ABI_VERSION == 5
    for code in (OK, NULL, SHAPE, UNSUP, OVF, WS, HIP, ALIGN):
        assert lib.lci_status_str(code).decode().startswith("LCI_")
    assert b"unknown" in lib.lci_status_str(123)
    assert lib.lci_last_hip_error() == 0


def geom(**kw):
    base = dict(B=1, Tq=16, Tk=64, Hq=8, Hkv=2, d=128, H_I=8, d_I=64, K=8,
                q_offset=FAKE, kv_len=FAKE, block=0, sets=0)
    base.update(kw)
    return lci.lci_geom(base["B"], base["Tq"], base["Tk"], base["Hq"], base["Hkv"], base["d"],
                        base["H_I"], base["d_I"], base["K"], base["q_offset"], base["kv_len"],
                        base["block"], base["sets"])


def score(lib, g, q=FAKE, k=FAKE, w=FAKE, out=FAKE, wsb=0, wsq=0):
    return lib.lci_idx_score(ctypes.byref(g) if g is not None else None, q, k, w, wsb, wsq, out,
                             None)


def attn(lib, g, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, gate=None, mix=None, out=FAKE, ws=None, nb=0,
         scale=0.1):
    return lib.lci_sparse_attn_fwd(ctypes.byref(g), q, k, v, idx, gate, mix, scale, out, None, ws,
                                   nb, None)


def fused(lib, g, fn="lci_prefill_fwd", ws=FAKE, nb=None, scale=0.1, **ptrs):
    p = dict(qi=FAKE, ki=FAKE, w=FAKE, q=FAKE, k=FAKE, v=FAKE, gate=None, mix=None, out=FAKE)
    p.update(ptrs)
    if nb is None:
        nb = lib.lci_workspace_bytes(lci.ENTRY_PREFILL, ctypes.byref(g))
    return getattr(lib, fn)(ctypes.byref(g), p["qi"], p["ki"], p["w"], 0, 0, p["q"], p["k"], p["v"],
                            p["gate"], p["mix"], scale, p["out"], None, None, ws, nb, None)


def test_null_arguments(lib):
    assert score(lib, None) == NULL
    assert score(lib, geom(q_offset=None)) == NULL
    assert score(lib, geom(kv_len=None)) == NULL
    assert score(lib, geom(), q=None) == NULL
    assert score(lib, geom(), out=None) == NULL
    assert attn(lib, geom(), idx=None) == NULL
    assert fused(lib, geom(), v=None) == NULL
    assert lib.lci_topk_select(ctypes.byref(geom()), None, FAKE, None, None, 0, None) == NULL
    # the other branch's output is mixed in by the gate: without a gate it has no weight
    assert attn(lib, geom(), mix=FAKE) == NULL
    assert fused(lib, geom(), mix=FAKE) == NULL
    assert fused(lib, geom(Tq=1, Tk=1024), fn="lci_decode_fwd", mix=FAKE) == NULL


@pytest.mark.parametrize("field,value", [("B", 0), ("Tq", 0), ("Tk", 0), ("K", 0), ("K", 4097),
                                         ("Tq", -3)])
def test_shape_errors(lib, field, value):
    assert score(lib, geom(**{field: value})) == SHAPE


def test_indexer_limits(lib):
    assert score(lib, geom(H_I=16, d_I=128)) == OVF          # 2048 > 1024
    assert score(lib, geom(H_I=32, d_I=64)) == OVF
    assert score(lib, geom(H_I=3, d_I=64)) == UNSUP
    assert score(lib, geom(H_I=8, d_I=48)) == UNSUP
    assert score(lib, geom(H_I=0)) == SHAPE
    assert score(lib, geom(), wsb=-1) == SHAPE
    assert score(lib, geom(Tk=1 << 30, d_I=64)) == SHAPE     # Tk*d_I >= 2^31


def test_attention_limits(lib):
    assert attn(lib, geom(d=96)) == UNSUP
    assert attn(lib, geom(Hq=12, Hkv=8)) == SHAPE            # not a multiple
    assert attn(lib, geom(Hq=48, Hkv=16)) == UNSUP           # Hkv > 8
    assert attn(lib, geom(Hq=64, Hkv=2)) == UNSUP            # group of 32 query heads
    assert attn(lib, geom(Hq=6, Hkv=2)) == UNSUP             # group of 3


def test_block_granularity_limits(lib):
    assert score(lib, geom(block=-1)) == SHAPE
    assert score(lib, geom(block=3)) == UNSUP                 # not a power of two
    assert score(lib, geom(block=512)) == UNSUP
    assert score(lib, geom(block=64, K=65)) == SHAPE          # 4160 positions per row
    assert score(lib, geom(block=16, Tk=16 * 8192 + 1)) == UNSUP
    g = geom(block=64, K=64, Tk=8192)
    assert lib.lci_workspace_bytes(lci.ENTRY_PREFILL, ctypes.byref(g)) >= 16 * 4096 * 4
    gd = geom(Tq=1, block=64, K=32, Tk=1 << 17)
    assert lib.lci_workspace_bytes(lci.ENTRY_DECODE, ctypes.byref(gd)) > 0


def test_index_set_limits(lib):
    # query head h reads set h / (Hq/sets): the sets divide Hq (8); the indexer
    # heads (8) split evenly into them
    assert attn(lib, geom(sets=-1)) == SHAPE
    assert attn(lib, geom(sets=3)) == SHAPE                   # does not divide Hq
    assert attn(lib, geom(sets=16)) == SHAPE                  # more sets than query heads
    assert fused(lib, geom(sets=2, H_I=1, d_I=64)) == SHAPE   # 1 indexer head for 2 sets
    assert fused(lib, geom(sets=8, H_I=4, d_I=64)) == SHAPE   # 4 indexer heads for 8 sets
    assert score(lib, geom(sets=3)) == SHAPE
    assert score(lib, geom(sets=16)) == SHAPE
    assert lib.lci_topk_select(ctypes.byref(geom(sets=-1)), FAKE, FAKE, None, None, 0,
                               None) == SHAPE
    for sets in (2, 4, 8):   # per key/value head, between, per query head
        g = geom(sets=sets, Tk=4096, K=64)
        need = lib.lci_workspace_bytes(lci.ENTRY_PREFILL, ctypes.byref(g))
        assert need >= sets * 16 * 64 * 4                     # index rows of every set
        assert lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN, ctypes.byref(g)) > 0
        assert fused(lib, g, nb=need - 1) == WS


def test_backward_arguments(lib):
    def bwd(g, dgate=None, dmix=None, gate=None, mix=None, ws=FAKE, nb=None, dq=FAKE):
        if nb is None:
            nb = lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN_BWD, ctypes.byref(g))
        return lib.lci_sparse_attn_bwd(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, gate, mix, FAKE,
                                       0.1, dq, FAKE, FAKE, dgate, dmix, ws, nb, None)
    assert bwd(geom(), dq=None) == NULL
    assert bwd(geom(), dgate=FAKE) == NULL                     # dgate without a gate
    assert bwd(geom(), gate=FAKE, dmix=FAKE) == NULL          # dmix without a mix
    assert bwd(geom(sets=3)) == SHAPE                         # does not divide Hq
    assert bwd(geom(sets=16)) == SHAPE                        # more sets than query heads
    two = lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN_BWD, ctypes.byref(geom(sets=2)))
    per_head = lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN_BWD, ctypes.byref(geom(sets=8)))
    assert per_head > two > 0                                 # position lists per set
    assert bwd(geom(), nb=16) == WS
    assert bwd(geom(), ws=None) == WS
    assert bwd(geom(), dq=FAKE + 4) == ALIGN
    g = geom(B=2, Tq=64, Tk=4096, K=64)
    assert lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN_BWD, ctypes.byref(g)) >= 2 * 64 * 64 * 4


def test_softmax_scale_must_be_positive(lib):
    # running maxima are taken on raw dot products: only a positive scale keeps them maxima
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert attn(lib, geom(), scale=bad) == SHAPE
        assert fused(lib, geom(), scale=bad) == SHAPE


def test_alignment(lib):
    assert attn(lib, geom(), q=FAKE + 2) == ALIGN
    assert attn(lib, geom(), gate=FAKE + 8) == ALIGN
    assert attn(lib, geom(), gate=FAKE, mix=FAKE + 8) == ALIGN
    assert fused(lib, geom(), gate=FAKE, mix=FAKE + 2) == ALIGN
    assert score(lib, geom(), q=FAKE + 4) == ALIGN
    assert score(lib, geom(), out=FAKE + 2) == ALIGN
    assert score(lib, geom(q_offset=FAKE + 2)) == ALIGN


def test_workspace_checks(lib):
    g = geom(B=2, Tq=64, Tk=4096, K=64)
    need = lib.lci_workspace_bytes(lci.ENTRY_PREFILL, ctypes.byref(g))
    assert need >= 2 * 64 * 64 * 4          # at least the index rows
    assert fused(lib, g, nb=need - 1) == WS
    assert fused(lib, g, ws=None) == WS
    assert fused(lib, g, ws=FAKE + 8, nb=need) == ALIGN
    gd = geom(B=4, Tq=1, Tk=1 << 16, K=2048)
    needd = lib.lci_workspace_bytes(lci.ENTRY_DECODE, ctypes.byref(gd))
    assert needd > 0
    assert fused(lib, gd, fn="lci_decode_fwd", nb=needd - 1) == WS
    # split-K attention of few long rows needs partials
    need_a = lib.lci_workspace_bytes(lci.ENTRY_SPARSE_ATTN, ctypes.byref(gd))
    assert need_a > 0
    assert attn(lib, gd, ws=None) == WS
    assert attn(lib, gd, ws=FAKE, nb=need_a - 4) == WS
    assert lib.lci_workspace_bytes(99, ctypes.byref(g)) == 0
    assert lib.lci_workspace_bytes(lci.ENTRY_PREFILL, ctypes.byref(geom(K=0))) == 0
    assert lib.lci_workspace_bytes(lci.ENTRY_IDX_SCORE, ctypes.byref(g)) == 0


def append(lib, g, n_new=None, qo=FAKE, kl=FAKE + 64, **ptrs):
    p = dict(kn=FAKE, vn=FAKE, kin=FAKE, kc=FAKE, vc=FAKE, kic=FAKE)
    p.update(ptrs)
    return lib.lci_kv_append(ctypes.byref(g) if g is not None else None, p["kn"], p["vn"], p["kin"],
                             n_new, p["kc"], p["vc"], p["kic"], qo, kl, None)


def test_kv_append_arguments(lib):
    assert append(lib, None) == NULL
    assert append(lib, geom(kv_len=None)) == NULL
    assert append(lib, geom(q_offset=None), kc=None) == NULL
    assert append(lib, geom(q_offset=None), kin=None) == NULL
    assert append(lib, geom(B=0)) == SHAPE
    assert append(lib, geom(B=65536)) == SHAPE
    assert append(lib, geom(Tq=0)) == SHAPE
    assert append(lib, geom(d_I=0)) == SHAPE
    assert append(lib, geom(), qo=FAKE, kl=FAKE) == SHAPE      # both outputs in one array
    assert append(lib, geom(Hkv=1, d=4)) == UNSUP               # 8-byte rows
    assert append(lib, geom(d_I=40)) == UNSUP
    assert append(lib, geom(), kc=FAKE + 8) == ALIGN
    assert append(lib, geom(), n_new=FAKE + 2) == ALIGN
    assert append(lib, geom(kv_len=FAKE + 2)) == ALIGN


def test_decode_needs_one_row(lib):
    g = geom(Tq=2, Tk=1024)
    assert fused(lib, g, fn="lci_decode_fwd") == SHAPE


def test_kernel_timing_log_on_the_host(lib):
    # switching the log on and off touches no device; reads validate their arguments
    assert [lci.kernel_name(k) for k in range(len(lci.KERNELS))] == list(lci.KERNELS)
    assert lib.lci_kernel_name(len(lci.KERNELS)) is None
    assert lib.lci_kernel_timing(1) == OK
    assert lci.kernel_timing_read("attn_dense") == (0.0, 0)
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.lci_kernel_timing_read(99, ctypes.byref(ms), ctypes.byref(n)) == SHAPE
    assert lib.lci_kernel_timing_read(0, None, ctypes.byref(n)) == NULL
    assert lib.lci_kernel_timing(0) == OK


def test_attn_overlap_modes(lib):
    """The schedule switch takes the three modes and refuses others (it only
    sets a process-wide value: no stream or device is touched here)."""
    for m in (lci.OVERLAP_OFF, lci.OVERLAP_ON, lci.OVERLAP_AUTO):
        assert lib.lci_attn_overlap(m) == 0
    assert lib.lci_attn_overlap(3) == SHAPE
    assert lib.lci_attn_overlap(-1) == SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    z = torch.zeros(1, 4, 2, 32, dtype=torch.int8)
    with pytest.raises((ValueError, RuntimeError)):
        lci.idx_score(z, torch.zeros(1, 4, 32, dtype=torch.int8), torch.ones(2, dtype=torch.int8),
                      torch.zeros(1, dtype=torch.int32), torch.ones(1, dtype=torch.int32))


def test_dense_row_limit(lib):
    def lim(entry, g):
        return lib.lci_dense_row_limit(entry, ctypes.byref(g))
    g = geom(B=1, Tq=65536, Tk=65536, Hq=32, Hkv=4, K=2048)
    assert lim(lci.ENTRY_PREFILL, g) == lim(lci.ENTRY_SPARSE_ATTN, g) == 16 * 2048
    assert lim(lci.ENTRY_PREFILL, geom(B=1, Tq=4096, Tk=4096, K=2048)) == 4096   # whole history
    assert lim(lci.ENTRY_DECODE, geom(B=64, Tq=1, Tk=1 << 17, K=2048)) == 0     # split-K decode
    assert lim(lci.ENTRY_PREFILL, geom(B=2, Tq=8, Tk=4096, K=2048)) == 0        # few rows
    assert lim(lci.ENTRY_IDX_SCORE, g) == 0
    assert lim(lci.ENTRY_PREFILL, geom(d=96)) == 0                              # invalid


def test_decode_noalloc_arguments(lib):
    """The allocation-free decode refuses, before touching any device, a geometry
    whose workspace exceeds its static scratch array, and passes every other
    argument error through from the decode entry."""
    SCRATCH = -8
    cap = lib.lci_noalloc_scratch_bytes()
    assert cap == 128 << 20

    def call(g, q=FAKE):
        return lib.lci_decode_fwd_noalloc(ctypes.byref(g), FAKE, FAKE, FAKE, 0, 0, q, FAKE, FAKE,
                                          FAKE, None, 0.1, FAKE, None, None, None)
    big = geom(B=128, Tq=1, Tk=1 << 17, Hq=32, Hkv=4, K=2048)
    assert lib.lci_workspace_bytes(lci.ENTRY_DECODE, ctypes.byref(big)) > cap
    assert call(big) == SCRATCH
    assert b"scratch" in lib.lci_status_str(SCRATCH)
    for fits in (geom(B=64, Tq=1, Tk=1 << 17, Hq=32, Hkv=4, K=2048),
                 geom(B=8, Tq=1, Tk=1 << 20, Hq=32, Hkv=4, K=2048)):
        assert 0 < lib.lci_workspace_bytes(lci.ENTRY_DECODE, ctypes.byref(fits)) <= cap
    assert call(geom(Tq=2)) == SHAPE                      # decode takes one row per sequence
    assert call(geom(Tq=1), q=None) == NULL
    assert lib.lci_decode_fwd_noalloc(None, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, None,
                                      0.1, FAKE, None, None, None) == NULL


def test_indexer_bwd_arguments(lib):
    def call(g, q=FAKE, teacher=FAKE, tau=0.01, ws=FAKE, nb=None, dq=FAKE):
        if nb is None:
            nb = lib.lci_workspace_bytes(lci.ENTRY_INDEXER_BWD, ctypes.byref(g))
        return lib.lci_indexer_bwd(ctypes.byref(g), q, FAKE, FAKE, 0, 0, FAKE, teacher, tau, None,
                                   dq, FAKE, FAKE, ws, nb, None)
    g = geom(B=2, Tq=16, Tk=300, H_I=8, d_I=64, K=32)
    # per entry g (4 B), masks (2 B) and its number in its position's list (4 B);
    # per position a count, an offset and a cursor
    need = lib.lci_workspace_bytes(lci.ENTRY_INDEXER_BWD, ctypes.byref(g))
    assert need >= 2 * 16 * 32 * 10 + 2 * 300 * 12
    assert call(g, q=None) == NULL
    assert call(g, teacher=None) == NULL
    assert call(g, tau=float("inf")) == SHAPE
    assert call(g, tau=float("nan")) == SHAPE
    assert call(geom(H_I=32, d_I=64)) == OVF
    # index sets: S must divide H_I; the sets share one workspace (no larger than
    # one set's), so validation is all a host test can call
    g8 = dict(B=2, Tq=16, Tk=300, H_I=8, d_I=64, K=32)
    assert call(geom(**g8, sets=3)) == SHAPE
    assert call(geom(**g8, sets=-1)) == SHAPE
    one = lib.lci_workspace_bytes(lci.ENTRY_INDEXER_BWD, ctypes.byref(geom(**g8)))
    two = lib.lci_workspace_bytes(lci.ENTRY_INDEXER_BWD, ctypes.byref(geom(**g8, sets=2)))
    assert 0 < two <= one
    assert lib.lci_workspace_bytes(lci.ENTRY_INDEXER_BWD, ctypes.byref(geom(**g8, sets=3))) == 0
    assert call(g, nb=8) == WS
    assert call(g, ws=None) == WS
    assert call(g, dq=FAKE + 4) == ALIGN
