"""Gated fine-grained sparse attention for AMD MI355X (gfx950).

A thin ctypes binding over liblci.so, the HIP library whose C ABI is declared in
include/lci.h. Every step of the layer (indexer scoring, Top-K selection, sparse
attention, sigmoid gate and its mix with another branch) runs in the library's
kernels; this module only checks tensor dtypes/shapes/contiguity, passes device
pointers and the current HIP stream, and turns status codes into exceptions.
PyTorch supplies device memory and streams. There is no CPU fallback: without
the built library every call raises.

Entry points (same names as the C ABI, without the ``lci_`` prefix):
    idx_score, topk_select, sparse_attn_fwd, prefill_fwd, decode_fwd, decode_fwd_noalloc,
    kv_append, sparse_attn_bwd, indexer_bwd,
    workspace_bytes, dense_row_limit, kernel_timing, kernel_timing_read, kernel_name
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblci.so")

(ENTRY_IDX_SCORE, ENTRY_TOPK_SELECT, ENTRY_SPARSE_ATTN, ENTRY_PREFILL, ENTRY_DECODE,
 ENTRY_SPARSE_ATTN_BWD, ENTRY_INDEXER_BWD) = range(7)

# LCI_ABI_VERSION of the signatures declared below
ABI_VERSION = 5

EXPORTS = ("lci_idx_score", "lci_topk_select", "lci_sparse_attn_fwd", "lci_prefill_fwd",
           "lci_decode_fwd", "lci_kv_append", "lci_sparse_attn_bwd", "lci_workspace_bytes",
           "lci_dense_row_limit", "lci_indexer_bwd", "lci_decode_fwd_noalloc", "lci_noalloc_scratch_bytes",
           "lci_status_str", "lci_last_hip_error",
           "lci_abi_version", "lci_kernel_timing", "lci_kernel_timing_read", "lci_kernel_name",
           "lci_attn_overlap", "lci_attn_overlap_forks")

# schedules of lci_attn_overlap (LCI_OVERLAP_* in lci.h)
OVERLAP_AUTO, OVERLAP_OFF, OVERLAP_ON = range(3)

# kernel kinds of the timing log (LCI_KERNEL_* in lci.h)
KERNELS = ("idx_score", "topk", "idx_mask", "attn_dense", "attn_gather", "attn_combine",
           "dec_sample", "dec_thresh", "dec_score", "dec_select", "kv_append",
           "kv_lengths", "bwd_prologue", "bwd_dq", "bwd_transpose", "bwd_dkdv", "sel_scan",
           "sel_rows", "sel_fallback", "ibwd_rows", "ibwd_transpose", "ibwd_dk")


class LciError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class lci_geom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("H_I", ctypes.c_int32), ("d_I", ctypes.c_int32), ("K", ctypes.c_int32),
                ("q_offset", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
                ("block", ctypes.c_int32), ("sets", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblci.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m long_context_indexer_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    G = ctypes.POINTER(lci_geom)
    lib.lci_idx_score.argtypes = [G, P, P, P, i64, i64, P, P]
    lib.lci_topk_select.argtypes = [G, P, P, P, P, sz, P]
    lib.lci_sparse_attn_fwd.argtypes = [G, P, P, P, P, P, P, ctypes.c_float, P, P, P, sz, P]
    fused = [G, P, P, P, i64, i64, P, P, P, P, P, ctypes.c_float, P, P, P, P, sz, P]
    lib.lci_prefill_fwd.argtypes = fused
    lib.lci_decode_fwd.argtypes = fused
    lib.lci_decode_fwd_noalloc.argtypes = fused[:-3] + [P]
    lib.lci_decode_fwd_noalloc.restype = ctypes.c_int
    lib.lci_noalloc_scratch_bytes.restype = sz
    lib.lci_kv_append.argtypes = [G, P, P, P, P, P, P, P, P, P, P]
    lib.lci_sparse_attn_bwd.argtypes = [G, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P,
                                        P, sz, P]
    lib.lci_indexer_bwd.argtypes = [G, P, P, P, i64, i64, P, P, ctypes.c_float, P, P, P, P, P,
                                    sz, P]
    lib.lci_indexer_bwd.restype = ctypes.c_int
    lib.lci_workspace_bytes.argtypes = [ctypes.c_int, G]
    lib.lci_workspace_bytes.restype = sz
    lib.lci_dense_row_limit.argtypes = [ctypes.c_int, G]
    lib.lci_dense_row_limit.restype = ctypes.c_int
    lib.lci_status_str.argtypes = [ctypes.c_int]
    lib.lci_status_str.restype = ctypes.c_char_p
    lib.lci_last_hip_error.restype = ctypes.c_int
    lib.lci_abi_version.restype = ctypes.c_int
    if lib.lci_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.lci_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it")
    lib.lci_kernel_timing.argtypes = [ctypes.c_int]
    lib.lci_kernel_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int64)]
    lib.lci_kernel_name.argtypes = [ctypes.c_int]
    lib.lci_attn_overlap.argtypes = [ctypes.c_int]
    lib.lci_attn_overlap.restype = ctypes.c_int
    lib.lci_attn_overlap_forks.restype = ctypes.c_longlong
    lib.lci_kernel_name.restype = ctypes.c_char_p
    for fn in ("lci_idx_score", "lci_topk_select", "lci_sparse_attn_fwd", "lci_prefill_fwd",
               "lci_decode_fwd", "lci_kv_append", "lci_sparse_attn_bwd", "lci_kernel_timing", "lci_kernel_timing_read"):
        getattr(lib, fn).restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        msg = lib.lci_status_str(rc).decode()
        if rc == -6:
            msg += f" (hipError {lib.lci_last_hip_error()})"
        raise LciError(rc, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t, dtype, name, ndim=None):
    import torch
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def make_geom(B, Tq, Tk, K, q_offset, kv_len, Hq=0, Hkv=0, d=0, H_I=0, d_I=0,
              block=1, sets=1) -> lci_geom:
    import torch
    _dev(q_offset, torch.int32, "q_offset", 1)
    _dev(kv_len, torch.int32, "kv_len", 1)
    if q_offset.numel() != B or kv_len.numel() != B:
        raise ValueError("q_offset and kv_len need one entry per sequence")
    g = lci_geom(B, Tq, Tk, Hq, Hkv, d, H_I, d_I, K, q_offset.data_ptr(), kv_len.data_ptr(),
                 block, sets)
    g._keep = (q_offset, kv_len)
    return g


def _w_strides(w, B, Tq, H_I):
    """Element strides (sequence, row) of indexer weights shaped [H_I], [Tq,H_I] or [B,Tq,H_I]."""
    if w.dim() == 1 and w.shape[0] == H_I:
        return 0, 0
    if w.dim() == 2 and tuple(w.shape) == (Tq, H_I):
        return 0, H_I
    if w.dim() == 3 and tuple(w.shape) == (B, Tq, H_I):
        return Tq * H_I, H_I
    raise ValueError(f"indexer weights must be [H_I], [Tq,H_I] or [B,Tq,H_I]; got {tuple(w.shape)}")


def workspace_bytes(entry: int, geom: lci_geom) -> int:
    return int(load_library().lci_workspace_bytes(entry, ctypes.byref(geom)))


def dense_row_limit(geom: lci_geom, entry: int = ENTRY_PREFILL) -> int:
    """Rows with p + 1 <= this limit take the dense-tile attention path (0: none)."""
    return int(load_library().lci_dense_row_limit(entry, ctypes.byref(geom)))


def attn_overlap(mode: int) -> None:
    """Process-wide schedule of the tile and gather attention kernels:
    OVERLAP_AUTO (default), OVERLAP_OFF or OVERLAP_ON (results identical)."""
    _check(load_library().lci_attn_overlap(int(mode)))


def attn_overlap_forks() -> int:
    """Calls so far that ran the tile and gather kernels at once on the library streams."""
    return int(load_library().lci_attn_overlap_forks())


def kernel_timing(enable: bool) -> None:
    """Switch the library's per-kernel event log on (cleared) or off."""
    _check(load_library().lci_kernel_timing(1 if enable else 0))


def kernel_timing_read(kernel) -> tuple:
    """(total_ms, launches) of one kernel kind (index or name) since timing was switched on."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().lci_kernel_timing_read(k, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def kernel_name(kernel: int) -> Optional[str]:
    r = load_library().lci_kernel_name(int(kernel))
    return None if r is None else r.decode()


def _workspace(entry, geom, workspace, device):
    import torch
    need = workspace_bytes(entry, geom)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def idx_score(q_idx, k_idx, w, q_offset, kv_len, scores=None, stream=None, sets=1):
    """Indexer scores int32 [B,Tq,Tk]; only s <= p of each valid row is written.
    With sets > 1 the indexer heads split into `sets` groups, each scoring its
    own set: scores [B,sets,Tq,Tk]."""
    import torch
    _dev(q_idx, torch.int8, "q_idx", 4)
    _dev(k_idx, torch.int8, "k_idx", 3)
    _dev(w, torch.int8, "w")
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    if k_idx.shape[0] != B or k_idx.shape[2] != d_I:
        raise ValueError("k_idx must be [B,Tk,d_I]")
    wsb, wsq = _w_strides(w, B, Tq, H_I)
    g = make_geom(B, Tq, Tk, 1, q_offset, kv_len, H_I=H_I, d_I=d_I, sets=sets)
    shape = (B, Tq, Tk) if sets <= 1 else (B, sets, Tq, Tk)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.int32, device=q_idx.device)
    _dev(scores, torch.int32, "scores", len(shape))
    if tuple(scores.shape) != shape:
        raise ValueError(f"scores must be {list(shape)}")
    lib = load_library()
    _check(lib.lci_idx_score(ctypes.byref(g), _ptr(q_idx), _ptr(k_idx), _ptr(w), wsb, wsq,
                             _ptr(scores), _stream(stream)))
    return scores


def topk_select(scores, K, q_offset, kv_len, idx=None, sel_scores=None, want_scores=False,
                workspace=None, stream=None, block=1):
    """Top-K positions int32 [B,Tq,K] (ascending, -1 padded) and optional scores.
    With block > 1, the K best blocks of `block` positions: idx [B,Tq,K*block]
    holds their positions, sel_scores [B,Tq,K] the blocks' scores. Scores of
    several index sets, [B,sets,Tq,Tk], give idx [B,sets,Tq,K*block] and
    sel_scores [B,sets,Tq,K]."""
    import torch
    if scores is not None and scores.dim() == 4:
        _dev(scores, torch.int32, "scores", 4)
        B, sets, Tq, Tk = scores.shape
    else:
        _dev(scores, torch.int32, "scores", 3)
        (B, Tq, Tk), sets = scores.shape, 1
    lead = (B, Tq) if scores.dim() == 3 else (B, sets, Tq)
    g = make_geom(B, Tq, Tk, K, q_offset, kv_len, block=block, sets=sets)
    if idx is None:
        idx = torch.empty(lead + (K * max(block, 1),), dtype=torch.int32, device=scores.device)
    if want_scores and sel_scores is None:
        sel_scores = torch.empty(lead + (K,), dtype=torch.int32, device=scores.device)
    _dev(idx, torch.int32, "idx", len(lead) + 1)
    _dev(sel_scores, torch.int32, "sel_scores", len(lead) + 1)
    if tuple(idx.shape) != lead + (K * max(block, 1),) or \
            (sel_scores is not None and tuple(sel_scores.shape) != lead + (K,)):
        raise ValueError("idx / sel_scores do not match the score rows")
    ws, nb = _workspace(ENTRY_TOPK_SELECT, g, workspace, scores.device)
    lib = load_library()
    _check(lib.lci_topk_select(ctypes.byref(g), _ptr(scores), _ptr(idx), _ptr(sel_scores),
                               _ptr(ws), nb, _stream(stream)))
    return (idx, sel_scores) if want_scores or sel_scores is not None else idx


def sparse_attn_fwd(q, k, v, idx, gate, scale, kv_len, q_offset=None, out=None, lse=None,
                    want_lse=False, workspace=None, stream=None, mix=None):
    """Gated attention over the listed positions: out bf16 [B,Tq,Hq,d] (and lse).
    idx int32 [B,Tq,K] (one index set per row) or [B,sets,Tq,K] with sets
    dividing Hq: query head h attends over set h // (Hq // sets) (sets = Hkv:
    one per key/value head; sets = Hq: one per query head). With ``mix`` (bf16,
    the shape of q) the gate mixes: s*o + (1-s)*mix."""
    import torch
    _dev(q, torch.bfloat16, "q", 4)
    _dev(k, torch.bfloat16, "k", 4)
    _dev(v, torch.bfloat16, "v", 4)
    sets = 1
    if idx is not None and idx.dim() == 4:
        sets = idx.shape[1]
        _dev(idx, torch.int32, "idx", 4)
        if idx.shape[0] != q.shape[0] or idx.shape[2] != q.shape[1] or q.shape[2] % sets:
            raise ValueError("per-head index rows must be [B,sets,Tq,K], sets dividing Hq")
        idx3 = idx.view(idx.shape[0], sets * idx.shape[2], idx.shape[3])
    else:
        _dev(idx, torch.int32, "idx", 3)
        idx3 = idx
    _dev(gate, torch.bfloat16, "gate", 4)
    _dev(mix, torch.bfloat16, "mix", 4)
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Tk, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [B,Tk,Hkv,d]")
    if sets == 1 and idx.shape[:2] != (B, Tq):
        raise ValueError("idx must be [B,Tq,K]")
    _gate_args(q, gate, mix)
    if q_offset is None:
        q_offset = torch.zeros(B, dtype=torch.int32, device=q.device)
    g = make_geom(B, Tq, Tk, idx3.shape[2], q_offset, kv_len, Hq=Hq, Hkv=Hkv, d=d, sets=sets)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dev(out, torch.bfloat16, "out", 4)
    _dev(lse, torch.float32, "lse", 3)
    ws, nb = _workspace(ENTRY_SPARSE_ATTN, g, workspace, q.device)
    lib = load_library()
    _check(lib.lci_sparse_attn_fwd(ctypes.byref(g), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                   _ptr(gate), _ptr(mix), float(scale), _ptr(out), _ptr(lse),
                                   _ptr(ws), nb, _stream(stream)))
    return (out, lse) if lse is not None else out


def _gate_args(q, gate, mix):
    if gate is not None and tuple(gate.shape) != tuple(q.shape):
        raise ValueError("gate must match q")
    if mix is not None and tuple(mix.shape) != tuple(q.shape):
        raise ValueError("mix must match q")
    if mix is not None and gate is None:
        raise ValueError("mix needs a gate")


def _fused(fn_name, entry, q_idx, k_idx, w, q, k, v, gate, mix, scale, q_offset, kv_len, K,
           out, lse, idx_out, want_lse, want_idx, workspace, stream, block=1, sets=1,
           noalloc=False):
    import torch
    _dev(q_idx, torch.int8, "q_idx", 4)
    _dev(k_idx, torch.int8, "k_idx", 3)
    _dev(w, torch.int8, "w")
    _dev(q, torch.bfloat16, "q", 4)
    _dev(k, torch.bfloat16, "k", 4)
    _dev(v, torch.bfloat16, "v", 4)
    _dev(gate, torch.bfloat16, "gate", 4)
    _dev(mix, torch.bfloat16, "mix", 4)
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    _, _, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(q.shape[:2]) != (B, Tq) or tuple(k.shape) != (B, Tk, Hkv, d) or \
            tuple(v.shape) != tuple(k.shape) or tuple(k_idx.shape) != (B, Tk, d_I):
        raise ValueError("inconsistent shapes")
    _gate_args(q, gate, mix)
    wsb, wsq = _w_strides(w, B, Tq, H_I)
    g = make_geom(B, Tq, Tk, K, q_offset, kv_len, Hq=Hq, Hkv=Hkv, d=d, H_I=H_I, d_I=d_I,
                  block=block, sets=sets)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if want_idx and idx_out is None:
        shape = (B, Tq, K * max(block, 1)) if sets <= 1 else (B, sets, Tq, K * max(block, 1))
        idx_out = torch.empty(shape, dtype=torch.int32, device=q.device)
    _dev(out, torch.bfloat16, "out", 4)
    _dev(lse, torch.float32, "lse", 3)
    _dev(idx_out, torch.int32, "idx_out", 3 if sets <= 1 else 4)
    lib = load_library()
    args = [ctypes.byref(g), _ptr(q_idx), _ptr(k_idx), _ptr(w), wsb, wsq, _ptr(q), _ptr(k),
            _ptr(v), _ptr(gate), _ptr(mix), float(scale), _ptr(out), _ptr(lse), _ptr(idx_out)]
    if not noalloc:
        ws, nb = _workspace(entry, g, workspace, q.device)
        args += [_ptr(ws), nb]
    _check(getattr(lib, fn_name)(*args, _stream(stream)))
    res = [out]
    if idx_out is not None:
        res.append(idx_out)
    if lse is not None:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def prefill_fwd(q_idx, k_idx, w, q, k, v, gate, scale, q_offset, kv_len, K, out=None, lse=None,
                idx_out=None, want_lse=False, want_idx=False, workspace=None, stream=None,
                mix=None, block=1, sets=1):
    """Fused layer for many query rows: returns out (and idx, lse when asked).
    ``mix`` as in ``sparse_attn_fwd``; with block > 1 the selection keeps K blocks
    of `block` positions and idx rows hold K*block positions; with sets > 1
    (dividing Hq and H_I) query head h attends over index set h // (Hq // sets),
    scored by the set's group of H_I // sets indexer heads (sets = Hkv: one per
    key/value head; sets = Hq: one per query head; idx [B,sets,Tq,K*block])."""
    return _fused("lci_prefill_fwd", ENTRY_PREFILL, q_idx, k_idx, w, q, k, v, gate, mix, scale,
                  q_offset, kv_len, K, out, lse, idx_out, want_lse, want_idx, workspace, stream,
                  block, sets)


def decode_fwd(q_idx, k_idx, w, q, k, v, gate, scale, q_offset, kv_len, K, out=None, lse=None,
               idx_out=None, want_lse=False, want_idx=False, workspace=None, stream=None,
               mix=None, block=1, sets=1):
    """Fused layer for one query row per sequence (Tq == 1) over a long history.
    ``mix``, ``block`` and ``sets`` as in ``prefill_fwd``."""
    return _fused("lci_decode_fwd", ENTRY_DECODE, q_idx, k_idx, w, q, k, v, gate, mix, scale,
                  q_offset, kv_len, K, out, lse, idx_out, want_lse, want_idx, workspace, stream,
                  block, sets)


def indexer_bwd(q_idx, k_idx, w, idx, teacher, tau, q_offset, kv_len, loss=True, workspace=None,
                stream=None):
    """Gradients of the scorer's distillation loss over index rows idx int32
    [B,Tq,K] with the teacher's weights teacher fp32 [B,Tq,K] and score scale tau.
    With index sets, idx and teacher are [B,S,Tq,K] (S dividing H_I; set j is
    scored by indexer heads j*H_I/S .. (j+1)*H_I/S - 1) and loss [B,S,Tq].
    Returns dict(loss [B,Tq] or None, dq [B,Tq,H_I,d_I], dk [B,Tk,d_I], dw [B,Tq,H_I])."""
    import torch
    _dev(q_idx, torch.int8, "q_idx", 4)
    _dev(k_idx, torch.int8, "k_idx", 3)
    _dev(w, torch.int8, "w")
    _dev(idx, torch.int32, "idx")
    _dev(teacher, torch.float32, "teacher")
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    if idx.dim() not in (3, 4):
        raise ValueError("idx must be [B,Tq,K] or [B,S,Tq,K]")
    sets = idx.shape[1] if idx.dim() == 4 else 1
    K = idx.shape[-1]
    want = (B, sets, Tq, K) if idx.dim() == 4 else (B, Tq, K)
    if tuple(idx.shape) != want or tuple(teacher.shape) != want or \
            tuple(k_idx.shape) != (B, Tk, d_I) or H_I % sets:
        raise ValueError("inconsistent shapes")
    wsb, wsq = _w_strides(w, B, Tq, H_I)
    g = make_geom(B, Tq, Tk, K, q_offset, kv_len, H_I=H_I, d_I=d_I, sets=sets)
    dev = q_idx.device
    out_loss = None
    if loss:
        out_loss = torch.empty((B, sets, Tq) if idx.dim() == 4 else (B, Tq), dtype=torch.float32,
                               device=dev)
    dq = torch.empty((B, Tq, H_I, d_I), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Tk, d_I), dtype=torch.float32, device=dev)
    dw = torch.empty((B, Tq, H_I), dtype=torch.float32, device=dev)
    ws, nb = _workspace(ENTRY_INDEXER_BWD, g, workspace, dev)
    _check(load_library().lci_indexer_bwd(ctypes.byref(g), _ptr(q_idx), _ptr(k_idx), _ptr(w), wsb,
                                          wsq, _ptr(idx), _ptr(teacher), float(tau),
                                          _ptr(out_loss), _ptr(dq), _ptr(dk), _ptr(dw), _ptr(ws),
                                          nb, _stream(stream)))
    return dict(loss=out_loss, dq=dq, dk=dk, dw=dw)


def decode_fwd_noalloc(q_idx, k_idx, w, q, k, v, gate, scale, q_offset, kv_len, K, out=None,
                       lse=None, idx_out=None, want_lse=False, want_idx=False, stream=None,
                       mix=None, block=1, sets=1):
    """``decode_fwd`` without a workspace: the library carves it out of its static
    per-device scratch array (no device allocation inside the library; the
    outputs are allocated here only when the caller passes none). Calls that
    overlap on one GPU race on that array."""
    return _fused("lci_decode_fwd_noalloc", ENTRY_DECODE, q_idx, k_idx, w, q, k, v, gate, mix,
                  scale, q_offset, kv_len, K, out, lse, idx_out, want_lse, want_idx, None,
                  stream, block, sets, noalloc=True)


def noalloc_scratch_bytes() -> int:
    """Bytes of the static scratch array behind ``decode_fwd_noalloc``."""
    return int(load_library().lci_noalloc_scratch_bytes())


def kv_append(k_new, v_new, kI_new, k_cache, v_cache, kI_cache, kv_len, n_new=None,
              q_offset_out=None, kv_len_out=None, stream=None):
    """Append rows to the key/value/indexer-key caches (in place) after each
    sequence's kv_len rows. k_new, v_new bf16 [B,Tn,Hkv,d], kI_new int8 [B,Tn,d_I];
    caches [B,Tk,...]; n_new int32 [B] rows per sequence (None: all Tn).
    Returns (q_offset_out, kv_len_out): the first appended position and the new
    length per sequence; kv_len_out may be kv_len itself (updated in place)."""
    import torch
    _dev(k_new, torch.bfloat16, "k_new", 4)
    _dev(v_new, torch.bfloat16, "v_new", 4)
    _dev(kI_new, torch.int8, "kI_new", 3)
    _dev(k_cache, torch.bfloat16, "k_cache", 4)
    _dev(v_cache, torch.bfloat16, "v_cache", 4)
    _dev(kI_cache, torch.int8, "kI_cache", 3)
    _dev(kv_len, torch.int32, "kv_len", 1)
    _dev(n_new, torch.int32, "n_new", 1)
    B, Tn, Hkv, d = k_new.shape
    Tk, d_I = k_cache.shape[1], kI_new.shape[2]
    if tuple(v_new.shape) != tuple(k_new.shape) or tuple(kI_new.shape[:2]) != (B, Tn) or \
            tuple(k_cache.shape) != (B, Tk, Hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or tuple(kI_cache.shape) != (B, Tk, d_I) or kv_len.numel() != B or \
            (n_new is not None and n_new.numel() != B):
        raise ValueError("inconsistent shapes")
    if q_offset_out is None:
        q_offset_out = torch.empty_like(kv_len)
    if kv_len_out is None:
        kv_len_out = torch.empty_like(kv_len)
    _dev(q_offset_out, torch.int32, "q_offset_out", 1)
    _dev(kv_len_out, torch.int32, "kv_len_out", 1)
    g = lci_geom(B, Tn, Tk, 0, Hkv, d, 0, d_I, 0, None, kv_len.data_ptr())
    _check(load_library().lci_kv_append(ctypes.byref(g), _ptr(k_new), _ptr(v_new), _ptr(kI_new),
                                        _ptr(n_new), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(kI_cache), _ptr(q_offset_out), _ptr(kv_len_out),
                                        _stream(stream)))
    return q_offset_out, kv_len_out


def sparse_attn_bwd(q, k, v, idx, gate, scale, kv_len, dy, q_offset=None, mix=None,
                    workspace=None, stream=None):
    """Gradients of sparse_attn_fwd for the output gradient dy (bf16, the shape of q):
    returns dict(dq, dk, dv, dgate, dmix) as float32 tensors (dgate / dmix None
    without gate / mix). idx int32 [B,Tq,K] (one index set) or [B,sets,Tq,K]
    (query head h reads set h // (Hq // sets)), as in sparse_attn_fwd."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dy, "dy")):
        _dev(t, torch.bfloat16, n, 4)
    B, Tq, Hq, d = q.shape
    sets = 1
    if idx is not None and idx.dim() == 4:
        _dev(idx, torch.int32, "idx", 4)
        sets = idx.shape[1]
        if idx.shape[0] != B or idx.shape[2] != Tq or Hq % sets:
            raise ValueError("per-head index rows must be [B,sets,Tq,K], sets dividing Hq")
    else:
        _dev(idx, torch.int32, "idx", 3)
        if idx.shape[:2] != (B, Tq):
            raise ValueError("idx must be [B,Tq,K]")
    _dev(gate, torch.bfloat16, "gate", 4)
    _dev(mix, torch.bfloat16, "mix", 4)
    Tk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Tk, Hkv, d) or tuple(v.shape) != tuple(k.shape) or \
            tuple(dy.shape) != tuple(q.shape):
        raise ValueError("inconsistent shapes")
    _gate_args(q, gate, mix)
    if q_offset is None:
        q_offset = torch.zeros(B, dtype=torch.int32, device=q.device)
    g = make_geom(B, Tq, Tk, idx.shape[-1], q_offset, kv_len, Hq=Hq, Hkv=Hkv, d=d, sets=sets)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(k.shape, **f32)
    dg = torch.empty(q.shape, **f32) if gate is not None else None
    dm = torch.empty(q.shape, **f32) if mix is not None else None
    ws, nb = _workspace(ENTRY_SPARSE_ATTN_BWD, g, workspace, q.device)
    _check(load_library().lci_sparse_attn_bwd(ctypes.byref(g), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(idx), _ptr(gate), _ptr(mix), _ptr(dy),
                                              float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                              _ptr(dg), _ptr(dm), _ptr(ws), nb, _stream(stream)))
    return dict(dq=dq, dk=dk, dv=dv, dgate=dg, dmix=dm)
