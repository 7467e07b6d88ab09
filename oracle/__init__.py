"""CPU oracle for the gated fine-grained sparse attention layer (ctypes over oracle.c).

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. It shares no code with
the GPU library and the GPU library never calls it.

Every function takes host numpy arrays. bf16 tensors are passed as their uint16
bit patterns; the oracle widens them exactly and computes in fp64. Indexer
arithmetic is exact (int64, checked against the int32 range).

Parity status of each function (pins live in tests/test_oracle_pins.py):
  scores     pinned: closed forms on unit-vector keys, zero queries, weight
             linearity, a hand-worked example (tests/golden/indexer_hand.json)
  topk       pinned: O(n^2) rank definition, closed forms (monotone and constant rows)
  attention  pinned: dense causal attention from torch's SDPA when K >= p+1, K = 1,
             constant values, a two-key closed form, permutation invariance;
             its fp32-source form (attention_f32): the same SDPA pin on fp32
             inputs, and equality with the bf16 form on bf16-exact values
  gate       pinned: G = 0 halves the output, G -> +inf leaves it, closed form
  gradients  pinned: torch autograd (fp64) through independent statements of the
             attention forward and of the indexer's distillation loss; closed
             forms (constant values; a teacher equal to the scorer's own
             distribution; one entry)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
OVERFLOW = 1


def compile_source(src_path: str, out_path: str) -> str:
    """Compile an oracle C source with gcc (OpenMP) into a shared library."""
    tmp = out_path + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Wno-unknown-pragmas", src_path, "-o", tmp, "-lm"])
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = False) -> str:
    """Compile oracle.c into oracle/liboracle.so (only when stale unless forced)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def open_library(path: str):
    """ctypes handle of a compiled oracle with its signatures declared."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_score_row.argtypes = [i32, i32, P, P, P, i64, P]
    lib.orc_score_row.restype = i32
    lib.orc_topk_row.argtypes = [P, i64, i32, P, P]
    lib.orc_attn_row.argtypes = [i32, i32, i32, P, P, P, i64, P, i32, i32, P, P, f64, P, P]
    lib.orc_scores_rows.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i64, i64, i64, P, P, P]
    lib.orc_scores_rows.restype = i32
    lib.orc_topk_rows.argtypes = [i64, P, i64, P, i32, P, P]
    lib.orc_attn_rows.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, f64, i64,
                                  P, P, P, P, P]
    lib.orc_attn_rows_f32.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, f64, i64,
                                      P, P, P, P, P]
    lib.orc_block_topk_rows.argtypes = [i64, P, i64, P, i32, i32, P, P, P]
    lib.orc_layer_rows.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                   i64, i64, P, P, P, P, P, f64, i64, P, P, P, P, P, P]
    lib.orc_layer_rows.restype = i32
    lib.orc_kv_append.argtypes = [i32, i32, i32, i64, P, P, P, P, P, P]
    lib.orc_attn_bwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                 f64, P, P, P, P, P]
    lib.orc_indexer_bwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, i64, i64, P,
                                    P, f64, P, P, P, P]
    lib.orc_num_threads.restype = i32
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _w_strides(w, B, Tq, H_I):
    """Element strides (per sequence, per row) of a weight array of shape [H_I],
    [Tq,H_I] or [B,Tq,H_I]; a missing leading axis broadcasts (stride 0)."""
    w = np.asarray(w)
    if w.ndim == 1:
        return 0, 0
    if w.ndim == 2:
        return 0, H_I
    return Tq * H_I, H_I


def _rows(rows, B, Tq):
    if rows is None:
        rb, ri = np.divmod(np.arange(B * Tq, dtype=np.int64), Tq)
    else:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        rb, ri = rows[:, 0], rows[:, 1]
    return _c(rb, np.int32), _c(ri, np.int32)


class Oracle:
    """One compiled oracle library (the real one, or a deliberately mutated
    build used to check that the pins catch plausible mistakes)."""

    def __init__(self, path: str):
        self.lib = open_library(path)

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def score_row(self, q_idx_row, k_idx, w, n):
        """Scores of one query row (qI [H_I,d_I]) against history rows 0..n-1.
        Returns (S int32 [n], overflowed bool)."""
        q_idx_row = _c(q_idx_row, np.int8)
        H_I, d_I = q_idx_row.shape
        k_idx = _c(k_idx, np.int8)
        w = _c(w, np.int8)
        S = np.empty(n, np.int32)
        rc = self.lib.orc_score_row(H_I, d_I, _p(q_idx_row), _p(k_idx), _p(w), n, _p(S))
        return S, rc == OVERFLOW

    def scores(self, q_idx, k_idx, w, q_offset, kv_len, rows=None):
        """Indexer scores for the listed (b, i) rows (default: all rows).
        Returns S int32 [nrows, Tk]; only positions 0..p of each row are defined
        (the rest hold INT32_MIN). Raises OverflowError on an int32 overflow."""
        q_idx = _c(q_idx, np.int8)
        k_idx = _c(k_idx, np.int8)
        B, Tq, H_I, d_I = q_idx.shape
        Tk = k_idx.shape[1]
        w = _c(w, np.int8)
        wsb, wsq = _w_strides(w, B, Tq, H_I)
        rb, ri = _rows(rows, B, Tq)
        S = np.full((len(rb), Tk), np.iinfo(np.int32).min, np.int32)
        rc = self.lib.orc_scores_rows(Tq, Tk, H_I, d_I, _p(_c(q_offset, np.int32)),
                                     _p(_c(kv_len, np.int32)), _p(q_idx), _p(k_idx), _p(w),
                                     wsb, wsq, len(rb), _p(rb), _p(ri), _p(S))
        if rc == OVERFLOW:
            raise OverflowError("indexer score outside the int32 range")
        return S

    def topk(self, S, n, K):
        """Top-K of each score row. S [nrows, stride] int32; n [nrows] candidates per row.
        Returns (idx int32 [nrows, K] ascending with -1 padding, sel int32 [nrows, K])."""
        S = _c(S, np.int32)
        if S.ndim == 1:
            S = S[None]
        n = _c(np.broadcast_to(np.asarray(n, dtype=np.int64), (S.shape[0],)), np.int64)
        idx = np.empty((S.shape[0], K), np.int32)
        sel = np.empty((S.shape[0], K), np.int32)
        self.lib.orc_topk_rows(S.shape[0], _p(S), S.shape[1], _p(n), K, _p(idx), _p(sel))
        return idx, sel

    def attention(self, q, k, v, gate, idx, kv_len, scale, rows=None, mix=None):
        """Gated attention over given index rows. q, gate, mix uint16 [B,Tq,Hq,d] (gate
        may be None: ungated; mix may be None: the gate only scales, else
        out = s*o + (1-s)*mix); k, v uint16 [B,Tk,Hkv,d]; idx int32 [nrows, K] (one
        set per row) or [nrows, sets, K] for the listed rows, where query head h
        reads set h // (Hq // sets) (one set per key/value head with sets = Hkv,
        per query head with sets = Hq). Returns (out float64 [nrows,Hq,d], lse
        float64 [nrows,Hq])."""
        q = _c(q, np.uint16)
        k = _c(k, np.uint16)
        v = _c(v, np.uint16)
        B, Tq, Hq, d = q.shape
        Tk, Hkv = k.shape[1], k.shape[2]
        gate = None if gate is None else _c(gate, np.uint16)
        mix = None if mix is None else _c(mix, np.uint16)
        for t in (gate, mix):
            if t is not None and t.shape != q.shape:
                raise ValueError("gate and mix have the shape of q")
        rb, ri = _rows(rows, B, Tq)
        idx = _c(idx, np.int32)
        sets = idx.shape[1] if idx.ndim == 3 else 1
        if Hq % sets:
            raise ValueError("the index sets divide the query heads")
        idx = idx.reshape(len(rb), sets, -1)
        K = idx.shape[2]
        out = np.empty((len(rb), Hq, d), np.float64)
        lse = np.empty((len(rb), Hq), np.float64)
        self.lib.orc_attn_rows(Tq, Tk, Hq, Hkv, d, K, sets, _p(_c(kv_len, np.int32)), _p(q), _p(k),
                              _p(v), _p(gate), _p(mix), float(scale), len(rb), _p(rb), _p(ri),
                              _p(idx), _p(out), _p(lse))
        return out, lse

    def attention_f32(self, q, k, v, gate, idx, kv_len, scale, rows=None):
        """``attention`` on fp32 sources (float32 q, gate [B,Tq,Hq,d], k, v
        [B,Tk,Hkv,d]; gate may be None), no mix: the same fp64 arithmetic on
        the fp32 values, for configurations whose inputs are drawn in fp32."""
        q = _c(q, np.float32)
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        B, Tq, Hq, d = q.shape
        Tk, Hkv = k.shape[1], k.shape[2]
        gate = None if gate is None else _c(gate, np.float32)
        if gate is not None and gate.shape != q.shape:
            raise ValueError("gate has the shape of q")
        rb, ri = _rows(rows, B, Tq)
        idx = _c(idx, np.int32)
        sets = idx.shape[1] if idx.ndim == 3 else 1
        if Hq % sets:
            raise ValueError("the index sets divide the query heads")
        idx = idx.reshape(len(rb), sets, -1)
        K = idx.shape[2]
        out = np.empty((len(rb), Hq, d), np.float64)
        lse = np.empty((len(rb), Hq), np.float64)
        self.lib.orc_attn_rows_f32(Tq, Tk, Hq, Hkv, d, K, sets, _p(_c(kv_len, np.int32)), _p(q),
                                   _p(k), _p(v), _p(gate), float(scale), len(rb), _p(rb), _p(ri),
                                   _p(idx), _p(out), _p(lse))
        return out, lse

    def block_topk(self, S, n, K, block):
        """Block-granular Top-K of each score row (blocks of `block` positions scored
        by their best position). Returns (idx int32 [nrows, K*block] positions
        ascending, -1 padded; blocks int32 [nrows, K] ascending, -1 padded; their
        scores int32 [nrows, K], INT32_MIN in the padding)."""
        S = _c(S, np.int32)
        if S.ndim == 1:
            S = S[None]
        n = _c(np.broadcast_to(np.asarray(n, dtype=np.int64), (S.shape[0],)), np.int64)
        if block < 1 or K < 1:
            raise ValueError("block and K are positive")
        idx = np.empty((S.shape[0], K * block), np.int32)
        blk = np.empty((S.shape[0], K), np.int32)
        sel = np.empty((S.shape[0], K), np.int32)
        self.lib.orc_block_topk_rows(S.shape[0], _p(S), S.shape[1], _p(n), block, K, _p(idx),
                                    _p(blk), _p(sel))
        return idx, blk, sel

    def attention_bwd(self, q, k, v, gate, idx, kv_len, scale, dy, mix=None):
        """Gradients of the gated attention over index rows idx int32 [B,Tq,K] (one
        set) or [B,Tq,sets,K] (query head h reads set h // (Hq // sets)) for the
        output gradient dy uint16 [B,Tq,Hq,d]. q, gate, mix, dy bf16 bits
        [B,Tq,Hq,d]; k, v [B,Tk,Hkv,d]. Returns dict(dq, dgate, dmix [B,Tq,Hq,d];
        dk, dv [B,Tk,Hkv,d]) in float64 (dgate / dmix None without gate / mix)."""
        q, k, v, dy = (_c(a, np.uint16) for a in (q, k, v, dy))
        B, Tq, Hq, d = q.shape
        Tk, Hkv = k.shape[1], k.shape[2]
        gate = None if gate is None else _c(gate, np.uint16)
        mix = None if mix is None else _c(mix, np.uint16)
        if mix is not None and gate is None:
            raise ValueError("mix needs a gate")
        idx = _c(idx, np.int32)
        sets = idx.shape[2] if idx.ndim == 4 else 1
        if Hq % sets:
            raise ValueError("the index sets divide the query heads")
        idx = idx.reshape(B, Tq, sets, -1)
        K = idx.shape[3]
        dq = np.empty((B, Tq, Hq, d), np.float64)
        dk = np.empty((B, Tk, Hkv, d), np.float64)
        dv = np.empty((B, Tk, Hkv, d), np.float64)
        dg = np.empty((B, Tq, Hq, d), np.float64) if gate is not None else None
        dm = np.empty((B, Tq, Hq, d), np.float64) if mix is not None else None
        self.lib.orc_attn_bwd(B, Tq, Tk, Hq, Hkv, d, K, sets, _p(_c(kv_len, np.int32)), _p(q), _p(k),
                              _p(v), _p(gate), _p(mix), _p(idx), _p(dy), float(scale), _p(dq),
                              _p(dk), _p(dv), _p(dg), _p(dm))
        return dict(dq=dq, dk=dk, dv=dv, dgate=dg, dmix=dm)

    def indexer_bwd(self, q_idx, k_idx, w, q_offset, kv_len, idx, teacher, tau):
        """Gradients of the indexer's distillation loss over index rows idx int32
        [B,Tq,K] with the teacher's weights teacher [B,Tq,K] (float) and score
        scale tau. Returns dict(loss [B,Tq], dq [B,Tq,H_I,d_I], dk [B,Tk,d_I],
        dw [B,Tq,H_I]) in float64 (dw per row; sum over rows for shared weights).
        With index sets, idx and teacher are [B,S,Tq,K] (S dividing H_I; set g
        scored by indexer heads g*H_I/S .. (g+1)*H_I/S - 1) and loss [B,S,Tq]."""
        q_idx = _c(q_idx, np.int8)
        k_idx = _c(k_idx, np.int8)
        B, Tq, H_I, d_I = q_idx.shape
        Tk = k_idx.shape[1]
        w = _c(w, np.int8)
        wsb, wsq = _w_strides(w, B, Tq, H_I)
        idx = _c(idx, np.int32)
        sets = idx.shape[1] if idx.ndim == 4 else 1
        if H_I % sets:
            raise ValueError("sets must divide H_I")
        idx = idx.reshape(B, sets, Tq, -1)
        K = idx.shape[3]
        T = _c(teacher, np.float64).reshape(B, sets, Tq, K)
        loss = np.empty((B, sets, Tq), np.float64)
        dq = np.empty((B, Tq, H_I, d_I), np.float64)
        dk = np.empty((B, Tk, d_I), np.float64)
        dw = np.empty((B, Tq, H_I), np.float64)
        self.lib.orc_indexer_bwd(B, Tq, Tk, H_I, d_I, K, sets, _p(_c(q_offset, np.int32)),
                                 _p(_c(kv_len, np.int32)), _p(q_idx), _p(k_idx), _p(w), wsb, wsq,
                                 _p(idx), _p(T), float(tau), _p(loss), _p(dq), _p(dk), _p(dw))
        return dict(loss=loss if sets > 1 else loss[:, 0], dq=dq, dk=dk, dw=dw)

    def layer(self, inp, K, rows=None, gated=True, block=1, sets=1):
        """The whole layer (score -> Top-K -> attention -> gate) for the listed rows
        of an input dict as produced by ``synth.host_inputs``; an entry "mix" (the
        other branch's output, uint16 [B,Tq,Hq,d]) is mixed in by the gate. With
        block > 1 the selection keeps K blocks of `block` positions: idx holds
        K*block positions per row and sel the K kept blocks' scores. With sets > 1
        (dividing Hq and H_I) query head h attends over index set h // (Hq // sets),
        scored by indexer heads g*H_I/sets .. (g+1)*H_I/sets - 1 of set g: sets =
        Hkv gives one set per key/value head, sets = Hq one per query head;
        idx [nrows, sets, K or K*block], sel [nrows, sets, K].
        Returns dict(idx, sel, out, lse) with out float64 [nrows,Hq,d]."""
        q_idx = _c(inp["q_idx"], np.int8)
        k_idx = _c(inp["k_idx"], np.int8)
        B, Tq, H_I, d_I = q_idx.shape
        Tk = k_idx.shape[1]
        q = _c(inp["q"], np.uint16)
        k = _c(inp["k"], np.uint16)
        v = _c(inp["v"], np.uint16)
        Hq, d = q.shape[2], q.shape[3]
        Hkv = k.shape[2]
        gate = _c(inp["gate"], np.uint16) if gated and inp.get("gate") is not None else None
        mix = _c(inp["mix"], np.uint16) if gate is not None and inp.get("mix") is not None else None
        if mix is not None and mix.shape != q.shape:
            raise ValueError("mix has the shape of q")
        w = _c(inp["w"], np.int8)
        wsb, wsq = _w_strides(w, B, Tq, H_I)
        rb, ri = _rows(rows, B, Tq)
        nr = len(rb)
        bl = max(int(block), 1)
        ns = max(int(sets), 1)
        if Hq % ns or H_I % ns:
            raise ValueError("sets divides Hq and H_I")
        idx = np.empty((nr, ns, K * bl), np.int32)
        sel = np.empty((nr, ns, K), np.int32)
        out = np.empty((nr, Hq, d), np.float64)
        lse = np.empty((nr, Hq), np.float64)
        rc = self.lib.orc_layer_rows(Tq, Tk, Hq, Hkv, d, H_I, d_I, K, bl, ns,
                                    _p(_c(inp["q_offset"], np.int32)), _p(_c(inp["kv_len"], np.int32)),
                                    _p(q_idx), _p(k_idx), _p(w), wsb, wsq, _p(q), _p(k), _p(v),
                                    _p(gate), _p(mix), float(inp["scale"]), nr, _p(rb), _p(ri), _p(idx),
                                    _p(sel), _p(out), _p(lse))
        if rc == OVERFLOW:
            raise OverflowError("indexer score outside the int32 range")
        if ns == 1:
            idx, sel = idx[:, 0], sel[:, 0]
        return dict(idx=idx, sel=sel, out=out, lse=lse)


    def kv_append(self, new, cache, kv_len, n_new=None):
        """Append rows to a cache: new [B, Tn, ...], cache [B, Tk, ...] (same trailing
        shape and dtype), kv_len int32 [B], n_new int32 [B] or None (all Tn rows).
        Returns (cache', q_offset_out, kv_len_out); the input cache is not modified."""
        new = np.ascontiguousarray(new)
        out = np.array(cache, copy=True, order="C")
        if new.dtype != out.dtype or new.shape[0] != out.shape[0] or new.shape[2:] != out.shape[2:]:
            raise ValueError("new and cache must agree in dtype, batch and row shape")
        B, Tn, Tk = new.shape[0], new.shape[1], out.shape[1]
        row_bytes = int(np.prod(new.shape[2:], dtype=np.int64)) * new.dtype.itemsize
        kv = _c(kv_len, np.int32)
        nn = None if n_new is None else _c(n_new, np.int32)
        if kv.shape != (B,) or (nn is not None and nn.shape != (B,)):
            raise ValueError("kv_len and n_new have one entry per sequence")
        qo = np.empty(B, np.int32)
        kl = np.empty(B, np.int32)
        self.lib.orc_kv_append(B, Tn, Tk, row_bytes, _p(new), _p(out), _p(kv), _p(nn), _p(qo),
                               _p(kl))
        return out, qo, kl


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def num_threads():
    return default().num_threads()


def score_row(*a, **k):
    return default().score_row(*a, **k)


def scores(*a, **k):
    return default().scores(*a, **k)


def topk(*a, **k):
    return default().topk(*a, **k)


def attention(*a, **k):
    return default().attention(*a, **k)


def layer(*a, **k):
    return default().layer(*a, **k)


def block_topk(*a, **k):
    return default().block_topk(*a, **k)


def attention_bwd(*a, **k):
    return default().attention_bwd(*a, **k)


def kv_append(*a, **k):
    return default().kv_append(*a, **k)


def indexer_bwd(*a, **k):
    return default().indexer_bwd(*a, **k)
