"""fp64 CPU oracle of the HiLS-Attention forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  The
arithmetic is in ``hils_oracle.c`` (plain C, double precision); this file only
marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhils_oracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2
LANDMARK, EXACT, GIVEN = 0, 1, 2


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "Hl", "d", "S", "K", "N", "r", "W")]


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp,
                               os.path.join(_HERE, "hils_oracle.c"), "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sp = ctypes.POINTER(Shape)
        lib.hr_compress.argtypes = [sp, vp, i32, vp, i32, vp, vp]
        lib.hr_qcal.argtypes = [sp, i32, vp, vp, vp, i32, vp]
        lib.hr_row_scores.argtypes = [sp, i32, i32, i32, i32, vp, i32, vp, i32, vp, vp, vp, vp, i32, vp]
        lib.hr_row_scores.restype = ctypes.c_int
        lib.hr_attend.argtypes = [sp, i32, i64, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32,
                                  vp, vp, vp, vp, vp, vp, vp]
        lib.hr_dense.argtypes = [sp, i64, vp, vp, vp, vp, i32, vp, vp, i32, vp]
        lib.hr_attend_backward.argtypes = [sp, i64, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, vp, i32,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        for f in (lib.hr_compress, lib.hr_qcal, lib.hr_attend, lib.hr_dense, lib.hr_attend_backward):
            f.restype = None
        _lib = lib
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("unsupported dtype %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def shape(B, Hq, Hkv, d, N, S=64, K=16, Hl=None, r=0, W=0) -> Shape:
    """W: local window in tokens (a multiple of S; 0 = S, the own chunk only)."""
    return Shape(B, Hq, Hkv, Hq if Hl is None else Hl, d, S, K, N, r, W)


def compress(s: Shape, k: np.ndarray, lmk: np.ndarray):
    """k' [B,Hl,C,d] and b' [B,Hl,C] (float64) of every complete chunk."""
    k, lmk = np.ascontiguousarray(k), np.ascontiguousarray(lmk)
    C = s.N // s.S
    kc = np.empty((s.B, s.Hl, C, s.d), np.float64)
    bc = np.empty((s.B, s.Hl, C), np.float64)
    _load().hr_compress(ctypes.byref(s), k.ctypes.data, _dt(k), lmk.ctypes.data, _dt(lmk),
                        kc.ctypes.data, bc.ctypes.data)
    return kc, bc


def qcal(s: Shape, h: int, q: np.ndarray, D=None, U=None) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    out = np.empty(s.d, np.float64)
    wdt = _dt(D) if D is not None else F64
    _load().hr_qcal(ctypes.byref(s), h, q.ctypes.data, _ptr(D), _ptr(U), wdt, out.ctypes.data)
    return out


def row_scores(s: Shape, b, h, pos, qrow, k=None, kc=None, bc=None, D=None, U=None, mode=LANDMARK):
    """The score of every candidate chunk of one query (the complete chunks before the window)."""
    qrow = np.ascontiguousarray(qrow)
    out = np.empty(max(1, min(pos // s.S, s.N // s.S)), np.float64)
    kdt = _dt(k) if k is not None else F64
    wdt = _dt(D) if D is not None else F64
    n = _load().hr_row_scores(ctypes.byref(s), mode, b, h, pos, qrow.ctypes.data, _dt(qrow), _ptr(k), kdt,
                              _ptr(kc), _ptr(bc), _ptr(D), _ptr(U), wdt, out.ctypes.data)
    return out[:n]


def attend(s: Shape, rows_b, rows_h, rows_pos, qrows, k, v, kc=None, bc=None, D=None, U=None,
           mode=LANDMARK, sel_in=None):
    """Full forward pass for a list of queries.

    qrows [n, d] are the query vectors (any of f64/f32/bf16-bits); the rest as in
    hils_oracle.h.  Returns a dict of o, sel_idx, sel_score, gap, lse_own, nsel.
    """
    rb = np.ascontiguousarray(rows_b, np.int32)
    rh = np.ascontiguousarray(rows_h, np.int32)
    rp = np.ascontiguousarray(rows_pos, np.int32)
    n = rb.size
    qrows = np.ascontiguousarray(qrows).reshape(n, s.d)
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    assert k.dtype == v.dtype
    o = np.empty((n, s.d), np.float64)
    sel_idx = np.empty((n, s.K), np.int32)
    sel_score = np.empty((n, s.K), np.float64)
    gap = np.empty(n, np.float64)
    lse = np.empty(n, np.float64)
    nsel = np.empty(n, np.int32)
    if sel_in is not None:
        sel_in = np.ascontiguousarray(sel_in, np.int32).reshape(n, s.K)
        mode = GIVEN
    wdt = _dt(D) if D is not None else F64
    if kc is not None:
        kc = np.ascontiguousarray(kc, np.float64)
        bc = np.ascontiguousarray(bc, np.float64)
    _load().hr_attend(ctypes.byref(s), mode, n, rb.ctypes.data, rh.ctypes.data, rp.ctypes.data,
                      qrows.ctypes.data, _dt(qrows), k.ctypes.data, v.ctypes.data, _dt(k), _ptr(kc),
                      _ptr(bc), _ptr(D), _ptr(U), wdt, _ptr(sel_in), o.ctypes.data, sel_idx.ctypes.data,
                      sel_score.ctypes.data, gap.ctypes.data, lse.ctypes.data, nsel.ctypes.data)
    return {"o": o, "sel_idx": sel_idx, "sel_score": sel_score, "gap": gap, "lse_own": lse, "nsel": nsel}


def prefill_rows(s: Shape, q, k, v, kc, bc, rows, D=None, U=None, mode=LANDMARK):
    """Forward pass for prefill queries rows = [(b, h, i), ...] of q [B,Hq,N,d]."""
    rows = np.asarray(rows, np.int64).reshape(-1, 3)
    qrows = q[rows[:, 0], rows[:, 1], rows[:, 2], :]
    return attend(s, rows[:, 0], rows[:, 1], rows[:, 2], qrows, k, v, kc, bc, D, U, mode)


def dense(s: Shape, rows_b, rows_h, rows_pos, qrows, k, v):
    """Dense causal attention for a list of queries (the baseline); returns o [n, d]."""
    rb = np.ascontiguousarray(rows_b, np.int32)
    rh = np.ascontiguousarray(rows_h, np.int32)
    rp = np.ascontiguousarray(rows_pos, np.int32)
    n = rb.size
    qrows = np.ascontiguousarray(qrows).reshape(n, s.d)
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    assert k.dtype == v.dtype
    o = np.empty((n, s.d), np.float64)
    _load().hr_dense(ctypes.byref(s), n, rb.ctypes.data, rh.ctypes.data, rp.ctypes.data, qrows.ctypes.data,
                     _dt(qrows), k.ctypes.data, v.ctypes.data, _dt(k), o.ctypes.data)
    return o


def attend_backward(s: Shape, rows_b, rows_h, rows_pos, qrows, k, v, kc, bc, lmk, sel_idx, dO, D=None, U=None):
    """Gradients of attend()'s output o for the given rows, with their selections sel_idx
    [n, K] held fixed and output gradients dO [n, d].  Returns a dict of dq [n, d], dk, dv
    [B,Hkv,N,d], dkc [B,Hl,C,d], dbc [B,Hl,C], dlmk [B,Hl,C,d], dD [Hq,r,d], dU [Hq,d,r]."""
    rb = np.ascontiguousarray(rows_b, np.int32)
    rh = np.ascontiguousarray(rows_h, np.int32)
    rp = np.ascontiguousarray(rows_pos, np.int32)
    n = rb.size
    qrows = np.ascontiguousarray(qrows).reshape(n, s.d)
    k, v, lmk = np.ascontiguousarray(k), np.ascontiguousarray(v), np.ascontiguousarray(lmk)
    kc = np.ascontiguousarray(kc, np.float64)
    bc = np.ascontiguousarray(bc, np.float64)
    sel = np.ascontiguousarray(sel_idx, np.int32).reshape(n, s.K)
    dO = np.ascontiguousarray(dO, np.float64).reshape(n, s.d)
    C = s.N // s.S
    out = {"dq": np.empty((n, s.d)), "dk": np.empty((s.B, s.Hkv, s.N, s.d)), "dv": np.empty((s.B, s.Hkv, s.N, s.d)),
           "dkc": np.empty((s.B, s.Hl, C, s.d)), "dbc": np.empty((s.B, s.Hl, C)), "dlmk": np.empty((s.B, s.Hl, C, s.d)),
           "dD": np.zeros((s.Hq, max(s.r, 0), s.d)), "dU": np.zeros((s.Hq, s.d, max(s.r, 0)))}
    wdt = _dt(D) if D is not None else F64
    _load().hr_attend_backward(ctypes.byref(s), n, rb.ctypes.data, rh.ctypes.data, rp.ctypes.data, qrows.ctypes.data,
                               _dt(qrows), k.ctypes.data, v.ctypes.data, _dt(k), kc.ctypes.data, bc.ctypes.data,
                               lmk.ctypes.data, _dt(lmk), _ptr(D), _ptr(U), wdt, sel.ctypes.data, dO.ctypes.data,
                               out["dq"].ctypes.data, out["dk"].ctypes.data, out["dv"].ctypes.data,
                               out["dkc"].ctypes.data, out["dbc"].ctypes.data, out["dlmk"].ctypes.data,
                               out["dD"].ctypes.data if s.r > 0 else None, out["dU"].ctypes.data if s.r > 0 else None)
    return out
