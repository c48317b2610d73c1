"""Seeded synthetic inputs shaped like the HiLS-Attention workloads.

This package makes inputs only (no attention arithmetic).  The numbers come
from ``synth.c`` (a counter-based SplitMix64 + Box-Muller generator), so the
oracle and the GPU path always see identical bits.

Workload structure (stands in for the retrieval benchmarks the pages evaluate
on, which are not available here):
  * k, v, landmark queries: iid N(0, 1); Q-Cal D, U: iid N(0, 0.02^2);
  * one seeded unit vector u in R^d;
  * needle chunks: round(f * C) of them, one drawn uniformly inside each of
    that many equal strata of the chunk range, so they spread over the whole
    sequence; every key of a needle chunk (all KV heads) gets + 3 u;
  * planted queries: exactly round(0.25 * N) token positions, uniform without
    replacement, get + 2 u on all query heads (decode: 2 of the B sequences).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16, F64 = 0, 1, 2

# tensor ids of the generator streams
T_Q, T_K, T_V, T_LMK, T_D, T_U, T_DIR, T_NEEDLE, T_QPLANT, T_SEQPLANT = range(1, 11)

BASE_SEED = 0x48694C53


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp,
                               os.path.join(_HERE, "synth.c"), "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u64, vp, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        lib.synth_uniform.argtypes = [vp, i64, u64, u64]
        lib.synth_normal.argtypes = [vp, ctypes.c_int, i64, u64, u64, dbl]
        lib.synth_tokens.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, u64, u64, dbl, vp, dbl, vp]
        for f in (lib.synth_uniform, lib.synth_normal, lib.synth_tokens):
            f.restype = None
        _lib = lib
    return _lib


def _np_dtype(dtype: int):
    return {F32: np.float32, BF16: np.uint16, F64: np.float64}[dtype]


def uniform(n: int, seed: int, tid: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform(out.ctypes.data, n, seed, tid)
    return out


def normal(shape, seed: int, tid: int, dtype: int = F64, scale: float = 1.0) -> np.ndarray:
    out = np.empty(shape, _np_dtype(dtype))
    _load().synth_normal(out.ctypes.data, dtype, out.size, seed, tid, scale)
    return out


def tokens(B, H, N, d, seed, tid, dtype, scale=1.0, u=None, alpha=0.0, mask=None) -> np.ndarray:
    """[B, H, N, d] tensor; rows whose token (b, n) has mask[b, n] get + alpha * u."""
    out = np.empty((B, H, N, d), _np_dtype(dtype))
    uptr = mptr = None
    if u is not None and mask is not None:
        u = np.ascontiguousarray(u, np.float64)
        mask = np.ascontiguousarray(mask, np.uint8)
        assert mask.shape == (B, N)
        uptr, mptr = u.ctypes.data, mask.ctypes.data
    _load().synth_tokens(out.ctypes.data, dtype, B, H, N, d, seed, tid, scale, uptr, alpha, mptr)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def round_half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


def unit_vector(d: int, seed: int) -> np.ndarray:
    z = normal(d, seed, T_DIR)
    return z / np.linalg.norm(z)


def needle_chunks(C: int, frac: float, seed: int, stream: int) -> np.ndarray:
    """One uniformly drawn chunk in each of round(frac*C) equal strata of [0, C)."""
    n = round_half_up(frac * C)
    if n <= 0:
        return np.zeros(0, np.int64)
    uu = uniform(n, seed, T_NEEDLE + 64 * stream)
    s = np.arange(n, dtype=np.int64)
    lo, hi = (s * C) // n, ((s + 1) * C) // n
    return lo + np.floor(uu * (hi - lo)).astype(np.int64)


def planted_positions(N: int, frac: float, seed: int, stream: int) -> np.ndarray:
    """Exactly round(frac*N) distinct positions of [0, N), uniform without replacement."""
    n = round_half_up(frac * N)
    keys = uniform(N, seed, T_QPLANT + 64 * stream)
    return np.sort(np.argsort(keys, kind="stable")[:n])


@dataclass
class Workload:
    """Shapes of one HiLS workload.  Names follow the pages' notation."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int                 # prefill tokens / decode cache capacity
    S: int = 64
    K: int = 16
    io: int = BF16
    qcal_rank: int = 0
    Hlmk: int = 0          # 0 -> Hq (one landmark query per chunk per query head)
    planted: bool = True
    needle_frac: float = 0.02
    query_frac: float = 0.25
    decode: bool = False
    seq_lens: list = field(default_factory=list)   # decode: cache length per sequence
    planted_seqs: int = 2                          # decode: sequences whose query gets + 2u
    window: int = 0        # local window in tokens (a multiple of S; 0 = the own chunk only)

    def __post_init__(self):
        if self.Hlmk == 0:
            self.Hlmk = self.Hq

    @property
    def C(self) -> int:
        return self.N // self.S

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads: a tiny fp32 case, a 345M-like 8K layer, a 128K layer,
# a 7B-like decode step at 512K and a 7B-like 256K prefill with Q-Cal.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, Hq=1, Hkv=1, d=64, N=1024, K=4, io=F32, planted=False),
    "prefill_8k": Workload("prefill_8k", B=1, Hq=16, Hkv=4, d=64, N=8192, K=16),
    "prefill_128k": Workload("prefill_128k", B=1, Hq=16, Hkv=4, d=64, N=131072, K=16),
    "decode_512k": Workload("decode_512k", B=8, Hq=32, Hkv=8, d=128, N=524288, K=32, needle_frac=0.01,
                            decode=True, seq_lens=[524288] * 8),
    "prefill_256k_qcal": Workload("prefill_256k_qcal", B=1, Hq=32, Hkv=8, d=128, N=262144, K=32,
                                  qcal_rank=32),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of w with some fields replaced (for smaller test shapes)."""
    import dataclasses
    if "Hq" in kw and "Hlmk" not in kw:
        kw["Hlmk"] = 0          # one landmark head per query head again
    return dataclasses.replace(w, **kw)


def make_inputs(w: Workload, seed: int) -> dict:
    """All input arrays of workload w as numpy arrays (bf16 as uint16 bit patterns).

    prefill: q [B,Hq,N,d], k, v [B,Hkv,N,d], lmk [B,Hlmk,C,d], (D [Hq,r,d], U [Hq,d,r])
    decode:  q [B,Hq,d],  k, v [B,Hkv,N,d] caches, lmk [B,Hlmk,C,d], seq_lens [B] int32, (D, U)
    """
    B, N, d, C = w.B, w.N, w.d, w.C
    out = {"seed": seed}
    u = unit_vector(d, seed)
    kmask = np.zeros((B, N), np.uint8)
    if w.planted:
        for b in range(B):
            for c in needle_chunks(C, w.needle_frac, seed, b):
                kmask[b, c * w.S:(c + 1) * w.S] = 1
    out["k"] = tokens(B, w.Hkv, N, d, seed, T_K, w.io, 1.0, u, 3.0, kmask)
    out["v"] = tokens(B, w.Hkv, N, d, seed, T_V, w.io)
    out["lmk"] = tokens(B, w.Hlmk, C, d, seed, T_LMK, w.io)
    if w.decode:
        qmask = np.zeros((B, 1), np.uint8)
        if w.planted and w.planted_seqs > 0:
            keys = uniform(B, seed, T_SEQPLANT)
            qmask[np.argsort(keys, kind="stable")[:w.planted_seqs], 0] = 1
        out["q"] = tokens(B, w.Hq, 1, d, seed, T_Q, w.io, 1.0, u, 2.0, qmask).reshape(B, w.Hq, d)
        lens = list(w.seq_lens) if w.seq_lens else [N] * B
        out["seq_lens"] = np.asarray(lens, np.int32)
    else:
        qmask = np.zeros((B, N), np.uint8)
        if w.planted:
            for b in range(B):
                qmask[b, planted_positions(N, w.query_frac, seed, b)] = 1
        out["q"] = tokens(B, w.Hq, N, d, seed, T_Q, w.io, 1.0, u, 2.0, qmask)
    if w.qcal_rank > 0:
        r = w.qcal_rank
        out["D"] = normal((w.Hq, r, d), seed, T_D, w.io, 0.02)
        out["U"] = normal((w.Hq, d, r), seed, T_U, w.io, 0.02)
    return out
