"""Thin Python binding of libhils.so (include/hils.h).

Argument marshalling only: every step of the HiLS forward pass runs in the HIP
kernels of the library.  torch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhils.so")

F32, BF16 = 0, 1
OP_COMPRESS, OP_SCORE_TOPK, OP_PREFILL, OP_DECODE, OP_BACKWARD, OP_DECODE_MIRROR, OP_DENSE_DECODE = 0, 1, 2, 3, 4, 5, 6
OK, E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4

SYMBOLS = ("hils_workspace_bytes", "hils_landmark_compress", "hils_chunk_score_topk", "hils_attn_prefill",
           "hils_attn_prefill_timed", "hils_attn_decode", "hils_attn_decode_timed", "hils_landmark_compress_paged",
           "hils_attn_decode_paged", "hils_dense_attention", "hils_attn_prefill_backward", "hils_attn_decode_noalloc",
           "hils_landmark_mirror", "hils_attn_decode_mirror", "hils_attn_decode_mirror_timed",
           "hils_attn_decode_paged_mirror", "hils_dense_decode", "hils_last_error")
NOALLOC_SCRATCH_BYTES = 16 << 20   # HILS_NOALLOC_SCRATCH_BYTES of include/hils.h
STAGES = ("compress", "score_threshold", "score_select", "bucket", "chunk_attend", "own_attend", "fuse")
DECODE_STAGES = ("scan", "merge", "attend_fuse")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "Hlmk", "d", "S", "K", "N", "qcal_rank", "io",
                                             "window")]

    def __repr__(self):
        return "Dims(%s)" % ", ".join("%s=%d" % (n, getattr(self, n)) for n, _ in self._fields_)


class HilsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


_lib = None


def load():
    """Load libhils.so (built in-tree by long_context_chunk_amd.build.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhils.so is not built (%s); run long_context_chunk_amd.build.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        lib.hils_workspace_bytes.argtypes = [dp, ctypes.c_int]
        lib.hils_workspace_bytes.restype = sz
        lib.hils_landmark_compress.argtypes = [dp, vp, vp, i32, i32, vp, vp, vp]
        lib.hils_chunk_score_topk.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_prefill.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_prefill_timed.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                ctypes.POINTER(ctypes.c_float)]
        lib.hils_attn_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_decode_timed.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                               ctypes.POINTER(ctypes.c_float)]
        lib.hils_dense_attention.argtypes = [dp, vp, vp, vp, vp, vp]
        lib.hils_dense_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.hils_landmark_compress_paged.argtypes = [dp, vp, vp, i32, i32, vp, i32, i32, vp, vp, vp]
        lib.hils_attn_decode_paged.argtypes = [dp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_decode_paged_mirror.argtypes = [dp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                      sz, vp]
        lib.hils_attn_prefill_backward.argtypes = [dp] + [vp] * 18 + [sz, vp]
        lib.hils_landmark_mirror.argtypes = [dp, vp, vp, i32, i32, vp, vp]
        lib.hils_attn_decode_mirror.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.hils_attn_decode_mirror_timed.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                      ctypes.POINTER(ctypes.c_float)]
        for f in ("hils_landmark_compress", "hils_chunk_score_topk", "hils_attn_prefill", "hils_attn_prefill_timed",
                  "hils_attn_decode", "hils_attn_decode_timed", "hils_dense_attention", "hils_landmark_compress_paged",
                  "hils_attn_decode_paged", "hils_attn_prefill_backward", "hils_attn_decode_noalloc",
                  "hils_landmark_mirror", "hils_attn_decode_mirror", "hils_attn_decode_mirror_timed",
                  "hils_attn_decode_paged_mirror", "hils_dense_decode"):
            getattr(lib, f).restype = ctypes.c_int
        lib.hils_last_error.argtypes = []
        lib.hils_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def dims(B, Hq, Hkv, d, N, K, S=64, qcal_rank=0, io=BF16, Hlmk=None, window=0) -> Dims:
    """window: local window in tokens (a multiple of S; 0 = the own chunk only)."""
    return Dims(B, Hq, Hkv, Hq if Hlmk is None else Hlmk, d, S, K, N, qcal_rank, io, window)


def _check(rc):
    if rc != OK:
        raise HilsError(rc, load().hils_last_error().decode())


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _io(t) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("io tensors must be bfloat16 or float32, got %s" % t.dtype)


def _req(t, name, shape=None, dtype=None):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous CUDA tensor" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return t


def workspace_bytes(dm: Dims, op: int) -> int:
    n = load().hils_workspace_bytes(ctypes.byref(dm), op)
    if n == ctypes.c_size_t(-1).value:
        raise HilsError(E_INVAL, load().hils_last_error().decode())
    return n


def workspace(dm: Dims, op: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(1, workspace_bytes(dm, op)), dtype=torch.uint8, device=device)


def landmark_compress(dm: Dims, k, lmk_q, kc, bc, c_begin=0, c_end=None):
    C = dm.N // dm.S
    c_end = C if c_end is None else c_end
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(k, "k", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(lmk_q, "lmk_q", (dm.B, dm.Hlmk, C, dm.d), dt)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _check(load().hils_landmark_compress(ctypes.byref(dm), _p(k), _p(lmk_q), c_begin, c_end, _p(kc), _p(bc),
                                         _stream()))


def chunk_score_topk(dm: Dims, q, kc, bc, sel_idx, sel_score, qcal_D=None, qcal_U=None, ws=None, q_pos0=None):
    """hils_chunk_score_topk for q [B, Hq, Nq, d]: query i of batch b at position q_pos0[b] + i
    (q_pos0: int32 [B] on the device, or None for 0) against the context's kc/bc."""
    C = dm.N // dm.S
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    if q is None or q.dim() != 4:
        raise ValueError("q must be [B, Hq, Nq, d]")
    Nq = q.shape[2]
    _req(q, "q", (dm.B, dm.Hq, Nq, dm.d), dt)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _req(sel_idx, "sel_idx", (dm.B, dm.Hq, Nq, dm.K), torch.int32)
    _req(sel_score, "sel_score", (dm.B, dm.Hq, Nq, dm.K), torch.float32)
    if q_pos0 is not None:
        _req(q_pos0, "q_pos0", (dm.B,), torch.int32)
    if dm.qcal_rank > 0:
        _req(qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d), dt)
        _req(qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank), dt)
    if ws is None:
        ws = workspace(dm, OP_SCORE_TOPK)
    nws = ws.numel()
    _check(load().hils_chunk_score_topk(ctypes.byref(dm), Nq, _p(q), _p(q_pos0), _p(qcal_D), _p(qcal_U), _p(kc), _p(bc),
                                        _p(sel_idx), _p(sel_score), _p(ws), nws, _stream()))


def attn_prefill(dm: Dims, q, k, v, o, ws, lmk_q=None, kc=None, bc=None, qcal_D=None, qcal_U=None, sel_idx=None,
                 sel_score=None, timed=False):
    """hils_attn_prefill (timed=True: hils_attn_prefill_timed, returns {stage: ms})."""
    C = dm.N // dm.S
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(q, "q", (dm.B, dm.Hq, dm.N, dm.d), dt)
    _req(k, "k", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(v, "v", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(o, "o", (dm.B, dm.Hq, dm.N, dm.d), dt)
    _req(ws, "ws", dtype=torch.uint8)
    if lmk_q is not None:
        _req(lmk_q, "lmk_q", (dm.B, dm.Hlmk, C, dm.d), dt)
    if kc is not None:
        _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
        _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    if dm.qcal_rank > 0:
        _req(qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d), dt)
        _req(qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank), dt)
    if sel_idx is not None:
        _req(sel_idx, "sel_idx", (dm.B, dm.Hq, dm.N, dm.K), torch.int32)
    if sel_score is not None:
        _req(sel_score, "sel_score", (dm.B, dm.Hq, dm.N, dm.K), torch.float32)
    args = (ctypes.byref(dm), _p(q), _p(k), _p(v), _p(lmk_q), _p(kc), _p(bc), _p(qcal_D), _p(qcal_U), _p(sel_idx),
            _p(sel_score), _p(o), _p(ws), ws.numel(), _stream())
    if timed:
        ms = (ctypes.c_float * len(STAGES))()
        _check(load().hils_attn_prefill_timed(*args, ms))
        return dict(zip(STAGES, [float(x) for x in ms]))
    _check(load().hils_attn_prefill(*args))


def attn_prefill_backward(dm: Dims, q, k, v, lmk_q, kc, sel_idx, sel_score, o, dO, dq, dk, dv, dlmk, ws,
                          qcal_D=None, qcal_U=None, dD=None, dU=None):
    """hils_attn_prefill_backward: gradients of sum(o * dO) with the forward's selection held fixed."""
    C = dm.N // dm.S
    dt = torch.bfloat16
    for t, n, shp in ((q, "q", (dm.B, dm.Hq, dm.N, dm.d)), (k, "k", (dm.B, dm.Hkv, dm.N, dm.d)),
                      (v, "v", (dm.B, dm.Hkv, dm.N, dm.d)), (o, "o", (dm.B, dm.Hq, dm.N, dm.d)),
                      (dO, "dO", (dm.B, dm.Hq, dm.N, dm.d)), (dq, "dq", (dm.B, dm.Hq, dm.N, dm.d)),
                      (dk, "dk", (dm.B, dm.Hkv, dm.N, dm.d)), (dv, "dv", (dm.B, dm.Hkv, dm.N, dm.d))):
        _req(t, n, shp, dt)
    if C > 0:
        _req(lmk_q, "lmk_q", (dm.B, dm.Hlmk, C, dm.d), dt)
        _req(dlmk, "dlmk", (dm.B, dm.Hlmk, C, dm.d), dt)
        _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(sel_idx, "sel_idx", (dm.B, dm.Hq, dm.N, dm.K), torch.int32)
    _req(sel_score, "sel_score", (dm.B, dm.Hq, dm.N, dm.K), torch.float32)
    _req(ws, "ws", dtype=torch.uint8)
    if dm.qcal_rank > 0:
        for t, n, shp in ((qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d)), (qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank)),
                          (dD, "dD", (dm.Hq, dm.qcal_rank, dm.d)), (dU, "dU", (dm.Hq, dm.d, dm.qcal_rank))):
            _req(t, n, shp, dt)
    _check(load().hils_attn_prefill_backward(ctypes.byref(dm), _p(q), _p(k), _p(v), _p(lmk_q), _p(kc), _p(qcal_D),
                                              _p(qcal_U), _p(sel_idx), _p(sel_score), _p(o), _p(dO), _p(dq), _p(dk),
                                              _p(dv), _p(dlmk), _p(dD), _p(dU), _p(ws), ws.numel(), _stream()))


def mirror_shape(dm: Dims):
    """Shape of the landmark mirror: a flat uint8 tensor of B*Hlmk*C*(d + 8) bytes, the signed
    8-bit codes of k' [B, Hlmk, C, d], then per row (b', the codes' scale) as fp32 pairs."""
    return (dm.B * dm.Hlmk * (dm.N // dm.S) * (dm.d + 8),)


def landmark_mirror(dm: Dims, kc, bc, kc_mirror, c_begin=0, c_end=None):
    """hils_landmark_mirror: rows [c_begin, c_end) of the bf16 landmark mirror from kc/bc."""
    C = dm.N // dm.S
    c_end = C if c_end is None else c_end
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _req(kc_mirror, "kc_mirror", mirror_shape(dm), torch.uint8)
    _check(load().hils_landmark_mirror(ctypes.byref(dm), _p(kc), _p(bc), c_begin, c_end, _p(kc_mirror), _stream()))


def attn_decode(dm: Dims, q, k_cache, v_cache, seq_lens, kc, bc, o, ws, qcal_D=None, qcal_U=None, sel_idx=None,
                timed=False, kc_mirror=None):
    """hils_attn_decode (timed=True: hils_attn_decode_timed, returns {stage: ms}); with
    kc_mirror (the landmark mirror), hils_attn_decode_mirror / hils_attn_decode_mirror_timed."""
    C = dm.N // dm.S
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(q, "q", (dm.B, dm.Hq, dm.d), dt)
    _req(k_cache, "k_cache", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(v_cache, "v_cache", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(seq_lens, "seq_lens", (dm.B,), torch.int32)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _req(o, "o", (dm.B, dm.Hq, dm.d), dt)
    _req(ws, "ws", dtype=torch.uint8)
    if dm.qcal_rank > 0:
        _req(qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d), dt)
        _req(qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank), dt)
    if sel_idx is not None:
        _req(sel_idx, "sel_idx", (dm.B, dm.Hq, dm.K), torch.int32)
    if kc_mirror is not None:
        _req(kc_mirror, "kc_mirror", mirror_shape(dm), torch.uint8)
        args = (ctypes.byref(dm), _p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(kc), _p(bc), _p(kc_mirror),
                _p(qcal_D), _p(qcal_U), _p(sel_idx), _p(o), _p(ws), ws.numel(), _stream())
        if timed:
            ms = (ctypes.c_float * len(DECODE_STAGES))()
            _check(load().hils_attn_decode_mirror_timed(*args, ms))
            return dict(zip(DECODE_STAGES, [float(x) for x in ms]))
        _check(load().hils_attn_decode_mirror(*args))
        return None
    args = (ctypes.byref(dm), _p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(kc), _p(bc), _p(qcal_D), _p(qcal_U),
            _p(sel_idx), _p(o), _p(ws), ws.numel(), _stream())
    if timed:
        ms = (ctypes.c_float * len(DECODE_STAGES))()
        _check(load().hils_attn_decode_timed(*args, ms))
        return dict(zip(DECODE_STAGES, [float(x) for x in ms]))
    _check(load().hils_attn_decode(*args))


def attn_decode_noalloc(dm: Dims, q, k_cache, v_cache, seq_lens, kc, bc, o, qcal_D=None, qcal_U=None, sel_idx=None):
    """hils_attn_decode_noalloc: hils_attn_decode with the library's own scratch (no workspace)."""
    C = dm.N // dm.S
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(q, "q", (dm.B, dm.Hq, dm.d), dt)
    _req(k_cache, "k_cache", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(v_cache, "v_cache", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(seq_lens, "seq_lens", (dm.B,), torch.int32)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _req(o, "o", (dm.B, dm.Hq, dm.d), dt)
    if dm.qcal_rank > 0:
        _req(qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d), dt)
        _req(qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank), dt)
    if sel_idx is not None:
        _req(sel_idx, "sel_idx", (dm.B, dm.Hq, dm.K), torch.int32)
    _check(load().hils_attn_decode_noalloc(ctypes.byref(dm), _p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(kc),
                                           _p(bc), _p(qcal_D), _p(qcal_U), _p(sel_idx), _p(o), _stream()))


def dense_attention(dm: Dims, q, k, v, o):
    """hils_dense_attention: the dense causal baseline on the same tensors."""
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(q, "q", (dm.B, dm.Hq, dm.N, dm.d), dt)
    _req(k, "k", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(v, "v", (dm.B, dm.Hkv, dm.N, dm.d), dt)
    _req(o, "o", (dm.B, dm.Hq, dm.N, dm.d), dt)
    _check(load().hils_dense_attention(ctypes.byref(dm), _p(q), _p(k), _p(v), _p(o), _stream()))


def dense_decode(dm: Dims, q, k_cache, v_cache, seq_lens, o, ws):
    """hils_dense_decode: the dense baseline of a decode step (every cached key, bf16)."""
    _req(q, "q", (dm.B, dm.Hq, dm.d), torch.bfloat16)
    _req(k_cache, "k_cache", (dm.B, dm.Hkv, dm.N, dm.d), torch.bfloat16)
    _req(v_cache, "v_cache", (dm.B, dm.Hkv, dm.N, dm.d), torch.bfloat16)
    _req(seq_lens, "seq_lens", (dm.B,), torch.int32)
    _req(o, "o", (dm.B, dm.Hq, dm.d), torch.bfloat16)
    _check(load().hils_dense_decode(ctypes.byref(dm), _p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(o), _p(ws),
                                    ws.numel() * ws.element_size(), _stream()))


def landmark_compress_paged(dm: Dims, k_pages, block_table, lmk_q, kc, bc, c_begin=0, c_end=None):
    """hils_landmark_compress_paged: k_pages [pages,Hkv,S,d], block_table [B,max_blocks] int32."""
    C = dm.N // dm.S
    c_end = C if c_end is None else c_end
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(k_pages, "k_pages", None, dt)
    _req(block_table, "block_table", (dm.B, C), torch.int32)
    _req(lmk_q, "lmk_q", (dm.B, dm.Hlmk, C, dm.d), dt)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _check(load().hils_landmark_compress_paged(ctypes.byref(dm), _p(k_pages), _p(block_table), C, k_pages.shape[0],
                                               _p(lmk_q), c_begin, c_end, _p(kc), _p(bc), _stream()))


def attn_decode_paged(dm: Dims, q, k_pages, v_pages, block_table, seq_lens, kc, bc, o, ws, qcal_D=None, qcal_U=None,
                      sel_idx=None, kc_mirror=None):
    """hils_attn_decode_paged: hils_attn_decode on a chunk-paged KV cache (with kc_mirror, the
    landmark mirror: hils_attn_decode_paged_mirror)."""
    C = dm.N // dm.S
    dt = torch.float32 if dm.io == F32 else torch.bfloat16
    _req(q, "q", (dm.B, dm.Hq, dm.d), dt)
    _req(k_pages, "k_pages", None, dt)
    _req(v_pages, "v_pages", tuple(k_pages.shape), dt)
    if tuple(k_pages.shape[1:]) != (dm.Hkv, dm.S, dm.d):
        raise ValueError("k_pages must be [pages, Hkv, S, d], got %s" % (tuple(k_pages.shape),))
    _req(block_table, "block_table", (dm.B, C), torch.int32)
    _req(seq_lens, "seq_lens", (dm.B,), torch.int32)
    _req(kc, "kc", (dm.B, dm.Hlmk, C, dm.d), torch.float32)
    _req(bc, "bc", (dm.B, dm.Hlmk, C), torch.float32)
    _req(o, "o", (dm.B, dm.Hq, dm.d), dt)
    _req(ws, "ws", dtype=torch.uint8)
    if dm.qcal_rank > 0:
        _req(qcal_D, "qcal_D", (dm.Hq, dm.qcal_rank, dm.d), dt)
        _req(qcal_U, "qcal_U", (dm.Hq, dm.d, dm.qcal_rank), dt)
    if sel_idx is not None:
        _req(sel_idx, "sel_idx", (dm.B, dm.Hq, dm.K), torch.int32)
    if kc_mirror is not None:
        _req(kc_mirror, "kc_mirror", mirror_shape(dm), torch.uint8)
        _check(load().hils_attn_decode_paged_mirror(ctypes.byref(dm), _p(q), _p(k_pages), _p(v_pages), _p(block_table),
                                                    C, k_pages.shape[0], _p(seq_lens), _p(kc), _p(bc), _p(kc_mirror),
                                                    _p(qcal_D), _p(qcal_U), _p(sel_idx), _p(o), _p(ws), ws.numel(),
                                                    _stream()))
        return
    _check(load().hils_attn_decode_paged(ctypes.byref(dm), _p(q), _p(k_pages), _p(v_pages), _p(block_table), C,
                                         k_pages.shape[0], _p(seq_lens), _p(kc), _p(bc), _p(qcal_D), _p(qcal_U),
                                         _p(sel_idx), _p(o), _p(ws), ws.numel(), _stream()))
