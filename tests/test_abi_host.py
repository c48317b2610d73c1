"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every symbol include/hils.h declares, the header compiles as C99, and argument
validation returns the documented error codes without touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from long_context_chunk_amd import hils

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hils_[a-z_]+)\s*\(", src)))


def test_header_compiles_as_c99():
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER])


def test_library_exports_every_declared_symbol():
    lib = hils.load()
    names = _declared_functions()
    assert set(names) == set(hils.SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.check_output(["nm", "-D", "--defined-only", hils.LIB_PATH], text=True)
    for n in names:
        assert re.search(r"\bT %s\b" % n, out), n


def _rc(fn, *args):
    return fn(*args)


def test_workspace_bytes():
    d = hils.dims(1, 32, 8, 128, 262144, 32, qcal_rank=32)
    n = hils.workspace_bytes(d, hils.OP_PREFILL)
    # the fp16 per-pair partial outputs dominate: B*Hq*N*K*d*2 bytes
    assert n >= 1 * 32 * 262144 * 32 * 128 * 2
    assert hils.workspace_bytes(d, hils.OP_COMPRESS) == 0
    assert hils.workspace_bytes(d, hils.OP_SCORE_TOPK) >= 2 * 32 * 4096 * 128 * 2   # k' bf16 planes
    dd = hils.dims(8, 32, 8, 128, 524288, 32)
    assert 0 < hils.workspace_bytes(dd, hils.OP_DECODE) < 64 << 20
    with pytest.raises(hils.HilsError):
        hils.workspace_bytes(dd, hils.OP_PREFILL)   # 32-bit pair ids: B*Hq*N*K >= 2^32
    with pytest.raises(hils.HilsError):
        hils.workspace_bytes(d, 7)


@pytest.mark.parametrize("field,value,code", [
    ("d", 96, hils.E_UNSUPPORTED), ("S", 32, hils.E_UNSUPPORTED), ("K", 0, hils.E_INVAL), ("K", 65, hils.E_UNSUPPORTED),
    ("Hkv", 3, hils.E_INVAL), ("Hlmk", 3, hils.E_INVAL), ("Hlmk", 2, hils.E_INVAL), ("B", 0, hils.E_INVAL), ("N", 0, hils.E_INVAL),
    ("io", 5, hils.E_UNSUPPORTED), ("qcal_rank", -1, hils.E_INVAL), ("qcal_rank", 64, hils.E_UNSUPPORTED),
    ("window", -64, hils.E_INVAL), ("window", 100, hils.E_INVAL), ("window", 33 * 64, hils.E_UNSUPPORTED),
])
def test_invalid_dims_rejected(field, value, code):
    lib = hils.load()
    d = hils.dims(1, 16, 4, 64, 1024, 16)
    setattr(d, field, value)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    rc = lib.hils_landmark_compress(ctypes.byref(d), fake, fake, 0, 1, fake, fake, None)
    assert rc == code, (rc, lib.hils_last_error())
    assert lib.hils_last_error()
    rc = lib.hils_attn_prefill(ctypes.byref(d), fake, fake, fake, None, fake, fake, None, None, None, None, fake,
                               fake, 1 << 40, None)
    assert rc == code


def test_window_workspace():
    """The local window adds decode slots (one per window chunk) and no prefill workspace."""
    d0 = hils.dims(2, 8, 2, 128, 4096, 16)
    d1 = hils.dims(2, 8, 2, 128, 4096, 16, window=512)
    d2 = hils.dims(2, 8, 2, 128, 4096, 16, window=64)
    assert hils.workspace_bytes(d1, hils.OP_PREFILL) <= hils.workspace_bytes(d0, hils.OP_PREFILL)
    assert hils.workspace_bytes(d2, hils.OP_PREFILL) == hils.workspace_bytes(d0, hils.OP_PREFILL)
    assert hils.workspace_bytes(d2, hils.OP_DECODE) == hils.workspace_bytes(d0, hils.OP_DECODE)
    # 7 more slots per (b, h): an fp32 output row and a score each
    assert hils.workspace_bytes(d1, hils.OP_DECODE) >= hils.workspace_bytes(d0, hils.OP_DECODE) + 2 * 8 * 7 * 128 * 4
    assert hils.workspace_bytes(hils.dims(1, 4, 1, 64, 4096, 32, window=32 * 64), hils.OP_DECODE) > 0


def test_null_pointers_and_ranges_rejected():
    lib = hils.load()
    d = hils.dims(1, 16, 4, 64, 1024, 16)
    fake = ctypes.c_void_p(0x1000)
    assert lib.hils_landmark_compress(None, fake, fake, 0, 1, fake, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_compress(ctypes.byref(d), None, fake, 0, 1, fake, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_compress(ctypes.byref(d), fake, fake, 5, 4, fake, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_compress(ctypes.byref(d), fake, fake, 0, 17, fake, fake, None) == hils.E_INVAL
    assert lib.hils_chunk_score_topk(ctypes.byref(d), 1024, fake, None, None, None, fake, fake, None, fake, None, 0,
                                     None) == hils.E_INVAL
    # prefill without landmark queries needs kc/bc
    assert lib.hils_attn_prefill(ctypes.byref(d), fake, fake, fake, None, None, None, None, None, None, None, fake,
                                 fake, 1 << 40, None) == hils.E_INVAL
    # Q-Cal rank without matrices
    dq = hils.dims(1, 16, 4, 64, 1024, 16, qcal_rank=8)
    assert lib.hils_attn_prefill(ctypes.byref(dq), fake, fake, fake, fake, fake, fake, None, None, None, None, fake,
                                 fake, 1 << 40, None) == hils.E_INVAL
    assert lib.hils_attn_decode(ctypes.byref(d), fake, fake, fake, None, fake, fake, None, None, None, fake, fake,
                                1 << 30, None) == hils.E_INVAL


def test_workspace_too_small_rejected():
    lib = hils.load()
    d = hils.dims(1, 16, 4, 64, 1024, 16)
    fake = ctypes.c_void_p(0x1000)
    need = hils.workspace_bytes(d, hils.OP_PREFILL)
    rc = lib.hils_attn_prefill(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None, None, None, None, fake, fake,
                               need - 1, None)
    assert rc == hils.E_WORKSPACE
    assert b"too small" in lib.hils_last_error()
    need = hils.workspace_bytes(d, hils.OP_DECODE)
    rc = lib.hils_attn_decode(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                              need - 1, None)
    assert rc == hils.E_WORKSPACE


def test_product_path_does_not_import_oracle():
    """The library binding and package never reference the oracle."""
    pkg = os.path.join(ROOT, "long_context_chunk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "hils_oracle" not in txt and "from oracle" not in txt, f


def test_dense_attention_validation():
    lib = hils.load()
    d = hils.dims(1, 4, 2, 64, 100, 4)
    fake = ctypes.c_void_p(0x1000)
    assert lib.hils_dense_attention(None, fake, fake, fake, fake, None) == hils.E_INVAL
    assert lib.hils_dense_attention(ctypes.byref(d), fake, None, fake, fake, None) == hils.E_INVAL
    bad = hils.dims(1, 4, 3, 64, 100, 4)   # Hq not a multiple of Hkv
    assert lib.hils_dense_attention(ctypes.byref(bad), fake, fake, fake, fake, None) == hils.E_INVAL
    bad = hils.dims(1, 4, 2, 96, 100, 4)   # unsupported head dim
    assert lib.hils_dense_attention(ctypes.byref(bad), fake, fake, fake, fake, None) == hils.E_UNSUPPORTED


def test_paged_entry_points_validation():
    lib = hils.load()
    d = hils.dims(2, 4, 2, 64, 1024, 8)   # N = 16 chunks
    fake = ctypes.c_void_p(0x1000)
    # capacity N must be max_blocks * S
    assert lib.hils_landmark_compress_paged(ctypes.byref(d), fake, fake, 15, 40, fake, 0, 1, fake, fake,
                                            None) == hils.E_INVAL
    assert lib.hils_landmark_compress_paged(ctypes.byref(d), fake, None, 16, 40, fake, 0, 1, fake, fake,
                                            None) == hils.E_INVAL
    assert lib.hils_landmark_compress_paged(ctypes.byref(d), fake, fake, 16, 0, fake, 0, 1, fake, fake,
                                            None) == hils.E_INVAL
    assert lib.hils_landmark_compress_paged(ctypes.byref(d), fake, fake, 16, 40, fake, 3, 2, fake, fake,
                                            None) == hils.E_INVAL
    need = hils.workspace_bytes(d, hils.OP_DECODE)
    assert lib.hils_attn_decode_paged(ctypes.byref(d), fake, fake, fake, fake, 8, 40, fake, fake, fake, None, None,
                                      None, fake, fake, need, None) == hils.E_INVAL
    assert lib.hils_attn_decode_paged(ctypes.byref(d), fake, fake, fake, fake, 16, 40, fake, fake, fake, None, None,
                                      None, fake, fake, need - 1, None) == hils.E_WORKSPACE


def test_backward_validation_and_workspace():
    """The backward entry: bf16 only, the documented NULL checks and the workspace size, checked
    before anything touches the device."""
    lib = hils.load()
    d = hils.dims(1, 8, 2, 64, 1024, 8)   # N = 16 chunks
    fake = ctypes.c_void_p(0x1000)
    need = hils.workspace_bytes(d, hils.OP_BACKWARD)
    # the bf16 per-pair dq partials alone: B*Hq*N*K*d*2 bytes
    assert need >= 1 * 8 * 1024 * 8 * 64 * 2
    dr = hils.dims(1, 8, 2, 64, 1024, 8, qcal_rank=4)
    assert hils.workspace_bytes(dr, hils.OP_BACKWARD) > need   # plus the per-head d x d sums

    def call(dm, lmk=fake, kc=fake, D=None, U=None, dlmk=fake, dD=None, dU=None, dq=fake, ws_bytes=need):
        return lib.hils_attn_prefill_backward(ctypes.byref(dm), fake, fake, fake, lmk, kc, D, U, fake, fake, fake,
                                              fake, dq, fake, fake, dlmk, dD, dU, fake, ws_bytes, None)

    assert call(d, dq=None) == hils.E_INVAL
    assert call(d, lmk=None) == hils.E_INVAL
    assert call(d, dlmk=None) == hils.E_INVAL
    assert call(dr, ws_bytes=1 << 40) == hils.E_INVAL            # Q-Cal without D, U, dD, dU
    assert call(d, ws_bytes=need - 1) == hils.E_WORKSPACE
    f32 = hils.dims(1, 8, 2, 64, 1024, 8, io=hils.F32)
    assert call(f32, ws_bytes=1 << 40) == hils.E_UNSUPPORTED
    assert b"bf16" in lib.hils_last_error()


def test_misaligned_tensor_pointers_rejected():
    """Tensor arguments must be 16-byte aligned (the kernels move rows with 16-byte
    accesses); a misaligned one is rejected on the host, before any HIP call."""
    lib = hils.load()
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x1008)      # 8-byte aligned only
    d = hils.dims(1, 8, 2, 64, 1024, 8)
    rc = lib.hils_attn_prefill(ctypes.byref(d), odd, fake, fake, fake, fake, fake, None, None, fake, fake, fake,
                               fake, ctypes.c_size_t(1 << 40), None)
    assert rc == hils.E_INVAL, (rc, lib.hils_last_error())
    assert b"16-byte aligned" in lib.hils_last_error()
    rc = lib.hils_dense_attention(ctypes.byref(d), fake, fake, fake, odd, None)
    assert rc == hils.E_INVAL and b"16-byte aligned" in lib.hils_last_error()
    dd = hils.dims(2, 8, 2, 64, 4096, 8)
    rc = lib.hils_attn_decode(ctypes.byref(dd), fake, odd, fake, fake, fake, fake, None, None, None, fake, fake,
                              ctypes.c_size_t(1 << 40), None)
    assert rc == hils.E_INVAL and b"16-byte aligned" in lib.hils_last_error()


def test_decode_noalloc_rejects_dims_beyond_its_scratch():
    """hils_attn_decode_noalloc checks its fixed scratch size on the host, before any HIP call."""
    lib = hils.load()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    big = hils.dims(64, 64, 8, 128, 1 << 20, 32)
    assert hils.workspace_bytes(big, hils.OP_DECODE) > hils.NOALLOC_SCRATCH_BYTES
    rc = lib.hils_attn_decode_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None, None, None, fake,
                                      None)
    assert rc == hils.E_UNSUPPORTED, (rc, lib.hils_last_error())
    assert b"scratch" in lib.hils_last_error()
    ok = hils.dims(8, 32, 8, 128, 524288, 32)   # the 512K decode workload fits
    assert hils.workspace_bytes(ok, hils.OP_DECODE) <= hils.NOALLOC_SCRATCH_BYTES
    rc = lib.hils_attn_decode_noalloc(ctypes.byref(ok), None, fake, fake, fake, fake, fake, None, None, None, fake, None)
    assert rc == hils.E_INVAL
    bad = hils.dims(8, 32, 8, 96, 4096, 32)
    rc = lib.hils_attn_decode_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None, None, None, fake, None)
    assert rc == hils.E_UNSUPPORTED


def test_landmark_heads_per_kv_group_accepted():
    """Hlmk = Hkv (one landmark head per KV group) is valid for every call, the backward
    pass included (it gets as far as the workspace check, with no workspace given)."""
    lib = hils.load()
    d = hils.dims(1, 16, 4, 64, 1024, 16, Hlmk=4)
    assert hils.workspace_bytes(d, hils.OP_PREFILL) > 0
    assert hils.workspace_bytes(d, hils.OP_SCORE_TOPK) >= 4 * 16 * (2 * 64 + 16) * 2   # k' planes of 4 landmark heads
    assert hils.workspace_bytes(d, hils.OP_BACKWARD) > 0
    fake = ctypes.c_void_p(0x1000)
    rc = lib.hils_attn_prefill_backward(ctypes.byref(d), *([fake] * 17), None, 0, None)
    assert rc == hils.E_WORKSPACE, lib.hils_last_error()


def test_k_above_32_limits():
    """K up to 64 is valid for every call, the backward pass included (it gets as far as
    the workspace check, with no workspace given); prefill also needs N*K < 2^26 (its
    bucketing keys) and says so before touching the device."""
    lib = hils.load()
    d = hils.dims(1, 16, 4, 64, 4096, 64)
    assert hils.workspace_bytes(d, hils.OP_PREFILL) > 0
    assert hils.workspace_bytes(d, hils.OP_DECODE) > 0
    assert hils.workspace_bytes(d, hils.OP_BACKWARD) > 0
    fake = ctypes.c_void_p(0x1000)
    rc = lib.hils_attn_prefill_backward(ctypes.byref(d), *([fake] * 17), None, 0, None)
    assert rc == hils.E_WORKSPACE, lib.hils_last_error()
    d65 = hils.dims(1, 16, 4, 64, 4096, 65)
    with pytest.raises(hils.HilsError):
        hils.workspace_bytes(d65, hils.OP_BACKWARD)
    big = hils.dims(1, 1, 1, 64, 16384 * 64, 64)   # N*K = 2^26
    with pytest.raises(hils.HilsError):
        hils.workspace_bytes(big, hils.OP_PREFILL)
    assert hils.workspace_bytes(big, hils.OP_DECODE) > 0


def test_score_topk_block_arguments():
    lib = hils.load()
    d = hils.dims(2, 4, 2, 64, 4096, 8)
    fake = ctypes.c_void_p(0x1000)
    args = lambda nq: (ctypes.byref(d), nq, fake, None, None, None, fake, fake, fake, fake, fake, 1 << 40, None)
    assert lib.hils_chunk_score_topk(*args(4097)) == hils.E_INVAL      # more queries than N
    assert lib.hils_chunk_score_topk(*args(-1)) == hils.E_INVAL
    # no query: nothing to do, NULL arrays allowed, nothing enqueued
    assert lib.hils_chunk_score_topk(ctypes.byref(d), 0, None, None, None, None, None, None, None, None, None, 0,
                                     None) == hils.OK


def test_mirror_entry_points_validation():
    """hils_landmark_mirror and hils_attn_decode_mirror(_timed) validate on the host: the
    chunk range, NULL buffers (the mirror may be NULL only without a complete chunk), and
    the decode's own checks; an empty range does nothing."""
    lib = hils.load()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    d = hils.dims(2, 8, 2, 128, 4096, 16)
    C = 4096 // 64
    assert lib.hils_landmark_mirror(ctypes.byref(d), fake, fake, 0, C + 1, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_mirror(ctypes.byref(d), fake, fake, 5, 4, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_mirror(ctypes.byref(d), fake, fake, -1, 4, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_mirror(ctypes.byref(d), None, fake, 0, 4, fake, None) == hils.E_INVAL
    assert lib.hils_landmark_mirror(ctypes.byref(d), fake, fake, 0, 4, None, None) == hils.E_INVAL
    assert lib.hils_landmark_mirror(ctypes.byref(d), None, None, 3, 3, None, None) == hils.OK
    bad = hils.dims(2, 8, 2, 96, 4096, 16)
    assert lib.hils_landmark_mirror(ctypes.byref(bad), fake, fake, 0, 4, fake, None) == hils.E_UNSUPPORTED
    ws_need = hils.workspace_bytes(d, hils.OP_DECODE_MIRROR)
    assert ws_need > hils.workspace_bytes(d, hils.OP_DECODE)   # plus the scan's survivor lists
    args = [fake, fake, fake, fake, fake, fake]
    rc = lib.hils_attn_decode_mirror(ctypes.byref(d), *args, None, None, None, None, fake, fake, ws_need, None)
    assert rc == hils.E_INVAL and b"kc_mirror" in lib.hils_last_error()
    rc = lib.hils_attn_decode_mirror(ctypes.byref(d), *args, fake, None, None, None, fake, fake, ws_need - 1, None)
    assert rc == hils.E_WORKSPACE
    rc = lib.hils_attn_decode_mirror(ctypes.byref(bad), *args, fake, None, None, None, fake, fake, 1 << 40, None)
    assert rc == hils.E_UNSUPPORTED
    ms = (ctypes.c_float * len(hils.DECODE_STAGES))()
    rc = lib.hils_attn_decode_mirror_timed(ctypes.byref(d), *args, fake, None, None, None, fake, fake, ws_need, None,
                                           None)
    assert rc == hils.E_INVAL and b"stage_ms" in lib.hils_last_error()
    rc = lib.hils_attn_decode_mirror_timed(ctypes.byref(d), *args, None, None, None, None, fake, fake, ws_need, None,
                                           ms)
    assert rc == hils.E_INVAL
    short = hils.dims(2, 8, 2, 128, 48, 16)   # N < S: no chunk, the mirror may be NULL
    rc = lib.hils_attn_decode_mirror(ctypes.byref(short), fake, fake, fake, fake, None, None, None, None, None, None,
                                     None, fake, 1 << 40, None)
    assert rc == hils.E_INVAL and b"o must" in lib.hils_last_error()


def test_paged_mirror_entry_point_validation():
    """hils_attn_decode_paged_mirror checks the mirror, the page table and the decode
    arguments on the host."""
    lib = hils.load()
    fake = ctypes.c_void_p(0x1000)
    d = hils.dims(2, 8, 2, 128, 4096, 16)
    C = 4096 // 64
    need = hils.workspace_bytes(d, hils.OP_DECODE_MIRROR)
    rc = lib.hils_attn_decode_paged_mirror(ctypes.byref(d), fake, fake, fake, fake, C, 4 * C, fake, fake, fake, None,
                                           None, None, None, fake, fake, need, None)
    assert rc == hils.E_INVAL and b"kc_mirror" in lib.hils_last_error()
    rc = lib.hils_attn_decode_paged_mirror(ctypes.byref(d), fake, fake, fake, None, C, 4 * C, fake, fake, fake, fake,
                                           None, None, None, fake, fake, need, None)
    assert rc == hils.E_INVAL
    rc = lib.hils_attn_decode_paged_mirror(ctypes.byref(d), fake, fake, fake, fake, C + 1, 4 * C, fake, fake, fake,
                                           fake, None, None, None, fake, fake, need, None)
    assert rc == hils.E_INVAL
    rc = lib.hils_attn_decode_paged_mirror(ctypes.byref(d), fake, fake, fake, fake, C, 4 * C, fake, fake, fake, fake,
                                           None, None, None, fake, fake, need - 1, None)
    assert rc == hils.E_WORKSPACE


def test_decode_chunk_limit():
    """Decode takes up to 65536 chunks (4M tokens at S = 64); prefill and scoring 16384."""
    ok = hils.dims(1, 2, 1, 64, 65536 * 64, 16)
    assert hils.workspace_bytes(ok, hils.OP_DECODE) > 0
    assert hils.workspace_bytes(ok, hils.OP_DECODE_MIRROR) > hils.workspace_bytes(ok, hils.OP_DECODE)
    for op in (hils.OP_DECODE, hils.OP_DECODE_MIRROR):
        with pytest.raises(hils.HilsError):
            hils.workspace_bytes(hils.dims(1, 2, 1, 64, 65537 * 64, 16), op)
    with pytest.raises(hils.HilsError):
        hils.workspace_bytes(hils.dims(1, 2, 1, 64, 16385 * 64, 16), hils.OP_PREFILL)


def test_dense_decode_validation():
    """hils_dense_decode checks its arguments before touching the device: bf16 only,
    Hq/Hkv in {1, 2, 4, 8}, non-NULL tensors, a workspace of the size it reports."""
    lib = hils.load()
    fake = ctypes.c_void_p(0x1000)
    ok = hils.dims(2, 8, 2, 128, 4096, 8)
    need = hils.workspace_bytes(ok, hils.OP_DENSE_DECODE)
    assert need == 2 * 8 * 2 * (128 + 2) * 4          # B * Hq * ceil(N / 2048) partials of d + 2 floats
    assert lib.hils_dense_decode(ctypes.byref(ok), fake, fake, fake, fake, fake, None, 0, None) == hils.E_WORKSPACE
    assert lib.hils_dense_decode(ctypes.byref(ok), None, fake, fake, fake, fake, fake, need, None) == hils.E_INVAL
    g3 = hils.dims(2, 6, 2, 128, 4096, 8)
    assert lib.hils_dense_decode(ctypes.byref(g3), fake, fake, fake, fake, fake, fake, 1 << 30, None) == \
        hils.E_UNSUPPORTED
    f32 = hils.dims(2, 8, 2, 128, 4096, 8, io=hils.F32)
    assert lib.hils_dense_decode(ctypes.byref(f32), fake, fake, fake, fake, fake, fake, 1 << 30, None) == \
        hils.E_UNSUPPORTED
