"""The landmark mirror (hils_landmark_mirror) and the decode step that scans it
(hils_attn_decode_mirror).

The mirror decode promises the result of hils_attn_decode bit for bit: its scan only
bounds every chunk's score from the 8-bit codes of k', and every chunk that can reach
the top K is rescored exactly.  So each case here runs both calls on the same inputs and
compares the selections and outputs bit for bit, and checks the mirror decode against
the fp64 oracle as the other decode tests do.  The mirror itself is checked against its
definition (signed codes rint(k' * fl(127 / m)), scale fl(m / 127), b' bit for bit) and
against the error bound the scan relies on, |k'_e - s code_e| <= s (1/2 + 2^-16).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hils_testutil import check_selection_and_output, dims_of, gpu_compress, gpu_decode, oracle_compress, shape_of
from long_context_chunk_amd import hils
from test_gpu_parity import DECODE_FUSED, DECODE_LONG, DECODE_SMALL, DECODE_WINDOW, TIE_DECODE, _assert_tie_rows, _twin_inputs

pytestmark = pytest.mark.gpu

SEED = synth.BASE_SEED


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _decode_rows(w, x):
    rows_b = [b for b in range(w.B) for h in range(w.Hq)]
    rows_h = [h for b in range(w.B) for h in range(w.Hq)]
    pos = [int(x["seq_lens"][b]) - 1 for b in rows_b]
    return rows_b, rows_h, pos


class _QView:
    """Indexes the decode queries [B, Hq, d] as [b, h, i] (check_selection_and_output's form)."""

    def __init__(self, q):
        self.q = q

    def __getitem__(self, key):
        b, h, _ = key
        return self.q[b, h]


def _check_against_oracle(w, x, g, label):
    kc_o, bc_o = oracle_compress(w, x)
    rows_b, rows_h, pos = _decode_rows(w, x)
    ref = oracle.attend(shape_of(w), rows_b, rows_h, pos, x["q"].reshape(-1, w.d), x["k"], x["v"], kc_o, bc_o,
                        D=x.get("D"), U=x.get("U"))
    xx = dict(x)
    xx["q"] = _QView(x["q"])
    return ref, check_selection_and_output(w, xx, kc_o, bc_o, list(zip(rows_b, rows_h, pos)), ref,
                                           g["sel_idx"].reshape(-1, w.K), None, g["o"].reshape(-1, w.d), label=label)


def _assert_same_step(a, b, label):
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"], err_msg=label + ": selections differ")
    np.testing.assert_array_equal(a["o_bits"], b["o_bits"], err_msg=label + ": outputs differ")


MIRROR_ROWS = [
    ("bf16_d128", synth.Workload("mir_a", B=2, Hq=4, Hkv=2, d=128, N=5000, K=8, decode=True, seq_lens=[5000, 77])),
    ("f32_d64_shared_lmk", synth.Workload("mir_b", B=2, Hq=4, Hkv=2, d=64, N=4100, K=8, io=synth.F32, decode=True,
                                          seq_lens=[4100, 4100], Hlmk=2, planted=False)),
]


@pytest.mark.parametrize("name,w", MIRROR_ROWS, ids=[n for n, _ in MIRROR_ROWS])
def test_mirror_rows(name, w):
    """The code plane and the (b', scale) plane against their definition and the bound;
    a chunk range leaves the other chunks of both planes alone; an all-zero chunk gets
    codes 0 and scale 0."""
    _say("mirror rows", name)
    x = synth.make_inputs(w, SEED + 5)
    dm = dims_of(w)
    kc, bc = gpu_compress(w, x)
    kc[:, :, 4] = 0.0
    torch.cuda.synchronize()
    sentinel = 0x5A
    kcm = torch.full(hils.mirror_shape(dm), sentinel, dtype=torch.uint8, device="cuda")
    c0, c1 = 3, w.C - 5
    hils.landmark_mirror(dm, kc, bc, kcm, c0, c1)
    torch.cuda.synchronize()
    m = kcm.cpu().numpy()
    kcn, bcn = kc.cpu().numpy(), bc.cpu().numpy()
    d, R = w.d, w.B * w.Hlmk * w.C
    codes = m[:R * d].view(np.int8).reshape(w.B, w.Hlmk, w.C, d)
    pairs = m[R * d:].view(np.uint32).reshape(w.B, w.Hlmk, w.C, 2)
    for plane, fill in ((codes, sentinel), (pairs, sentinel * 0x01010101)):   # 0x5A < 128: the same as int8
        assert np.all(plane[:, :, :c0] == fill) and np.all(plane[:, :, c1:] == fill), "chunks outside the range changed"
    k = kcn[:, :, c0:c1]
    mx = np.max(np.abs(k), axis=-1)
    with np.errstate(divide="ignore"):
        inv = np.where(mx > 0, np.float32(127.0) / mx, np.float32(0.0)).astype(np.float32)
    want = np.rint(k * inv[..., None]).astype(np.int64)
    np.testing.assert_array_equal(codes[:, :, c0:c1].astype(np.int64), want)
    np.testing.assert_array_equal(pairs[:, :, c0:c1, 0], bcn[:, :, c0:c1].view(np.uint32))
    sc = pairs[:, :, c0:c1, 1].view(np.float32)
    np.testing.assert_array_equal(sc, (mx / np.float32(127.0)).astype(np.float32))
    assert np.all(codes[:, :, 4] == 0) and np.all(sc[:, :, 4 - c0] == 0)
    err = np.abs(k.astype(np.float64) - sc[..., None].astype(np.float64) * codes[:, :, c0:c1])
    assert np.all(err <= sc[..., None] * (0.5 + 2.0 ** -16)), "a code misses its bound"
    # the empty range writes nothing
    hils.landmark_mirror(dm, kc, bc, kcm, 7, 7)
    torch.cuda.synchronize()
    assert np.array_equal(kcm.cpu().numpy(), m)


MIRROR_DECODE = DECODE_SMALL + DECODE_WINDOW + DECODE_FUSED + DECODE_LONG + [
    ("bf16_d128_shared_lmk_qcal", synth.Workload("mir_shl", B=3, Hq=8, Hkv=2, d=128, N=4096, K=16, decode=True,
                                                 seq_lens=[4096, 2222, 65], qcal_rank=8, Hlmk=2, needle_frac=0.05)),
    # three splits of 1024 chunks, K = 32
    ("bf16_d64_3splits", synth.Workload("mir_3s", B=2, Hq=4, Hkv=1, d=64, N=150000, K=32, decode=True,
                                        seq_lens=[150000, 65600], needle_frac=0.01)),
]


@pytest.mark.parametrize("name,w", MIRROR_DECODE, ids=[n for n, _ in MIRROR_DECODE])
def test_decode_mirror(name, w):
    _say("mirror decode", name)
    x = synth.make_inputs(w, SEED)
    a = gpu_decode(w, x)
    b = gpu_decode(w, x, kc=a["kc"], bc=a["bc"], mirror=True)
    _assert_same_step(a, b, name)
    _, summ = _check_against_oracle(w, x, b, "mirror " + name)
    _say(name, summ)


@pytest.mark.parametrize("name,w,twins", TIE_DECODE, ids=[t[0] for t in TIE_DECODE])
def test_decode_mirror_exact_ties(name, w, twins):
    """Twin chunks with bitwise-equal scores at the K boundary: the mirror decode takes the
    lower ids, as hils_attn_decode and the oracle do."""
    _say("mirror decode exact ties", name)
    x = _twin_inputs(w, SEED + 45, twins)
    a = gpu_decode(w, x)
    b = gpu_decode(w, x, kc=a["kc"], bc=a["bc"], mirror=True)
    _assert_same_step(a, b, name)
    ref, summ = _check_against_oracle(w, x, b, "mirror ties " + name)
    nt = _assert_tie_rows(name, ref, b["sel_idx"].reshape(-1, w.K), min_rows=w.B * w.Hq // 2)
    _say(name, "exact-tie rows", nt, summ)


@pytest.mark.parametrize("K", [8, 64])
def test_decode_mirror_all_chunks_identical(K):
    """Every chunk identical: every chunk's bounds reach the threshold, so all of them are
    rescored, in several batches of 1024 (1093 candidate chunks); the selection must be
    chunks 0..K-1, as from hils_attn_decode."""
    w = synth.Workload("mir_same_%d" % K, B=2, Hq=2, Hkv=1, d=64, N=70000, K=K, decode=True,
                       seq_lens=[70000, 30000], planted=False)
    _say("mirror decode, all chunks identical, K", K)
    x = _twin_inputs(w, SEED + 43, list(range(w.C)), kboost=0.0, qboost=0.0)
    a = gpu_decode(w, x)
    b = gpu_decode(w, x, kc=a["kc"], bc=a["bc"], mirror=True)
    _assert_same_step(a, b, "same_%d" % K)
    got = np.sort(b["sel_idx"].reshape(-1, K), axis=1)
    assert np.array_equal(got, np.broadcast_to(np.arange(K), got.shape))


def test_decode_mirror_near_ties_below_mirror_resolution():
    """Chunks whose keys differ by far less than the 8-bit codes resolve: their mirror
    bounds agree, their exact scores do not; the exact ones decide."""
    w = synth.Workload("mir_near", B=2, Hq=4, Hkv=2, d=128, N=8192, K=16, io=synth.F32, decode=True,
                       seq_lens=[8192, 6000], planted=False)
    _say("mirror decode near ties")
    twins = list(range(2, 90, 3))
    x = _twin_inputs(w, SEED + 47, twins)
    u = synth.unit_vector(w.d, SEED + 48)
    k = x["k"].copy()
    for n, t in enumerate(twins):   # distinct offsets of a few fp32 ulps along u, chunk by chunk
        k[:, :, t * w.S:(t + 1) * w.S] += np.float32(1e-5 * ((n * 7) % len(twins))) * u.astype(np.float32)
    x["k"] = np.ascontiguousarray(k, np.float32)
    a = gpu_decode(w, x)
    b = gpu_decode(w, x, kc=a["kc"], bc=a["bc"], mirror=True)
    _assert_same_step(a, b, "near")
    _, summ = _check_against_oracle(w, x, b, "mirror near ties")
    _say("near", summ)


def test_decode_mirror_sequences_below_one_chunk():
    """No complete chunk (N < S): the mirror is empty and the step is the own chunk alone."""
    w = synth.Workload("mir_short", B=2, Hq=2, Hkv=1, d=64, N=48, K=4, decode=True, seq_lens=[48, 1], planted=False)
    x = synth.make_inputs(w, SEED + 9)
    a = gpu_decode(w, x)
    b = gpu_decode(w, x, kc=a["kc"], bc=a["bc"], mirror=True)
    _assert_same_step(a, b, "short")
    _check_against_oracle(w, x, b, "mirror short")


def test_decode_mirror_timed_matches_untimed():
    """hils_attn_decode_mirror_timed: the same result, and a positive time per stage."""
    w = synth.Workload("mir_timed", B=8, Hq=32, Hkv=8, d=128, N=4096, K=16, decode=True,
                       seq_lens=[4096, 3000, 65, 1, 2048, 4095, 100, 700], needle_frac=0.05)
    x = synth.make_inputs(w, SEED + 3)
    a = gpu_decode(w, x, mirror=True)
    dm = dims_of(w)
    q = torch.from_numpy(x["q"].view(np.int16)).cuda().view(torch.bfloat16)
    k = torch.from_numpy(x["k"].view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(x["v"].view(np.int16)).cuda().view(torch.bfloat16)
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    o = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE_MIRROR)
    ms = hils.attn_decode(dm, q, k, v, lens, a["kc"], a["bc"], o, ws, sel_idx=sel, timed=True, kc_mirror=a["kcm"])
    assert set(ms) == set(hils.DECODE_STAGES) and all(t_ > 0 for t_ in ms.values()), ms
    np.testing.assert_array_equal(sel.cpu().numpy(), a["sel_idx"])
    np.testing.assert_array_equal(o.view(torch.int16).cpu().numpy(), a["o_bits"])
