"""GPU parity of the HIP path against the fp64 oracle at sizes the oracle
finishes in seconds (several tiles, ragged tails, degenerate cases).

All calls go through the C ABI (libhils.so) via the Python binding.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hils_testutil import (TOL, check_selection_and_output, dims_of, gpu_compress, gpu_decode, gpu_prefill,
                           oracle_compress, oracle_rows, shape_of, upload)
from long_context_chunk_amd import hils

pytestmark = pytest.mark.gpu

SEED = synth.BASE_SEED


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# small workloads: (name, Workload)
SMALL = [
    ("tiny_f32", synth.WORKLOADS["tiny_f32"]),
    ("bf16_d64_ragged", synth.scaled(synth.WORKLOADS["prefill_8k"], N=2000)),
    ("bf16_d128_qcal_ragged", synth.scaled(synth.WORKLOADS["prefill_256k_qcal"], N=1500, Hq=8, Hkv=2, K=8)),
    ("f32_d128_qcal", synth.Workload("f32_d128_qcal", B=2, Hq=4, Hkv=2, d=128, N=777, K=5, io=synth.F32,
                                     qcal_rank=16)),
    ("bf16_d64_B2_K32", synth.Workload("bf16_d64_B2_K32", B=2, Hq=4, Hkv=1, d=64, N=3000, K=32)),
    # K above 32: 64-entry candidate lists in the selection and decode kernels
    ("bf16_d64_K48", synth.Workload("bf16_d64_K48", B=1, Hq=4, Hkv=2, d=64, N=4000, K=48)),
    ("bf16_d128_qcal_K64", synth.Workload("bf16_d128_qcal_K64", B=1, Hq=4, Hkv=1, d=128, N=6000, K=64, qcal_rank=8)),
    ("f32_d64_K40", synth.Workload("f32_d64_K40", B=2, Hq=2, Hkv=1, d=64, N=3500, K=40, io=synth.F32)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[n for n, _ in SMALL])
def test_compress(name, w):
    _say("compress", name)
    x = synth.make_inputs(w, SEED)
    kc, bc = gpu_compress(w, x)
    kc_o, bc_o = oracle_compress(w, x)
    kc, bc = kc.cpu().numpy(), bc.cpu().numpy()
    np.testing.assert_allclose(kc, kc_o, rtol=0, atol=1e-5 * max(1.0, np.abs(kc_o).max()))
    np.testing.assert_allclose(bc, bc_o, rtol=0, atol=1e-5)


def test_compress_range_leaves_other_chunks():
    w = synth.scaled(synth.WORKLOADS["prefill_8k"], N=1024, Hq=4, Hkv=2)
    x = synth.make_inputs(w, SEED + 1)
    dm = dims_of(w)
    k, lmk = upload(x["k"], w.io), upload(x["lmk"], w.io)
    kc = torch.full((w.B, w.Hq, w.C, w.d), 7.0, device="cuda")
    bc = torch.full((w.B, w.Hq, w.C), 7.0, device="cuda")
    hils.landmark_compress(dm, k, lmk, kc, bc, 3, 9)
    torch.cuda.synchronize()
    kc_o, bc_o = oracle_compress(w, x)
    kc, bc = kc.cpu().numpy(), bc.cpu().numpy()
    assert np.all(kc[:, :, :3] == 7.0) and np.all(kc[:, :, 9:] == 7.0) and np.all(bc[:, :, 9:] == 7.0)
    np.testing.assert_allclose(kc[:, :, 3:9], kc_o[:, :, 3:9], atol=1e-5 * np.abs(kc_o).max())
    np.testing.assert_allclose(bc[:, :, 3:9], bc_o[:, :, 3:9], atol=1e-5)


@pytest.mark.parametrize("name,w", SMALL, ids=[n for n, _ in SMALL])
def test_score_topk_on_oracle_landmarks(name, w):
    """Staged: the GPU scores the oracle's k'/b' (rounded to fp32)."""
    _say("score_topk", name)
    x = synth.make_inputs(w, SEED)
    kc_o, bc_o = oracle_compress(w, x)
    dm = dims_of(w)
    q = upload(x["q"], w.io)
    kc = torch.from_numpy(kc_o.astype(np.float32)).cuda()
    bc = torch.from_numpy(bc_o.astype(np.float32)).cuda()
    sel = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.float32, device="cuda")
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    hils.chunk_score_topk(dm, q, kc, bc, sel, scr, qcal_D=D, qcal_U=U)
    torch.cuda.synchronize()
    sel, scr = sel.cpu().numpy(), scr.cpu().numpy()
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o.astype(np.float32).astype(np.float64), bc_o.astype(np.float32).astype(np.float64),
                      rows)
    mism = 0
    for t, (b, h, i) in enumerate(rows):
        ns = ref["nsel"][t]
        g = sel[b, h, i]
        assert np.all(g[ns:] == -1) and np.all(np.isneginf(scr[b, h, i][ns:]))
        if ref["gap"][t] > 1e-4:
            if not np.array_equal(np.sort(g[:ns]), np.sort(ref["sel_idx"][t][:ns])):
                mism += 1
        # ids ascending
        assert np.all(np.diff(g[:ns]) > 0)
    assert mism == 0, "%d rows with gap > 1e-4 select different chunks" % mism


@pytest.mark.parametrize("name,w", SMALL, ids=[n for n, _ in SMALL])
def test_prefill_end_to_end(name, w):
    _say("prefill", name)
    x = synth.make_inputs(w, SEED)
    g = gpu_prefill(w, x, fused=True)
    kc_o, bc_o = oracle_compress(w, x)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label=name)
    _say(name, summ)


def test_prefill_unfused_matches_fused():
    w = SMALL[1][1]
    x = synth.make_inputs(w, SEED + 2)
    a = gpu_prefill(w, x, fused=True)
    kc = torch.from_numpy(a["kc"]).cuda()
    bc = torch.from_numpy(a["bc"]).cuda()
    b = gpu_prefill(w, x, fused=False, kc=kc, bc=bc)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])
    np.testing.assert_array_equal(a["o"], b["o"])


def test_prefill_deterministic():
    w = SMALL[2][1]
    x = synth.make_inputs(w, SEED + 3)
    a = gpu_prefill(w, x)
    b = gpu_prefill(w, x)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])
    np.testing.assert_array_equal(a["sel_score"], b["sel_score"])
    np.testing.assert_array_equal(a["o"], b["o"])


@pytest.mark.parametrize("N", [1, 17, 64, 65, 128, 129])
def test_prefill_short_sequences(N):
    """Sequences shorter than a few chunks: no or one past chunk, partial own chunk."""
    w = synth.Workload("short", B=1, Hq=2, Hkv=1, d=64, N=N, K=3)
    x = synth.make_inputs(w, SEED + N)
    g = gpu_prefill(w, x)
    kc_o, bc_o = oracle_compress(w, x)
    rows = [(0, h, i) for h in range(2) for i in range(N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                               g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]], g["o"][rr[:, 0], rr[:, 1], rr[:, 2]],
                               label="N=%d" % N)


def _dense_causal_rows(q, k, v, tau):
    qt = torch.from_numpy(q.astype(np.float64))[None, None]
    kt = torch.from_numpy(k.astype(np.float64))[None, None]
    vt = torch.from_numpy(v.astype(np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=tau)[0, 0].numpy()


@pytest.mark.parametrize("io", [synth.F32, synth.BF16])
def test_dense_reduction_chunk_constant_keys(io):
    """Chunk-constant keys and K >= number of chunks: HiLS equals dense causal attention."""
    d, S, C = 64, 64, 20
    N = C * S + 30
    rng = np.random.default_rng(5)
    kappa = rng.standard_normal((C + 1, d)).astype(np.float32)
    k = np.repeat(kappa, S, axis=0)[:N]
    v = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((N, d)).astype(np.float32)
    lmk = rng.standard_normal((C, d)).astype(np.float32)
    if io == synth.BF16:
        to = lambda a: torch.from_numpy(a).to(torch.bfloat16)
        k, v, q, lmk = [to(a).float().numpy() for a in (k, v, q, lmk)]
    w = synth.Workload("dense", B=1, Hq=1, Hkv=1, d=d, N=N, K=32, io=io, planted=False)
    dm = dims_of(w)
    dev = lambda a: torch.from_numpy(a.reshape(1, 1, *a.shape)).cuda().to(torch.float32 if io == synth.F32
                                                                          else torch.bfloat16)
    qt, kt, vt, lt = dev(q), dev(k), dev(v), dev(lmk)
    o = torch.empty_like(qt)
    ws = hils.workspace(dm, hils.OP_PREFILL)
    hils.attn_prefill(dm, qt, kt, vt, o, ws, lmk_q=lt)
    torch.cuda.synchronize()
    ref = _dense_causal_rows(q, k, v, 1 / math.sqrt(d))
    diff = np.abs(o.float().cpu().numpy()[0, 0] - ref)
    mx, mean = TOL[io]
    assert diff.max() <= mx and diff.mean() <= mean, (diff.max(), diff.mean())


DECODE_SMALL = [
    ("bf16_d128", synth.Workload("dec_bf16_d128", B=5, Hq=8, Hkv=2, d=128, N=4096, K=8, decode=True,
                                 seq_lens=[1, 64, 65, 1000, 4096], needle_frac=0.05)),
    ("bf16_d64_qcal", synth.Workload("dec_bf16_d64_qcal", B=3, Hq=4, Hkv=4, d=64, N=3000, K=16, decode=True,
                                     seq_lens=[2999, 3000, 640], qcal_rank=8, planted_seqs=1)),
    ("f32_d64", synth.Workload("dec_f32_d64", B=2, Hq=2, Hkv=1, d=64, N=2048, K=4, io=synth.F32, decode=True,
                               seq_lens=[2048, 1111], planted=False)),
    ("bf16_d128_K64", synth.Workload("dec_bf16_d128_K64", B=3, Hq=4, Hkv=2, d=128, N=70000, K=64, decode=True,
                                     seq_lens=[70000, 5000, 4100], needle_frac=0.02)),
]


@pytest.mark.parametrize("name,w", DECODE_SMALL, ids=[n for n, _ in DECODE_SMALL])
def test_decode(name, w):
    _say("decode", name)
    x = synth.make_inputs(w, SEED)
    g = gpu_decode(w, x)
    kc_o, bc_o = oracle_compress(w, x)
    s = shape_of(w)
    rows_b = [b for b in range(w.B) for h in range(w.Hq)]
    rows_h = [h for b in range(w.B) for h in range(w.Hq)]
    pos = [int(x["seq_lens"][b]) - 1 for b in rows_b]
    qrows = x["q"].reshape(w.B * w.Hq, w.d)
    ref = oracle.attend(s, rows_b, rows_h, pos, qrows, x["k"], x["v"], kc_o, bc_o, D=x.get("D"), U=x.get("U"))
    xx = dict(x)

    class QView:  # check_selection_and_output indexes q as [b, h, i]

        def __getitem__(self, key):
            b, h, i = key
            return x["q"][b, h]
    xx["q"] = QView()
    rows = list(zip(rows_b, rows_h, pos))
    summ = check_selection_and_output(w, xx, kc_o, bc_o, rows, ref, g["sel_idx"].reshape(-1, w.K), None,
                                      g["o"].reshape(-1, w.d), label=name)
    _say(name, summ)


# 256 (sequence, head) pairs or more: on MI355X's 256 CUs the step runs attention and fusion
# in one workgroup per pair (decode_attend_fused) instead of one per chunk plus a combine
DECODE_FUSED = [
    ("bf16_d128_B8_H32", synth.Workload("decf_a", B=8, Hq=32, Hkv=8, d=128, N=4096, K=16, decode=True,
                                        seq_lens=[4096, 1, 64, 65, 1000, 3000, 2049, 4095], needle_frac=0.05)),
    ("bf16_d64_B16_H16_qcal", synth.Workload("decf_b", B=16, Hq=16, Hkv=4, d=64, N=2048, K=8, decode=True,
                                             seq_lens=[2048 - 97 * i for i in range(16)], qcal_rank=8, planted_seqs=3)),
    ("bf16_d128_H64_K64_w1024", synth.Workload("decf_c", B=4, Hq=64, Hkv=8, d=128, N=8192, K=64, decode=True,
                                               seq_lens=[8192, 5000, 1100, 300], needle_frac=0.02, window=1024)),
]


@pytest.mark.parametrize("name,w", DECODE_FUSED, ids=[n for n, _ in DECODE_FUSED])
def test_decode_fused_attention(name, w):
    test_decode(name, w)


# caches of more than 16384 chunks (over 1M tokens): more than 16 scan splits per (b, h)
DECODE_LONG = [
    ("bf16_d64_1.2M", synth.Workload("declong_a", B=1, Hq=2, Hkv=1, d=64, N=1200000, K=16, decode=True,
                                     seq_lens=[1200000], needle_frac=0.002)),
    ("bf16_d128_K48_1.1M", synth.Workload("declong_b", B=1, Hq=2, Hkv=1, d=128, N=1100000, K=48, decode=True,
                                          seq_lens=[1048700], needle_frac=0.002, qcal_rank=8)),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,w", DECODE_LONG, ids=[n for n, _ in DECODE_LONG])
def test_decode_beyond_16384_chunks(name, w):
    test_decode(name, w)


def test_decode_matches_prefill_row():
    """A decode step at cache length L reproduces prefill row L-1 (same kernels' inputs)."""
    L = 1000
    w = synth.Workload("pre", B=1, Hq=4, Hkv=2, d=128, N=L, K=8)
    x = synth.make_inputs(w, SEED + 9)
    pre = gpu_prefill(w, x)
    wd = synth.Workload("dec", B=1, Hq=4, Hkv=2, d=128, N=L, K=8, decode=True, seq_lens=[L])
    xd = {"k": x["k"], "v": x["v"], "lmk": x["lmk"], "q": np.ascontiguousarray(x["q"][:, :, L - 1]),
          "seq_lens": np.asarray([L], np.int32)}
    dec = gpu_decode(wd, xd, kc=torch.from_numpy(pre["kc"]).cuda(), bc=torch.from_numpy(pre["bc"]).cuda())
    for h in range(4):
        assert set(dec["sel_idx"][0, h]) == set(pre["sel_idx"][0, h, L - 1])
    np.testing.assert_allclose(dec["o"][0], pre["o"][0, :, L - 1], rtol=0, atol=1e-2)


# ---------------------------------------------------------------- dense baseline
DENSE = [
    ("bf16_d128_gqa_ragged", synth.Workload("dense_a", B=1, Hq=4, Hkv=2, d=128, N=700, K=4)),
    ("bf16_d64_B2_mqa", synth.Workload("dense_b", B=2, Hq=2, Hkv=1, d=64, N=333, K=4)),
    ("f32_d64", synth.Workload("dense_c", B=1, Hq=2, Hkv=2, d=64, N=200, K=4, io=synth.F32)),
    ("f32_d128_one_row", synth.Workload("dense_d", B=1, Hq=1, Hkv=1, d=128, N=1, K=4, io=synth.F32)),
]


@pytest.mark.parametrize("name,w", DENSE, ids=[n for n, _ in DENSE])
def test_dense_baseline(name, w):
    """hils_dense_attention against the oracle's dense causal attention, every row."""
    _say("dense", name)
    x = synth.make_inputs(w, SEED + 7)
    q, k, v = (upload(x[n], w.io) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    hils.dense_attention(dims_of(w), q, k, v, o)
    torch.cuda.synchronize()
    rows = np.asarray([(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)])
    ref = oracle.dense(shape_of(w), rows[:, 0], rows[:, 1], rows[:, 2], x["q"][rows[:, 0], rows[:, 1], rows[:, 2]],
                       x["k"], x["v"])
    got = o.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = np.abs(got - ref)
    mx, mean = TOL[w.io]
    assert err.max() <= mx and err.mean() <= mean, (err.max(), err.mean())


DENSE_DECODE = [
    ("d128_g4", synth.Workload("dd_a", B=4, Hq=8, Hkv=2, d=128, N=6000, K=8, decode=True,
                               seq_lens=[1, 2047, 2049, 6000])),
    ("d64_g8", synth.Workload("dd_b", B=2, Hq=8, Hkv=1, d=64, N=5000, K=8, decode=True, seq_lens=[4097, 333])),
    ("d128_g1", synth.Workload("dd_c", B=2, Hq=2, Hkv=2, d=128, N=3000, K=8, decode=True, seq_lens=[64, 3000])),
    ("d64_g2", synth.Workload("dd_d", B=3, Hq=4, Hkv=2, d=64, N=4100, K=8, decode=True, seq_lens=[4100, 2048, 65])),
]


@pytest.mark.parametrize("name,w", DENSE_DECODE, ids=[n for n, _ in DENSE_DECODE])
def test_dense_decode_baseline(name, w):
    """hils_dense_decode against the oracle's dense causal attention of each sequence's
    last row (every cached key; splits of 2048 keys, ragged lengths across them)."""
    _say("dense decode", name)
    x = synth.make_inputs(w, SEED + 9)
    dm = dims_of(w)
    q, k, v = (upload(x[n], w.io) for n in ("q", "k", "v"))
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    o = torch.full_like(q, float("nan"))
    hils.dense_decode(dm, q, k, v, lens, o, hils.workspace(dm, hils.OP_DENSE_DECODE))
    torch.cuda.synchronize()
    rows = np.asarray([(b, h, int(x["seq_lens"][b]) - 1) for b in range(w.B) for h in range(w.Hq)])
    ref = oracle.dense(shape_of(w), rows[:, 0], rows[:, 1], rows[:, 2], x["q"][rows[:, 0], rows[:, 1]], x["k"],
                       x["v"])
    got = o.float().cpu().numpy()[rows[:, 0], rows[:, 1]]
    err = np.abs(got - ref)
    mx, mean = TOL[w.io]
    assert np.all(np.isfinite(got)) and err.max() <= mx and err.mean() <= mean, (err.max(), err.mean())


# ------------------------------------------ ablation variants of the chunk summary
# The pages' ablations replace the learned landmark: mean pooling of the chunk's keys
# (a_j = 1/S, what a zero landmark query gives) and one shared query for every chunk.
# Both are inputs to the same kernels.
@pytest.mark.parametrize("variant", ["mean_pooled", "shared_query"])
def test_summary_ablation_variants(variant):
    w = synth.Workload("ablation_" + variant, B=1, Hq=4, Hkv=2, d=64, N=1500, K=8)
    _say("ablation", variant)
    x = synth.make_inputs(w, SEED + 11)
    if variant == "mean_pooled":
        x["lmk"] = np.zeros_like(x["lmk"])
    else:
        x["lmk"] = np.ascontiguousarray(np.broadcast_to(x["lmk"][:, :, :1, :], x["lmk"].shape))
    g = gpu_prefill(w, x, fused=True)
    kc_o, bc_o = oracle_compress(w, x)
    if variant == "mean_pooled":  # closed form: the chunk mean and the entropy of uniform weights
        kf = synth_bf16_to_f64(x["k"][:, :, :w.C * w.S]).reshape(w.B, w.Hkv, w.C, w.S, w.d).mean(axis=3)
        kf = np.repeat(kf, w.Hq // w.Hkv, axis=1)
        np.testing.assert_allclose(g["kc"], kf, rtol=0, atol=1e-5)
        np.testing.assert_allclose(g["bc"], math.log(w.S), rtol=0, atol=1e-5)
    rows = [(0, h, i) for h in range(w.Hq) for i in range(0, w.N, 2)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label=variant)
    _say(variant, summ)


def synth_bf16_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------- chunk-paged KV cache (decode)
def _paginate(w, x, seed):
    """The contiguous caches scattered into shuffled pages of one chunk each (plus spare pages)."""
    C = w.C
    rng = np.random.default_rng(seed)
    npages = w.B * C + 3
    perm = rng.permutation(npages)[: w.B * C].astype(np.int32)
    table = perm.reshape(w.B, C)
    kp = np.zeros((npages, w.Hkv, w.S, w.d), x["k"].dtype)
    vp = np.zeros_like(kp)
    for b in range(w.B):
        for c in range(C):
            kp[table[b, c]] = x["k"][b, :, c * w.S:(c + 1) * w.S]
            vp[table[b, c]] = x["v"][b, :, c * w.S:(c + 1) * w.S]
    return kp, vp, table


@pytest.mark.parametrize("qcal", [0, 8])
def test_paged_decode_matches_contiguous(qcal):
    """Same kernels, different K/V addressing: outputs and selections are identical."""
    w = synth.Workload("paged", B=3, Hq=4, Hkv=2, d=128, N=2048, K=8, decode=True, seq_lens=[2048, 1000, 70],
                       qcal_rank=qcal)
    _say("paged decode, qcal", qcal)
    x = synth.make_inputs(w, SEED + 13)
    ref = gpu_decode(w, x)
    kp, vp, table = _paginate(w, x, 5)
    dm = dims_of(w)
    kpt, vpt = upload(kp, w.io), upload(vp, w.io)
    tab = torch.from_numpy(table).cuda()
    kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
    lmk = upload(x["lmk"], w.io)
    for c in range(w.C):  # incremental: one chunk at a time, as chunks complete during decoding
        hils.landmark_compress_paged(dm, kpt, tab, lmk, kc, bc, c, c + 1)
    torch.cuda.synchronize()
    assert torch.equal(kc, ref["kc"]) and torch.equal(bc, ref["bc"])
    q = upload(x["q"], w.io)
    o = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE)
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    hils.attn_decode_paged(dm, q, kpt, vpt, tab, torch.from_numpy(x["seq_lens"]).cuda(), kc, bc, o, ws, qcal_D=D,
                           qcal_U=U, sel_idx=sel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel_idx"])
    np.testing.assert_array_equal(o.float().cpu().numpy(), ref["o"])


# ---------------------------------------------------------------- local window
WINDOW = [
    ("bf16_d64_w512_ragged", synth.scaled(synth.WORKLOADS["prefill_8k"], N=2000, window=512)),
    ("bf16_d128_qcal_w256", synth.scaled(synth.WORKLOADS["prefill_256k_qcal"], N=1500, Hq=8, Hkv=2, K=8,
                                         window=256)),
    ("f32_d128_qcal_w128", synth.Workload("f32_w128", B=2, Hq=4, Hkv=2, d=128, N=777, K=5, io=synth.F32,
                                          qcal_rank=16, window=128)),
    ("bf16_d64_B2_K32_w2048", synth.Workload("w2048", B=2, Hq=4, Hkv=1, d=64, N=3000, K=32, window=2048)),
    ("bf16_window_covers_all", synth.Workload("wall", B=1, Hq=2, Hkv=1, d=128, N=300, K=3, window=512)),
]


@pytest.mark.parametrize("name,w", WINDOW, ids=[n for n, _ in WINDOW])
def test_prefill_window(name, w):
    """Local window of W/S chunks: every row against the oracle (selection from the chunks
    before the window, one exact-LSE entry for the window)."""
    _say("prefill window", name)
    x = synth.make_inputs(w, SEED + 21)
    g = gpu_prefill(w, x, fused=True)
    kc_o, bc_o = oracle_compress(w, x)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    nw = w.window // w.S
    assert np.array_equal(ref["nsel"], [min(w.K, w.C, max(0, i // w.S - nw + 1)) for _, _, i in rows])
    rr = np.asarray(rows)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label=name)
    _say(name, summ)


def test_window_of_one_chunk_is_no_window():
    """window = S and window = 0 are the same method: bit-identical prefill and decode."""
    w0 = SMALL[2][1]
    w1 = synth.scaled(w0, window=w0.S)
    x = synth.make_inputs(w0, SEED + 22)
    a, b = gpu_prefill(w0, x), gpu_prefill(w1, x)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])
    np.testing.assert_array_equal(a["o"], b["o"])
    d0 = DECODE_SMALL[0][1]
    xd = synth.make_inputs(d0, SEED + 23)
    p, r = gpu_decode(d0, xd), gpu_decode(synth.scaled(d0, window=d0.S), xd)
    np.testing.assert_array_equal(p["sel_idx"], r["sel_idx"])
    np.testing.assert_array_equal(p["o"], r["o"])


DECODE_WINDOW = [
    ("bf16_d128_w512", synth.Workload("dw512", B=5, Hq=8, Hkv=2, d=128, N=4096, K=8, decode=True,
                                      seq_lens=[1, 64, 300, 1000, 4096], needle_frac=0.05, window=512)),
    ("f32_d64_K32_w2048", synth.Workload("dw2048", B=3, Hq=2, Hkv=1, d=64, N=4096, K=32, io=synth.F32, decode=True,
                                         seq_lens=[4096, 2100, 2047], planted=False, window=2048)),
    ("bf16_d64_qcal_w192", synth.Workload("dw192", B=2, Hq=4, Hkv=4, d=64, N=3000, K=16, decode=True,
                                          seq_lens=[2999, 640], qcal_rank=8, planted_seqs=1, window=192)),
    # K + W/S = 72 slots: the combine's second weight register
    ("f32_d64_K56_w1024", synth.Workload("dw1024", B=2, Hq=2, Hkv=1, d=64, N=8192, K=56, io=synth.F32, decode=True,
                                         seq_lens=[8192, 5000], planted=False, window=1024)),
]


@pytest.mark.parametrize("name,w", DECODE_WINDOW, ids=[n for n, _ in DECODE_WINDOW])
def test_decode_window(name, w):
    """Decode with a local window (K + W/S slots, up to 64) against the oracle."""
    test_decode(name, w)


def test_decode_window_matches_prefill_row():
    L = 1000
    w = synth.Workload("prew", B=1, Hq=4, Hkv=2, d=128, N=L, K=8, window=384)
    x = synth.make_inputs(w, SEED + 24)
    pre = gpu_prefill(w, x)
    wd = synth.Workload("decw", B=1, Hq=4, Hkv=2, d=128, N=L, K=8, decode=True, seq_lens=[L], window=384)
    xd = {"k": x["k"], "v": x["v"], "lmk": x["lmk"], "q": np.ascontiguousarray(x["q"][:, :, L - 1]),
          "seq_lens": np.asarray([L], np.int32)}
    dec = gpu_decode(wd, xd, kc=torch.from_numpy(pre["kc"]).cuda(), bc=torch.from_numpy(pre["bc"]).cuda())
    for h in range(4):
        assert set(dec["sel_idx"][0, h]) == set(pre["sel_idx"][0, h, L - 1])
    np.testing.assert_allclose(dec["o"][0], pre["o"][0, :, L - 1], rtol=0, atol=1e-2)


def test_paged_decode_window_matches_contiguous():
    w = synth.Workload("pagedw", B=3, Hq=4, Hkv=2, d=128, N=2048, K=8, decode=True, seq_lens=[2048, 1000, 70],
                       window=512)
    x = synth.make_inputs(w, SEED + 25)
    ref = gpu_decode(w, x)
    kp, vp, table = _paginate(w, x, 6)
    dm = dims_of(w)
    kpt, vpt = upload(kp, w.io), upload(vp, w.io)
    tab = torch.from_numpy(table).cuda()
    q = upload(x["q"], w.io)
    o = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE)
    hils.attn_decode_paged(dm, q, kpt, vpt, tab, torch.from_numpy(x["seq_lens"]).cuda(), ref["kc"], ref["bc"], o, ws,
                           sel_idx=sel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel_idx"])
    np.testing.assert_array_equal(o.float().cpu().numpy(), ref["o"])


# --------------------------------------- chunk-paged KV cache against the oracle
PAGED = [
    ("bf16_d128", 0, 0),
    ("bf16_d128_qcal", 8, 0),
    ("bf16_d128_w512", 0, 512),
    ("bf16_d128_qcal_w256", 8, 256),
]


@pytest.mark.parametrize("name,qcal,window", PAGED, ids=[p[0] for p in PAGED])
def test_paged_decode_against_oracle(name, qcal, window):
    """The paged path on its own: landmark compression one chunk at a time from shuffled
    pages against the oracle's compression, then the paged decode step against the oracle's
    forward pass on the contiguous cache (selection and output, the usual bar), and the
    paged step over the landmark mirror bit-equal to it."""
    w = synth.Workload("paged_" + name, B=3, Hq=4, Hkv=2, d=128, N=2048, K=8, decode=True,
                       seq_lens=[2048, 1000, 70], qcal_rank=qcal, window=window, needle_frac=0.05)
    _paged_decode_case(w, name)


def test_paged_decode_fused_attention_against_oracle():
    """The same at 256 (sequence, head) pairs, where attention and fusion run in one kernel."""
    w = synth.Workload("paged_fused", B=8, Hq=32, Hkv=8, d=128, N=2048, K=16, decode=True,
                       seq_lens=[2048, 1000, 70, 1, 65, 640, 1999, 2047], qcal_rank=8, window=256, needle_frac=0.05)
    _paged_decode_case(w, "fused")


def _paged_decode_case(w, name):
    _say("paged decode vs oracle", name)
    x = synth.make_inputs(w, SEED + 31)
    kp, vp, table = _paginate(w, x, 17)
    dm = dims_of(w)
    kpt, vpt = upload(kp, w.io), upload(vp, w.io)
    tab = torch.from_numpy(table).cuda()
    kc = torch.full((w.B, w.Hlmk, w.C, w.d), float("nan"), dtype=torch.float32, device="cuda")
    bc = torch.full((w.B, w.Hlmk, w.C), float("nan"), dtype=torch.float32, device="cuda")
    lmk = upload(x["lmk"], w.io)
    for c in range(w.C):  # incremental, as chunks complete during decoding
        hils.landmark_compress_paged(dm, kpt, tab, lmk, kc, bc, c, c + 1)
    torch.cuda.synchronize()
    kc_o, bc_o = oracle_compress(w, x)
    np.testing.assert_allclose(kc.cpu().numpy(), kc_o, rtol=0, atol=1e-5 * max(1.0, np.abs(kc_o).max()))
    np.testing.assert_allclose(bc.cpu().numpy(), bc_o, rtol=0, atol=1e-5)
    q = upload(x["q"], w.io)
    o = torch.full_like(q, float("nan"))
    sel = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE)
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    hils.attn_decode_paged(dm, q, kpt, vpt, tab, lens, kc, bc, o, ws, qcal_D=D, qcal_U=U, sel_idx=sel)
    # the same step over the landmark mirror (built chunk by chunk too)
    kcm = torch.zeros(hils.mirror_shape(dm), dtype=torch.uint8, device="cuda")
    for c in range(w.C):
        hils.landmark_mirror(dm, kc, bc, kcm, c, c + 1)
    om = torch.full_like(q, float("nan"))
    selm = torch.empty_like(sel)
    wsm = hils.workspace(dm, hils.OP_DECODE_MIRROR)
    hils.attn_decode_paged(dm, q, kpt, vpt, tab, lens, kc, bc, om, wsm, qcal_D=D, qcal_U=U, sel_idx=selm,
                           kc_mirror=kcm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(selm.cpu().numpy(), sel.cpu().numpy())
    np.testing.assert_array_equal(om.view(torch.int16).cpu().numpy(), o.view(torch.int16).cpu().numpy())
    rows_b = [b for b in range(w.B) for h in range(w.Hq)]
    rows_h = [h for b in range(w.B) for h in range(w.Hq)]
    pos = [int(x["seq_lens"][b]) - 1 for b in rows_b]
    ref = oracle.attend(shape_of(w), rows_b, rows_h, pos, x["q"].reshape(-1, w.d), x["k"], x["v"], kc_o, bc_o,
                        D=x.get("D"), U=x.get("U"))
    xx = dict(x)

    class QView:
        def __getitem__(self, key):
            b, h, i = key
            return x["q"][b, h]
    xx["q"] = QView()
    summ = check_selection_and_output(w, xx, kc_o, bc_o, list(zip(rows_b, rows_h, pos)), ref,
                                      sel.cpu().numpy().reshape(-1, w.K), None, o.float().cpu().numpy().reshape(-1, w.d),
                                      label="paged " + name)
    _say(name, summ)


# ------------------------------------------------------------------ exact ties
# Bitwise-identical chunks (the same keys and the same landmark query) get bitwise-identical
# k', b' and scores on both sides, so wherever the K-th and (K+1)-th best scores of a row
# come from two such twins the tie rule alone decides the selection: the lower chunk id wins.
# The twins carry a strong shared direction that the queries share too, so they outscore
# every other chunk and the K boundary falls inside the twin group.
def _to_bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _io_to_f32(a, io):
    return synth.bf16_to_f32(a) if io == synth.BF16 else np.asarray(a, np.float32)


def _io_from_f32(a, io):
    return _to_bf16_bits(a) if io == synth.BF16 else np.ascontiguousarray(a, np.float32)


def _twin_inputs(w, seed, twins, kboost=6.0, qboost=4.0):
    """Inputs of w where every chunk in `twins` is a copy of chunk twins[0] (keys of every KV
    head and landmark queries of every landmark head), boosted along a unit vector u that
    every query also carries (decode: every sequence's query)."""
    x = synth.make_inputs(w, seed)
    u = synth.unit_vector(w.d, seed + 1)
    S, t0 = w.S, twins[0]
    k = _io_to_f32(x["k"], w.io).copy()
    base = k[:, :, t0 * S:(t0 + 1) * S] + kboost * u
    lmk = x["lmk"].copy()
    for t in twins:
        k[:, :, t * S:(t + 1) * S] = base
        lmk[:, :, t] = x["lmk"][:, :, t0]
    x["k"] = _io_from_f32(k, w.io)
    x["lmk"] = lmk
    x["q"] = _io_from_f32(_io_to_f32(x["q"], w.io) + qboost * u, w.io)
    return x


def _assert_tie_rows(label, ref, gpu_sel, min_rows):
    """Rows whose oracle K-th and (K+1)-th scores are exactly equal: the GPU set must be the
    oracle's, which takes the lower chunk ids (no tolerance, no near-tie allowance)."""
    gap = np.asarray(ref["gap"])
    ties = np.flatnonzero(gap == 0.0)
    assert ties.size >= min_rows, "%s: only %d exact-tie rows (setup)" % (label, ties.size)
    for t in ties:
        ns = ref["nsel"][t]
        o_sel = np.sort(ref["sel_idx"][t][:ns])
        g = gpu_sel[t]
        assert np.array_equal(np.sort(g[g >= 0]), o_sel), "%s row %d: tie broken wrongly\n gpu %s\n ora %s" % (
            label, t, np.sort(g[g >= 0]), o_sel)
    return int(ties.size)


TIE_PREFILL = [
    ("bf16_d64", synth.Workload("tie_a", B=1, Hq=4, Hkv=2, d=64, N=4096, K=8, planted=False),
     [1, 2, 3, 5, 8, 9, 12, 15, 16, 20, 21, 37]),
    ("bf16_d128_qcal", synth.Workload("tie_b", B=1, Hq=4, Hkv=1, d=128, N=3000, K=5, qcal_rank=8, planted=False),
     [1, 2, 7, 11, 20, 21, 33, 40, 45]),
    ("f32_d64_K32", synth.Workload("tie_c", B=2, Hq=2, Hkv=2, d=64, N=4500, K=32, io=synth.F32, planted=False),
     list(range(1, 21)) + [22, 25, 27, 30, 31, 33, 36, 38, 40, 41, 43, 44, 46, 47]),
]


@pytest.mark.parametrize("name,w,twins", TIE_PREFILL, ids=[t[0] for t in TIE_PREFILL])
def test_prefill_exact_ties_to_lower_chunk(name, w, twins):
    _say("prefill exact ties", name)
    x = _twin_inputs(w, SEED + 41, twins)
    g = gpu_prefill(w, x, fused=True)
    kc_o, bc_o = oracle_compress(w, x)
    for t in twins[1:]:  # the twins are exact copies on both sides
        assert np.array_equal(kc_o[:, :, t], kc_o[:, :, twins[0]]) and np.array_equal(bc_o[:, :, t], bc_o[:, :, twins[0]])
        assert np.array_equal(g["kc"][:, :, t], g["kc"][:, :, twins[0]])
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    gsel = g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]]
    nt = _assert_tie_rows(name, ref, gsel, min_rows=len(rows) // 4)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, gsel, g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label=name)
    _say(name, "exact-tie rows", nt, summ)


@pytest.mark.parametrize("K", [8, 32, 64])
def test_prefill_all_chunks_identical(K):
    """Every chunk identical: every score of a row ties, so every row with more than K
    candidates must select chunks 0..K-1.  Every candidate passes the selection kernel's
    threshold, so its per-row candidate lists fill and are compacted again and again."""
    w = synth.Workload("same_%d" % K, B=1, Hq=2, Hkv=1, d=64, N=16384, K=K, planted=False)
    _say("all chunks identical, K", K)
    x = _twin_inputs(w, SEED + 43, list(range(w.C)), kboost=0.0, qboost=0.0)
    g = gpu_prefill(w, x, fused=True)
    P = np.minimum(np.arange(w.N) // w.S, w.C)
    sel = g["sel_idx"][0]
    expect = np.where(np.arange(K)[None, :] < np.minimum(P, K)[:, None], np.arange(K)[None, :], -1)
    for h in range(w.Hq):
        got = np.sort(np.where(sel[h] >= 0, sel[h], 1 << 30), axis=1)
        got = np.where(got == 1 << 30, -1, got)
        assert np.array_equal(got, expect), "head %d: rows %s" % (h, np.flatnonzero(np.any(got != expect, axis=1))[:8])
    kc_o, bc_o = oracle_compress(w, x)
    rows = [(0, h, i) for h in range(w.Hq) for i in range(0, w.N, 7)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    gsel = g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]]
    _assert_tie_rows("same_%d" % K, ref, gsel, min_rows=len(rows) // 2)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, gsel, g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label="same_%d" % K)
    _say("same", K, summ)


TIE_DECODE = [
    ("bf16_d128", synth.Workload("tie_dec_a", B=4, Hq=8, Hkv=2, d=128, N=4096, K=8, decode=True,
                                 seq_lens=[4096, 3001, 1500, 700], planted=False),
     [1, 2, 4, 5, 7, 8, 9, 10, 12, 15, 18, 44]),
    ("bf16_d64_qcal_K32", synth.Workload("tie_dec_b", B=2, Hq=4, Hkv=4, d=64, N=8192, K=32, decode=True,
                                         seq_lens=[8192, 5000], qcal_rank=8, planted=False),
     list(range(1, 100, 2))),
]


@pytest.mark.parametrize("name,w,twins", TIE_DECODE, ids=[t[0] for t in TIE_DECODE])
def test_decode_exact_ties_to_lower_chunk(name, w, twins):
    _say("decode exact ties", name)
    x = _twin_inputs(w, SEED + 45, twins)
    g = gpu_decode(w, x)
    kc_o, bc_o = oracle_compress(w, x)
    rows_b = [b for b in range(w.B) for h in range(w.Hq)]
    rows_h = [h for b in range(w.B) for h in range(w.Hq)]
    pos = [int(x["seq_lens"][b]) - 1 for b in rows_b]
    ref = oracle.attend(shape_of(w), rows_b, rows_h, pos, x["q"].reshape(-1, w.d), x["k"], x["v"], kc_o, bc_o,
                        D=x.get("D"), U=x.get("U"))
    gsel = g["sel_idx"].reshape(-1, w.K)
    nt = _assert_tie_rows(name, ref, gsel, min_rows=len(rows_b) // 2)
    xx = dict(x)

    class QView:
        def __getitem__(self, key):
            b, h, i = key
            return x["q"][b, h]
    xx["q"] = QView()
    summ = check_selection_and_output(w, xx, kc_o, bc_o, list(zip(rows_b, rows_h, pos)), ref, gsel, None,
                                      g["o"].reshape(-1, w.d), label=name)
    _say(name, "exact-tie rows", nt, summ)


# ------------------------------------------- a block of queries at a position offset
# hils_chunk_score_topk scores any block of Nq queries of a sequence whose context kc/bc
# holds floor(N/S) complete chunks: query i of batch b sits at q_pos0[b] + i (chunked
# prefill, several new tokens of a decode stream).
from hils_testutil import check_selection  # noqa: E402

OFFSET = [
    ("bf16_d64", synth.Workload("off_a", B=2, Hq=4, Hkv=2, d=64, N=4096, K=8), 700, [1000, 3333]),
    ("bf16_d128_qcal", synth.Workload("off_b", B=2, Hq=4, Hkv=1, d=128, N=5000, K=16, qcal_rank=8), 333, [64, 4600]),
    ("f32_d64_w256", synth.Workload("off_c", B=1, Hq=2, Hkv=1, d=64, N=3000, K=5, io=synth.F32, window=256), 257,
     [2100]),
    ("bf16_d64_shared_lmk", synth.Workload("off_d", B=2, Hq=8, Hkv=2, d=64, N=4096, K=8, Hlmk=2), 500, [0, 3500]),
    ("bf16_d64_past_end", synth.Workload("off_e", B=1, Hq=2, Hkv=2, d=64, N=2048, K=8), 130, [2000]),
]


@pytest.mark.parametrize("name,w,Nq,p0", OFFSET, ids=[o[0] for o in OFFSET])
def test_score_topk_query_block_at_offset(name, w, Nq, p0):
    _say("score_topk block at offset", name)
    x = synth.make_inputs(w, SEED + 51)
    kc_o, bc_o = oracle_compress(w, x)
    pos0 = np.asarray(p0, np.int32)
    # the block's queries: rows q_pos0[b] .. of the sequence where they exist, fresh draws past its end
    qb = synth.normal((w.B, w.Hq, Nq, w.d), SEED + 52, 901, w.io)
    for b in range(w.B):
        n_in = max(0, min(Nq, w.N - int(pos0[b])))
        qb[b, :, :n_in] = x["q"][b, :, pos0[b]:pos0[b] + n_in]
    dm = dims_of(w)
    sel = torch.full((w.B, w.Hq, Nq, w.K), -9, dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, Nq, w.K), dtype=torch.float32, device="cuda")
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    hils.chunk_score_topk(dm, upload(qb, w.io), torch.from_numpy(kc_o.astype(np.float32)).cuda(),
                          torch.from_numpy(bc_o.astype(np.float32)).cuda(), sel, scr, qcal_D=D, qcal_U=U,
                          q_pos0=torch.from_numpy(pos0).cuda())
    torch.cuda.synchronize()
    kc32 = kc_o.astype(np.float32).astype(np.float64)
    bc32 = bc_o.astype(np.float32).astype(np.float64)
    rows = [(b, h, int(pos0[b]) + i) for b in range(w.B) for h in range(w.Hq) for i in range(Nq)]
    qrows = np.stack([qb[b, h, i] for b in range(w.B) for h in range(w.Hq) for i in range(Nq)])
    ref = oracle.attend(shape_of(w), [r[0] for r in rows], [r[1] for r in rows], [r[2] for r in rows], qrows,
                        x["k"], x["v"], kc32, bc32, D=x.get("D"), U=x.get("U"))
    xx = dict(x)

    class QView:
        def __getitem__(self, key):
            b, h, i = key
            return qb[b, h, i - int(pos0[b])]
    xx["q"] = QView()
    summ = check_selection(w, xx, kc32, bc32, rows, ref, sel.cpu().numpy().reshape(-1, w.K),
                           scr.cpu().numpy().reshape(-1, w.K), label=name)
    _say(name, summ)


def test_score_topk_whole_sequence_block_matches_prefill():
    """Nq = N with no offsets is the prefill's own scoring: identical selection."""
    w = SMALL[2][1]
    x = synth.make_inputs(w, SEED + 53)
    g = gpu_prefill(w, x, fused=True)
    dm = dims_of(w)
    sel = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.float32, device="cuda")
    hils.chunk_score_topk(dm, upload(x["q"], w.io), torch.from_numpy(g["kc"]).cuda(), torch.from_numpy(g["bc"]).cuda(),
                          sel, scr, qcal_D=upload(x["D"], w.io), qcal_U=upload(x["U"], w.io),
                          q_pos0=torch.zeros(w.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), g["sel_idx"])
    np.testing.assert_array_equal(scr.cpu().numpy(), g["sel_score"])


# ------------------------------------ one landmark head per KV group (Hlmk = Hkv)
SHARED_LMK = [
    ("prefill_bf16_d128_qcal", synth.Workload("shl_a", B=1, Hq=8, Hkv=2, d=128, N=2500, K=8, qcal_rank=8, Hlmk=2)),
    ("prefill_f32_d64_w192", synth.Workload("shl_b", B=2, Hq=4, Hkv=1, d=64, N=1300, K=4, io=synth.F32, Hlmk=1,
                                            window=192)),
]


@pytest.mark.parametrize("name,w", SHARED_LMK, ids=[s_[0] for s_ in SHARED_LMK])
def test_prefill_landmark_head_per_kv_group(name, w):
    _say("shared landmark heads", name)
    x = synth.make_inputs(w, SEED + 55)
    g = gpu_prefill(w, x, fused=True)
    kc_o, bc_o = oracle_compress(w, x)
    assert g["kc"].shape == kc_o.shape == (w.B, w.Hkv, w.C, w.d)
    np.testing.assert_allclose(g["kc"], kc_o, rtol=0, atol=1e-5 * max(1.0, np.abs(kc_o).max()))
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    summ = check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                      g["o"][rr[:, 0], rr[:, 1], rr[:, 2]], label=name)
    _say(name, summ)


def test_decode_landmark_head_per_kv_group():
    w = synth.Workload("shl_dec", B=3, Hq=8, Hkv=2, d=128, N=4096, K=16, decode=True, seq_lens=[4096, 2222, 65],
                       qcal_rank=8, Hlmk=2, needle_frac=0.05)
    test_decode("shared_lmk", w)


def test_prefill_values_near_the_fp16_limit():
    """bf16 I/O carries each (query, chunk) output as fp16 between kernels: values up to
    about 5.4e4 (below fp16's 65504) must come through with the usual bar scaled by the
    value range."""
    w = synth.Workload("big_v", B=1, Hq=4, Hkv=2, d=128, N=1500, K=8, qcal_rank=8)
    x = synth.make_inputs(w, SEED + 71)
    scale = 12000.0
    vf = synth.bf16_to_f32(x["v"]) * scale
    x["v"] = _to_bf16_bits(vf)
    assert np.abs(synth.bf16_to_f32(x["v"])).max() < 65504
    g = gpu_prefill(w, x, fused=True)
    assert np.isfinite(g["o"]).all()
    kc_o, bc_o = oracle_compress(w, x)
    rows = [(0, h, i) for h in range(w.Hq) for i in range(w.N)]
    ref = oracle_rows(w, x, kc_o, bc_o, rows)
    rr = np.asarray(rows)
    exact = ref["gap"] > 1e-4
    got = g["o"][rr[:, 0], rr[:, 1], rr[:, 2]][exact]
    err = np.abs(got - ref["o"][exact])
    assert err.max() <= 1e-2 * scale and err.mean() <= 1e-3 * scale, (err.max() / scale, err.mean() / scale)
