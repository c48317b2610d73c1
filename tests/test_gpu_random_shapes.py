"""Parity on seeded random shapes: prefill, decode (plain and over the landmark mirror), the
dense decode baseline and the backward pass against the oracle, over head layouts (GQA, MQA, landmark heads
shared per KV group), d = 64 / 128, K from 1 to 64 (across the 16- and 32-entry list
boundaries), Q-Cal ranks, local windows, bf16 and fp32, ragged lengths and decode caches
of up to four scan splits.  Each case is one pytest item; the shapes come from a fixed
seed, so a failure names a reproducible case."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hils_testutil import (check_selection_and_output, dims_of, gpu_decode, gpu_prefill, oracle_compress, oracle_rows,
                           shape_of, upload, TOL)
from long_context_chunk_amd import hils

pytestmark = pytest.mark.gpu


def _cases(seed=2026, n=32):
    rng = np.random.default_rng(seed)
    out = []
    for ci in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        Hlmk = Hq if rng.random() < 0.7 else Hkv
        io = synth.BF16 if rng.random() < 0.75 else synth.F32
        K = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 48, 64]))
        r = int(rng.choice([0, 0, 8, 32]))
        W = int(rng.choice([0, 0, 0, 128, 512]))
        dec = bool(rng.random() < 0.5)
        B = int(rng.integers(1, 4))
        if not dec:
            N = int(rng.integers(1, 3000))
            w = synth.Workload("rnd%d" % ci, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, K=K, io=io, qcal_rank=r, Hlmk=Hlmk, window=W)
        else:
            N = int(rng.integers(64, 6000)) if rng.random() < 0.5 else int(rng.integers(60000, 250000))
            lens = [int(v) for v in rng.integers(1, N + 1, size=B)]
            w = synth.Workload("rnd%d" % ci, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, K=K, io=io, qcal_rank=r, Hlmk=Hlmk,
                               window=W, decode=True, seq_lens=lens)
        label = "%d_%s_d%d_h%d-%d-%d_K%d_r%d_W%d_N%d_B%d_%s" % (ci, "dec" if dec else "pre", d, Hq, Hkv, Hlmk, K, r, W,
                                                                N, B, "bf16" if io == synth.BF16 else "f32")
        out.append((label, w, 5000 + ci))
    return out


CASES = _cases()


@pytest.mark.parametrize("label,w,seed", CASES, ids=[c[0] for c in CASES])
def test_random_shape(label, w, seed):
    print("random shape", label, flush=True)
    sys.stdout.flush()
    x = synth.make_inputs(w, seed)
    kc_o, bc_o = oracle_compress(w, x)
    if not w.decode:
        g = gpu_prefill(w, x)
        rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
        ref = oracle_rows(w, x, kc_o, bc_o, rows)
        rr = np.asarray(rows)
        check_selection_and_output(w, x, kc_o, bc_o, rows, ref, g["sel_idx"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                   g["sel_score"][rr[:, 0], rr[:, 1], rr[:, 2]], g["o"][rr[:, 0], rr[:, 1], rr[:, 2]],
                                   label=label)
        return
    g = gpu_decode(w, x)
    gm = gpu_decode(w, x, mirror=True)
    assert np.array_equal(g["sel_idx"], gm["sel_idx"]) and np.array_equal(g["o_bits"], gm["o_bits"]), \
        "%s: the mirror step differs from the plain step" % label
    s = shape_of(w)
    rows_b = [b for b in range(w.B) for h in range(w.Hq)]
    rows_h = [h for b in range(w.B) for h in range(w.Hq)]
    pos = [int(x["seq_lens"][b]) - 1 for b in rows_b]
    ref = oracle.attend(s, rows_b, rows_h, pos, x["q"].reshape(w.B * w.Hq, w.d), x["k"], x["v"], kc_o, bc_o,
                        D=x.get("D"), U=x.get("U"))
    xx = dict(x)

    class QView:  # check_selection_and_output indexes q as [b, h, i]

        def __getitem__(self, key):
            return x["q"][key[0], key[1]]
    xx["q"] = QView()
    check_selection_and_output(w, xx, kc_o, bc_o, list(zip(rows_b, rows_h, pos)), ref, g["sel_idx"].reshape(-1, w.K),
                               None, g["o"].reshape(-1, w.d), label=label)
    if w.io == synth.BF16:   # the dense decode baseline on the same cache
        dm = dims_of(w)
        q, k, v = (upload(x[n], w.io) for n in ("q", "k", "v"))
        o = torch.full_like(q, float("nan"))
        hils.dense_decode(dm, q, k, v, torch.from_numpy(x["seq_lens"]).cuda(), o,
                          hils.workspace(dm, hils.OP_DENSE_DECODE))
        torch.cuda.synchronize()
        rr = np.asarray(list(zip(rows_b, rows_h, pos)))
        dref = oracle.dense(s, rr[:, 0], rr[:, 1], rr[:, 2], x["q"][rr[:, 0], rr[:, 1]], x["k"], x["v"])
        err = np.abs(o.float().cpu().numpy()[rr[:, 0], rr[:, 1]] - dref)
        mx, mean = TOL[w.io]
        assert err.max() <= mx and err.mean() <= mean, (label, "dense decode", err.max(), err.mean())


def _backward_cases(seed=2027, n=12):
    rng = np.random.default_rng(seed)
    out = []
    for ci in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        Hlmk = Hq if rng.random() < 0.6 else Hkv
        K = int(rng.choice([1, 2, 5, 8, 16, 17, 32, 33, 48]))
        r = int(rng.choice([0, 8, 32]))
        W = int(rng.choice([0, 0, 128, 512]))
        B = int(rng.integers(1, 3))
        N = int(rng.integers(1, 1600))
        w = synth.Workload("rbw%d" % ci, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, K=K, qcal_rank=r, Hlmk=Hlmk, window=W)
        label = "%d_d%d_h%d-%d-%d_K%d_r%d_W%d_N%d_B%d" % (ci, d, Hq, Hkv, Hlmk, K, r, W, N, B)
        out.append((label, w, 7000 + ci))
    return out


BACKWARD_CASES = _backward_cases()


@pytest.mark.parametrize("label,w,seed", BACKWARD_CASES, ids=[c[0] for c in BACKWARD_CASES])
def test_random_shape_backward(label, w, seed):
    from test_gpu_backward import T_DO, _compare, gpu_backward, oracle_backward
    print("random backward shape", label, flush=True)
    sys.stdout.flush()
    x = synth.make_inputs(w, seed)
    g = gpu_prefill(w, x)
    dO = synth.normal((w.B, w.Hq, w.N, w.d), seed, T_DO, synth.BF16)
    got = gpu_backward(w, x, g, dO)
    ref = oracle_backward(w, x, g["sel_idx"], dO)
    for n in ["dq", "dk", "dv"] + (["dlmk"] if w.C else []) + (["dD", "dU"] if w.qcal_rank else []):
        if np.abs(ref[n]).max() > 0:   # a gradient that is zero everywhere (no complete chunk) has no scale
            _compare(n, got[n], ref[n], label)
        else:
            assert np.abs(got[n]).max() == 0, (label, n)
