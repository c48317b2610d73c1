"""GPU parity of the backward pass (hils_attn_prefill_backward) against the fp64
oracle's backward (itself pinned by finite differences, test_oracle_backward.py).

The GPU forward's selection is held fixed on both sides.  Inputs and the output
gradient are seeded bf16; the oracle works in fp64 on the same bits.  Bar (bf16 I/O,
fp32 accumulation, bf16 MFMA operands for P, dS, q, dO, K, V; gradients rounded to
bf16 once): per gradient tensor, max |g - g_ref| <= 2e-2 * max |g_ref| and mean
|g - g_ref| <= 2e-3 * max |g_ref|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hils_testutil import dims_of, gpu_prefill, shape_of, upload
from long_context_chunk_amd import hils

pytestmark = pytest.mark.gpu

SEED = synth.BASE_SEED + 40
T_DO = 977  # generator stream of the output gradient
MAX_REL, MEAN_REL = 2e-2, 2e-3

CASES = [
    ("d64_gqa_ragged", synth.Workload("bw_a", B=1, Hq=4, Hkv=2, d=64, N=500, K=4)),
    ("d128_qcal_mqa", synth.Workload("bw_b", B=1, Hq=4, Hkv=1, d=128, N=700, K=8, qcal_rank=16)),
    ("d64_B2_qcal_window", synth.Workload("bw_c", B=2, Hq=2, Hkv=2, d=64, N=333, K=3, qcal_rank=8, window=192)),
    ("d128_window512_K16", synth.Workload("bw_d", B=1, Hq=2, Hkv=1, d=128, N=1100, K=16, window=512)),
    ("one_chunk", synth.Workload("bw_e", B=1, Hq=2, Hkv=1, d=64, N=100, K=2)),
    ("no_complete_chunk", synth.Workload("bw_f", B=1, Hq=2, Hkv=2, d=128, N=40, K=2)),
    ("d128_qcal_K48", synth.Workload("bw_g", B=1, Hq=2, Hkv=1, d=128, N=3500, K=48, qcal_rank=8)),
    ("d64_qcal_shared_lmk", synth.Workload("bw_h", B=2, Hq=4, Hkv=2, d=64, N=900, K=6, qcal_rank=8, Hlmk=2)),
]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_backward(w, x, g, dO):
    dm = dims_of(w)
    q, k, v = upload(x["q"], w.io), upload(x["k"], w.io), upload(x["v"], w.io)
    o = torch.from_numpy(g["o"]).cuda().to(torch.bfloat16)  # the forward output (exactly bf16)
    dOt = upload(dO, w.io)
    C = w.C
    lmk = upload(x["lmk"], w.io) if C else None
    kc = torch.from_numpy(g["kc"]).cuda() if C else None
    sel = torch.from_numpy(g["sel_idx"]).cuda()
    scr = torch.from_numpy(g["sel_score"]).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dlmk = torch.empty_like(lmk) if C else None
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    dD = torch.empty_like(D) if w.qcal_rank else None
    dU = torch.empty_like(U) if w.qcal_rank else None
    ws = hils.workspace(dm, hils.OP_BACKWARD)
    hils.attn_prefill_backward(dm, q, k, v, lmk, kc, sel, scr, o, dOt, dq, dk, dv, dlmk, ws, qcal_D=D, qcal_U=U, dD=dD,
                               dU=dU)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float().cpu().numpy()
    return {"dq": f(dq), "dk": f(dk), "dv": f(dv), "dlmk": f(dlmk), "dD": f(dD), "dU": f(dU)}


def oracle_backward(w, x, sel, dO):
    s = shape_of(w)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.N)]
    rr = np.asarray(rows)
    C = w.C
    lmk = x["lmk"] if C else np.zeros((w.B, w.Hlmk, 0, w.d), np.uint16)
    kc, bc = oracle.compress(s, x["k"], lmk)
    qrows = x["q"][rr[:, 0], rr[:, 1], rr[:, 2]]
    g = oracle.attend_backward(s, rr[:, 0], rr[:, 1], rr[:, 2], qrows, x["k"], x["v"], kc, bc, lmk,
                               sel[rr[:, 0], rr[:, 1], rr[:, 2]], synth.bf16_to_f32(dO)[rr[:, 0], rr[:, 1], rr[:, 2]],
                               D=x.get("D"), U=x.get("U"))
    dq = np.zeros((w.B, w.Hq, w.N, w.d))
    dq[rr[:, 0], rr[:, 1], rr[:, 2]] = g["dq"]
    g["dq"] = dq
    return g


def _compare(name, got, ref, label):
    scale = np.abs(ref).max()
    assert scale > 0, (label, name)
    err = np.abs(got - ref)
    rel_max, rel_mean = err.max() / scale, err.mean() / scale
    _say("  %-5s max|ref| %.3g  max err %.3g (%.2e rel)  mean err %.3g (%.2e rel)" % (name, scale, err.max(), rel_max,
                                                                                      err.mean(), rel_mean))
    assert rel_max <= MAX_REL, "%s %s: max rel error %.3g" % (label, name, rel_max)
    assert rel_mean <= MEAN_REL, "%s %s: mean rel error %.3g" % (label, name, rel_mean)


@pytest.mark.parametrize("name,w", CASES, ids=[n for n, _ in CASES])
def test_backward_matches_oracle(name, w):
    _say("backward", name)
    x = synth.make_inputs(w, SEED)
    g = gpu_prefill(w, x)
    dO = synth.normal((w.B, w.Hq, w.N, w.d), SEED, T_DO, synth.BF16)
    got = gpu_backward(w, x, g, dO)
    ref = oracle_backward(w, x, g["sel_idx"], dO)
    names = ["dq", "dk", "dv"] + (["dlmk"] if w.C else []) + (["dD", "dU"] if w.qcal_rank else [])
    for n in names:
        _compare(n, got[n], ref[n], name)


def test_backward_rejects_fp32_io():
    w = synth.Workload("bw_f32", B=1, Hq=1, Hkv=1, d=64, N=128, K=2, io=synth.F32)
    dm = dims_of(w)
    z = torch.zeros(1, device="cuda")
    lib = hils.load()
    import ctypes
    p = ctypes.c_void_p(z.data_ptr())
    rc = lib.hils_attn_prefill_backward(ctypes.byref(dm), p, p, p, p, p, None, None, p, p, p, p, p, p, p, p, None,
                                        None, p, 1 << 30, None)
    assert rc == hils.E_UNSUPPORTED
