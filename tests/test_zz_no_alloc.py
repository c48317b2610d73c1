"""hils_attn_decode_noalloc (the decode step with the library's own scratch, for callers
that cannot allocate) against hils_attn_decode on the same inputs, through the C ABI:
two calls in a row, the second with a smaller input, each bit-identical to the entry
point with a caller workspace (the same kernels on the same inputs)."""
import sys

import numpy as np
import pytest
import torch

import synth
from hils_testutil import dims_of, upload
from long_context_chunk_amd import hils

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    x = synth.make_inputs(w, seed)
    dm = dims_of(w)
    k, v, lmk = upload(x["k"], w.io), upload(x["v"], w.io), upload(x["lmk"], w.io)
    kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
    hils.landmark_compress(dm, k, lmk, kc, bc)
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    return dm, upload(x["q"], w.io), k, v, torch.from_numpy(x["seq_lens"]).cuda(), kc, bc, D, U


CASES = [
    synth.Workload("noalloc_a", B=4, Hq=8, Hkv=2, d=128, N=8192, K=16, decode=True,
                   seq_lens=[8192, 5000, 640, 1], qcal_rank=8, window=256),
    synth.Workload("noalloc_b", B=2, Hq=4, Hkv=4, d=64, N=2048, K=8, decode=True, seq_lens=[2048, 999]),
]


def test_decode_noalloc_matches_decode_twice():
    for t, w in enumerate(CASES):   # the second call is the smaller input
        print("noalloc call", t, w.name, flush=True)
        dm, q, k, v, lens, kc, bc, D, U = _inputs(w, synth.BASE_SEED + 61 + t)
        o_ref = torch.full_like(q, float("nan"))
        sel_ref = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
        ws = hils.workspace(dm, hils.OP_DECODE)
        hils.attn_decode(dm, q, k, v, lens, kc, bc, o_ref, ws, qcal_D=D, qcal_U=U, sel_idx=sel_ref)
        o = torch.full_like(q, float("nan"))
        sel = torch.full((w.B, w.Hq, w.K), -7, dtype=torch.int32, device="cuda")
        hils.attn_decode_noalloc(dm, q, k, v, lens, kc, bc, o, qcal_D=D, qcal_U=U, sel_idx=sel)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), w.name
        assert torch.isfinite(o.float()).all(), w.name
        assert torch.equal(o, o_ref), (w.name, float((o.float() - o_ref.float()).abs().max()))
