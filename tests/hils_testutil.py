"""Shared helpers of the GPU parity tests: upload synthetic inputs, run the C ABI
through the binding, compute the oracle on the same bits, and compare.

Parity bar:
  * selected chunk ids bit-exact for every query whose oracle K-th/(K+1)-th
    score gap exceeds 1e-4;
  * near-tie queries (gap <= 1e-4): the GPU set must be a valid top-K within
    1e-4 of the oracle scores, and its output is compared with the oracle run on
    the GPU's own selection;
  * outputs: max |diff| <= 1e-2 and mean |diff| <= 1e-3 for bf16 I/O (fp32
    accumulation), <= 1e-5 for fp32 I/O.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from long_context_chunk_amd import hils

GAP = 1e-4
TOL = {synth.BF16: (1e-2, 1e-3), synth.F32: (1e-5, 1e-5)}


def upload(a: np.ndarray, io: int) -> torch.Tensor:
    if io == synth.BF16 and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def download_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def dims_of(w: synth.Workload) -> hils.Dims:
    return hils.dims(w.B, w.Hq, w.Hkv, w.d, w.N, w.K, S=w.S, qcal_rank=w.qcal_rank, io=w.io, Hlmk=w.Hlmk,
                     window=w.window)


def shape_of(w: synth.Workload) -> oracle.Shape:
    return oracle.shape(w.B, w.Hq, w.Hkv, w.d, w.N, S=w.S, K=w.K, Hl=w.Hlmk, r=w.qcal_rank, W=w.window)


def gpu_compress(w, x):
    dm = dims_of(w)
    k = upload(x["k"], w.io)
    lmk = upload(x["lmk"], w.io)
    kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
    hils.landmark_compress(dm, k, lmk, kc, bc)
    torch.cuda.synchronize()
    return kc, bc


def gpu_prefill(w, x, fused=True, kc=None, bc=None):
    """Full prefill through hils_attn_prefill.  Returns numpy outputs."""
    dm = dims_of(w)
    q, k, v = upload(x["q"], w.io), upload(x["k"], w.io), upload(x["v"], w.io)
    dt = q.dtype
    o = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.float32, device="cuda")
    ws = hils.workspace(dm, hils.OP_PREFILL)
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    if fused:
        kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
        bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
        hils.attn_prefill(dm, q, k, v, o, ws, lmk_q=upload(x["lmk"], w.io), kc=kc, bc=bc, qcal_D=D, qcal_U=U,
                          sel_idx=sel, sel_score=scr)
    else:
        hils.attn_prefill(dm, q, k, v, o, ws, kc=kc, bc=bc, qcal_D=D, qcal_U=U, sel_idx=sel, sel_score=scr)
    torch.cuda.synchronize()
    assert o.dtype == dt
    out = {"o": download_f32(o), "sel_idx": sel.cpu().numpy(), "sel_score": scr.cpu().numpy(),
           "kc": kc.cpu().numpy(), "bc": bc.cpu().numpy()}
    del ws
    return out


def oracle_compress(w, x):
    return oracle.compress(shape_of(w), x["k"], x["lmk"])


def oracle_rows(w, x, kc, bc, rows):
    return oracle.prefill_rows(shape_of(w), x["q"], x["k"], x["v"], kc, bc, rows, D=x.get("D"), U=x.get("U"))


def assert_ascending(sel, valid, label=""):
    """Valid ids (a prefix of each row) strictly ascending."""
    sel = np.asarray(sel)
    both = np.asarray(valid)[..., 1:]
    assert np.all(sel[..., 1:][both] > sel[..., :-1][both]), "%s: selected ids not in ascending order" % label


def check_selection_and_output(w, x, kc_o, bc_o, rows, ref, gpu_sel, gpu_score, gpu_o, label=""):
    """Compare the GPU's selection/output on `rows` with the oracle result `ref`.

    gpu_sel / gpu_score: [n, K], ascending chunk ids then padding; gpu_o: [n, d] (fp32 view
    of the io output).
    Rows whose gap exceeds GAP are checked together (array operations); near-tie rows one
    by one against the oracle's full score list.  Returns a summary dict.
    """
    s = shape_of(w)
    n = len(rows)
    K = w.K
    max_tol, mean_tol = TOL[w.io]
    gpu_sel = np.asarray(gpu_sel).reshape(n, K)
    gpu_o = np.asarray(gpu_o).reshape(n, w.d)
    ns = np.asarray(ref["nsel"])
    slot = np.arange(K)[None, :]
    valid = gpu_sel >= 0
    assert np.array_equal(valid.sum(1), ns), "%s: selected counts differ from the oracle's" % label
    assert np.array_equal(valid, slot < ns[:, None]), "%s: padding is not at the end" % label
    srt = np.sort(np.where(valid, gpu_sel, -1 - slot), axis=1)
    assert np.all(np.diff(srt, axis=1) != 0), "%s: duplicate chunk ids in a row" % label
    assert_ascending(gpu_sel, valid, label)
    o_sel = np.where(slot < ns[:, None], np.asarray(ref["sel_idx"]), -1 - slot)
    exact = np.asarray(ref["gap"]) > GAP
    same = np.all(np.sort(o_sel, axis=1) == srt, axis=1)
    bad = np.flatnonzero(exact & ~same)
    if bad.size:
        t = int(bad[0])
        raise AssertionError("%s: %d rows select different chunks; first row %s (gap %.3g)\n gpu %s\n ora %s" % (
            label, bad.size, rows[t], ref["gap"][t], srt[t][srt[t] >= 0], np.sort(o_sel[t][o_sel[t] >= 0])))
    diffs = np.zeros((n, w.d))
    diffs[exact] = gpu_o[exact] - np.asarray(ref["o"])[exact]
    if gpu_score is not None and exact.any():  # scores of the exact rows, slot by slot (both lists ascending)
        gs = np.asarray(gpu_score).reshape(n, K)[exact]
        rs = np.where(slot < ns[:, None], np.asarray(ref["sel_score"]), -np.inf)[exact]
        live = (slot < ns[exact][:, None])
        assert np.all(np.isfinite(gs[live])), "%s: non-finite selected score" % label
        err = np.abs(gs[live] - rs[live])
        assert err.size == 0 or err.max() <= 2e-5, "%s: selected scores differ by %.3g" % (label, err.max())
        assert np.all(np.isneginf(gs[~live]))
    tie_rows = np.flatnonzero(~exact)
    if tie_rows.size:
        tr = [rows[t] for t in tie_rows]
        for t in tie_rows:
            b, h, i = rows[t]
            g_valid = gpu_sel[t][gpu_sel[t] >= 0]
            allsc = oracle.row_scores(s, b, h, i, x["q"][b, h, i], kc=kc_o, bc=bc_o, D=x.get("D"), U=x.get("U"))
            chosen = np.zeros(len(allsc), bool)
            chosen[g_valid] = True
            if chosen.any() and (~chosen).any():
                assert allsc[chosen].min() >= allsc[~chosen].max() - GAP, "%s row %s: invalid near-tie set" % (
                    label, rows[t])
        qt = np.stack([np.asarray(x["q"][b, h, i]) for b, h, i in tr])
        r2 = oracle.attend(s, [r[0] for r in tr], [r[1] for r in tr], [r[2] for r in tr], qt, x["k"], x["v"], kc_o,
                           bc_o, D=x.get("D"), U=x.get("U"), sel_in=gpu_sel[tie_rows])
        diffs[tie_rows] = gpu_o[tie_rows] - r2["o"]
    ad = np.abs(diffs)
    assert np.all(np.isfinite(ad)), "%s: non-finite output" % label
    assert ad.max() <= max_tol, "%s: max |diff| %.3g > %.3g" % (label, ad.max(), max_tol)
    assert ad.mean() <= mean_tol, "%s: mean |diff| %.3g > %.3g" % (label, ad.mean(), mean_tol)
    return {"rows": n, "exact_rows": int(exact.sum()), "near_tie_rows": int(tie_rows.size), "max_abs": float(ad.max()),
            "mean_abs": float(ad.mean())}


def check_selection(w, x, kc_o, bc_o, rows, ref, gpu_sel, gpu_score, label=""):
    """Selection only (no output): bit-exact sets where the gap exceeds GAP, ids ascending,
    scores within 2e-5 there slot by slot, valid top-K sets within GAP on near-tie rows."""
    s = shape_of(w)
    n, K = len(rows), w.K
    gpu_sel = np.asarray(gpu_sel).reshape(n, K)
    gpu_score = np.asarray(gpu_score).reshape(n, K)
    ns = np.asarray(ref["nsel"])
    slot = np.arange(K)[None, :]
    valid = gpu_sel >= 0
    assert np.array_equal(valid, slot < ns[:, None]), "%s: selected counts or padding differ" % label
    assert np.all(np.isneginf(gpu_score[~valid])) and np.all(np.isfinite(gpu_score[valid]))
    srt = np.sort(np.where(valid, gpu_sel, -1 - slot), axis=1)
    assert np.all(np.diff(srt, axis=1) != 0), "%s: duplicate chunk ids" % label
    assert_ascending(gpu_sel, valid, label)
    o_sel = np.sort(np.where(slot < ns[:, None], np.asarray(ref["sel_idx"]), -1 - slot), axis=1)
    exact = np.asarray(ref["gap"]) > GAP
    bad = np.flatnonzero(exact & ~np.all(srt == o_sel, axis=1))
    assert bad.size == 0, "%s: %d rows select different chunks (first %s)" % (label, bad.size, rows[int(bad[0])])
    rs = np.where(slot < ns[:, None], np.asarray(ref["sel_score"]), -np.inf)  # both lists ascending
    live = valid & exact[:, None]
    if live.any():
        err = np.abs(gpu_score[live] - rs[live])
        assert err.max() <= 2e-5, "%s: selected scores differ by %.3g" % (label, err.max())
    for t in np.flatnonzero(~exact):
        b, h, i = rows[t]
        allsc = oracle.row_scores(s, b, h, i, x["q"][b, h, i], kc=kc_o, bc=bc_o, D=x.get("D"), U=x.get("U"))
        chosen = np.zeros(len(allsc), bool)
        chosen[gpu_sel[t][gpu_sel[t] >= 0]] = True
        if chosen.any() and (~chosen).any():
            assert allsc[chosen].min() >= allsc[~chosen].max() - GAP, "%s row %s: invalid near-tie set" % (label, rows[t])
    return {"rows": n, "exact_rows": int(exact.sum()), "near_tie_rows": int((~exact).sum())}


def gpu_decode(w, x, kc=None, bc=None, mirror=False):
    """One decode step through hils_attn_decode (mirror=True: the landmark mirror is built
    with hils_landmark_mirror and the step runs through hils_attn_decode_mirror)."""
    dm = dims_of(w)
    k, v = upload(x["k"], w.io), upload(x["v"], w.io)
    if kc is None:
        kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
        bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
        hils.landmark_compress(dm, k, upload(x["lmk"], w.io), kc, bc)
    q = upload(x["q"], w.io)
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    o = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hq, w.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE_MIRROR if mirror else hils.OP_DECODE)
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    kcm = None
    if mirror:
        kcm = torch.zeros(hils.mirror_shape(dm), dtype=torch.uint8, device="cuda")
        hils.landmark_mirror(dm, kc, bc, kcm)
    hils.attn_decode(dm, q, k, v, lens, kc, bc, o, ws, qcal_D=D, qcal_U=U, sel_idx=sel, kc_mirror=kcm)
    torch.cuda.synchronize()
    return {"o": download_f32(o), "o_bits": o.view(torch.int16 if w.io == synth.BF16 else torch.int32).cpu().numpy(),
            "sel_idx": sel.cpu().numpy(), "kc": kc, "bc": bc, "kcm": kcm}
