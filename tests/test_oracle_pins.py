"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Every test here runs on the CPU.  Each pin is chosen so that a plausible slip
in the oracle (a dropped term, a wrong sign, scale or index, a transposed
operand, a wrong tie rule) fails at least one of them:
  * the pages' worked example of the chunk score (tests/golden);
  * closed forms of the landmark compression (uniform weights, one dominant key);
  * the first-order Taylor identity behind the entropy bias (the surrogate is the
    tangent plane of the chunk's log-sum-exp at the landmark query), hence a
    global upper bound with equality at the landmark query;
  * chunk-constant keys, where the surrogate is exact;
  * brute-force top-K with the lower-index tie rule;
  * reductions of the whole pipeline to dense causal attention, checked against
    torch's scaled_dot_product_attention in float64 on the CPU;
  * Q-Cal special cases (D = 0, U D = I);
  * the dense causal baseline against torch SDPA (grouped heads), its identical-key
    closed form, and its equality with the HiLS pass under exact chunk scores;
  * a second, vectorised formulation of the full forward pass on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _dense_causal(q, k, v, pos_list, tau):
    """Textbook causal attention of queries q[n] at positions pos_list over k, v (torch SDPA)."""
    out = []
    for qi, p in zip(q, pos_list):
        qt = torch.from_numpy(np.asarray(qi, np.float64)).view(1, 1, 1, -1)
        kt = torch.from_numpy(np.asarray(k[: p + 1], np.float64)).view(1, 1, p + 1, -1)
        vt = torch.from_numpy(np.asarray(v[: p + 1], np.float64)).view(1, 1, p + 1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=tau)
        out.append(o.view(-1).numpy())
    return np.stack(out)


def test_worked_example_score():
    """aitrends.kr 'Methodology': q.k'/sqrt(64) = 2.0 and b' = 0.7 give s = 2.7, exp(s) ~ 14.9."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    d = g["d"]
    s = oracle.shape(1, 1, 1, d, N=128, S=64, K=1)
    # q = 4 e0 and k' = 4 e0: q.k' = 16, /sqrt(64) = 2.0
    q = np.zeros(d)
    q[0] = 4.0
    kc = np.zeros((1, 1, 2, d))
    kc[0, 0, 0, 0] = 4.0
    bc = np.zeros((1, 1, 2))
    bc[0, 0, 0] = g["b_prime"]
    sc = oracle.row_scores(s, 0, 0, 64, q, kc=kc, bc=bc)
    assert sc.shape == (1,)
    assert abs(sc[0] - g["score"]) < 1e-12
    assert abs(math.exp(sc[0]) - g["exp_score_as_printed"]) < g["printed_precision"]


def test_worked_example_fusion_weight():
    """Fusion by a softmax over chunk scores: chunk A (s = 2.7, v = 1) vs chunk B (s = 0, v = 0)."""
    d, S = 64, 64
    N = 3 * S
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=2)
    q = np.zeros(d)
    q[0] = 4.0
    kc = np.zeros((1, 1, 3, d))
    kc[0, 0, 0, 0] = 4.0
    bc = np.zeros((1, 1, 3))
    bc[0, 0, 0] = 0.7
    k = np.zeros((1, 1, N, d))
    k[0, 0, 2 * S:, 0] = -40.0          # own chunk: logits -20 -> tiny own weight
    v = np.zeros((1, 1, N, d))
    v[0, 0, :S, :] = 1.0                 # chunk A values 1, chunk B values 0, own values 0
    pos = 2 * S + 5
    r = oracle.attend(s, [0], [0], [pos], q[None], k, v, kc, bc)
    assert list(r["sel_idx"][0]) == [0, 1]
    lse_own = r["lse_own"][0]
    assert abs(lse_own - (-20.0 + math.log(6))) < 1e-12
    w_a = math.exp(2.7) / (math.exp(2.7) + 1.0 + math.exp(lse_own))
    np.testing.assert_allclose(r["o"][0], np.full(d, w_a), rtol=0, atol=1e-14)
    assert abs(w_a - 14.8797 / 15.8797) < 1e-4


def _compress_one(keys, L):
    """oracle compress of one chunk (keys [S, d], landmark query L [d])."""
    S, d = keys.shape
    s = oracle.shape(1, 1, 1, d, N=S, S=S, K=1)
    kc, bc = oracle.compress(s, keys.reshape(1, 1, S, d).astype(np.float64),
                             np.asarray(L, np.float64).reshape(1, 1, 1, d))
    return kc[0, 0, 0], bc[0, 0, 0]


def test_compress_identical_keys():
    rng = _rng(1)
    key = rng.standard_normal(64)
    keys = np.tile(key, (64, 1))
    kc, bc = _compress_one(keys, rng.standard_normal(64))
    np.testing.assert_allclose(kc, key, rtol=0, atol=1e-13)
    assert abs(bc - math.log(64)) < 1e-12
    assert abs(bc - 4.158883) < 1e-6


def test_compress_zero_landmark_is_mean():
    rng = _rng(2)
    keys = rng.standard_normal((64, 128))
    kc, bc = _compress_one(keys, np.zeros(128))
    np.testing.assert_allclose(kc, keys.mean(0), rtol=0, atol=1e-13)
    assert abs(bc - math.log(64)) < 1e-12


def test_compress_dominant_key():
    rng = _rng(3)
    d = 64
    keys = 0.01 * rng.standard_normal((64, d))
    keys[17, 0] = 10.0
    L = np.zeros(d)
    L[0] = 100.0                       # logit of key 17 = 1000/8 = 125, others ~ 0
    kc, bc = _compress_one(keys, L)
    assert 0.0 <= bc < 1e-40
    np.testing.assert_allclose(kc, keys[17], rtol=0, atol=1e-40)


def test_compress_random_bounds_and_taylor_identity():
    """b' = LSE_j(tau L.k_j) - tau L.k' (the Taylor constant term equals the entropy)."""
    rng = _rng(4)
    for d in (64, 128):
        tau = 1 / math.sqrt(d)
        for trial in range(20):
            keys = rng.standard_normal((64, d)) * (1 + trial % 3)
            L = rng.standard_normal(d) * (1 + trial % 4)
            kc, bc = _compress_one(keys, L)
            z = tau * keys @ L
            lse = z.max() + math.log(np.exp(z - z.max()).sum())
            assert abs(bc - (lse - tau * L @ kc)) < 1e-11
            assert -1e-12 <= bc <= math.log(64) + 1e-12
            assert np.all(kc <= keys.max(0) + 1e-12) and np.all(kc >= keys.min(0) - 1e-12)


def _random_chunks(rng, C, S, d, scale=1.0):
    k = rng.standard_normal((1, 1, C * S, d)) * scale
    lmk = rng.standard_normal((1, 1, C, d))
    return k, lmk


def test_surrogate_is_tangent_upper_bound():
    """s_ic <= LSE_c(q) for every q (convexity), with equality when q is the landmark query."""
    rng = _rng(5)
    d, S, C = 64, 64, 8
    tau = 1 / math.sqrt(d)
    s = oracle.shape(1, 1, 1, d, N=(C + 1) * S, S=S, K=4)
    k = rng.standard_normal((1, 1, (C + 1) * S, d))
    lmk = rng.standard_normal((1, 1, C + 1, d)) * 1.5
    kc, bc = oracle.compress(s, k, lmk)
    pos = C * S + 3
    for trial in range(30):
        q = rng.standard_normal(d) * (0.5 + trial / 10)
        sur = oracle.row_scores(s, 0, 0, pos, q, kc=kc, bc=bc)
        ex = oracle.row_scores(s, 0, 0, pos, q, k=k, mode=oracle.EXACT)
        assert sur.shape == (C,)
        for c in range(C):
            z = tau * k[0, 0, c * S:(c + 1) * S] @ q
            lse = z.max() + math.log(np.exp(z - z.max()).sum())
            assert abs(ex[c] - lse) < 1e-11
        assert np.all(sur <= ex + 1e-11)
    for c in range(C):
        L = lmk[0, 0, c]
        sur = oracle.row_scores(s, 0, 0, pos, L, kc=kc, bc=bc)
        ex = oracle.row_scores(s, 0, 0, pos, L, k=k, mode=oracle.EXACT)
        assert abs(sur[c] - ex[c]) < 1e-11


def test_chunk_constant_keys_surrogate_exact():
    rng = _rng(6)
    d, S, C = 64, 64, 6
    s = oracle.shape(1, 1, 1, d, N=(C + 1) * S, S=S, K=3)
    kappa = rng.standard_normal((C + 1, d))
    k = np.repeat(kappa, S, axis=0).reshape(1, 1, (C + 1) * S, d)
    lmk = rng.standard_normal((1, 1, C + 1, d))
    kc, bc = oracle.compress(s, k, lmk)
    np.testing.assert_allclose(bc[0, 0], math.log(S), atol=1e-12)
    for trial in range(10):
        q = rng.standard_normal(d) * 2
        sur = oracle.row_scores(s, 0, 0, C * S, q, kc=kc, bc=bc)
        expect = (kappa[:C] @ q) / math.sqrt(d) + math.log(S)
        np.testing.assert_allclose(sur, expect, rtol=0, atol=1e-12)


def test_topk_bruteforce_and_order():
    rng = _rng(7)
    d, S, C, K = 64, 64, 40, 7
    N = C * S
    s = oracle.shape(1, 2, 1, d, N=N, S=S, K=K)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    lmk = rng.standard_normal((1, 2, C, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    kc, bc = oracle.compress(s, k, lmk)
    rows = [(0, h, i) for h in range(2) for i in range(0, N, 37)]
    q = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    r = oracle.prefill_rows(s, q, k, v, kc, bc, rows)
    for n, (b, h, i) in enumerate(rows):
        sc = oracle.row_scores(s, b, h, i, q[b, h, i], kc=kc, bc=bc)
        P = i // S
        assert sc.shape == (P,)
        order = np.lexsort((np.arange(P), -sc))      # score desc, then index asc
        take = np.sort(order[:min(K, P)])
        got = r["sel_idx"][n]
        assert r["nsel"][n] == min(K, P)
        assert list(got[:min(K, P)]) == list(take)
        assert np.all(got[min(K, P):] == -1)
        assert np.all(np.diff(got[:min(K, P)]) > 0)
        np.testing.assert_array_equal(r["sel_score"][n][:min(K, P)], sc[take])
        if P > K:
            srt = sc[order]
            assert r["gap"][n] == srt[K - 1] - srt[K]
        else:
            assert r["gap"][n] == np.inf


def test_topk_tie_lower_index_wins():
    """Two chunks with identical keys and landmark queries tie exactly; the lower index is kept."""
    rng = _rng(8)
    d, S, C, K = 64, 64, 6, 3
    N = (C + 1) * S
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=K)
    k = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, C + 1, d))
    k[0, 0, 4 * S:5 * S] = k[0, 0, 1 * S:2 * S]   # chunk 4 duplicates chunk 1
    lmk[0, 0, 4] = lmk[0, 0, 1]
    kc, bc = oracle.compress(s, k, lmk)
    v = rng.standard_normal((1, 1, N, d))
    hits = 0
    for trial in range(400):
        q = rng.standard_normal(d) * 2
        sc = oracle.row_scores(s, 0, 0, C * S, q, kc=kc, bc=bc)
        assert sc[1] == sc[4]
        order = np.argsort(-sc, kind="stable")
        if order[K - 1] == 1:                         # the tie sits exactly at the K boundary
            assert order[K] == 4
            r = oracle.attend(s, [0], [0], [C * S], q[None], k, v, kc, bc)
            assert 1 in r["sel_idx"][0] and 4 not in r["sel_idx"][0]
            hits += 1
    assert hits > 5


def test_dense_reduction_chunk_constant_keys():
    """Chunk-constant keys and K >= number of chunks: HiLS equals dense causal attention."""
    rng = _rng(9)
    d, S, C = 64, 64, 5
    N = C * S + 17
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=C)
    kappa = rng.standard_normal((C + 1, d))
    k = np.repeat(kappa, S, axis=0)[:N].reshape(1, 1, N, d)
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, C, d))
    q = rng.standard_normal((1, 1, N, d)) * 1.5
    kc, bc = oracle.compress(s, k, lmk)
    pos = list(range(N))
    r = oracle.prefill_rows(s, q, k, v, kc, bc, [(0, 0, i) for i in pos])
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_dense_reduction_exact_lse_mode():
    """Exact-LSE chunk scores and K >= number of chunks: HiLS equals dense causal attention."""
    rng = _rng(10)
    d, S, C = 32, 16, 7
    N = C * S + 5
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=C)
    k = rng.standard_normal((1, 1, N, d)) * 1.3
    v = rng.standard_normal((1, 1, N, d))
    q = rng.standard_normal((1, 1, N, d))
    pos = list(range(N))
    r = oracle.prefill_rows(s, q, k, v, None, None, [(0, 0, i) for i in pos], mode=oracle.EXACT)
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nw", [2, 3, 5, 40])
def test_window_exact_lse_mode_is_dense(nw):
    """Local window of nw chunks, exact-LSE scores and K >= every candidate: the window entry
    and the selected chunks partition the keys j <= i, so the fusion is dense causal attention
    (a gap or an overlap between window and candidates breaks it)."""
    rng = _rng(30 + nw)
    d, S, C = 16, 8, 9
    N = C * S + 3
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=C, W=nw * S)
    k = rng.standard_normal((1, 1, N, d)) * 1.3
    v = rng.standard_normal((1, 1, N, d))
    q = rng.standard_normal((1, 1, N, d))
    pos = list(range(N))
    r = oracle.prefill_rows(s, q, k, v, None, None, [(0, 0, i) for i in pos], mode=oracle.EXACT)
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r["nsel"], [min(C, max(0, i // S - nw + 1)) for i in pos])


def test_window_covering_the_sequence_is_dense():
    """A window longer than the sequence leaves no candidate: every row is dense causal attention."""
    rng = _rng(36)
    d, S, C = 32, 16, 6
    N = C * S
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=2, W=(C + 1) * S)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, C, d))
    q = rng.standard_normal((1, 1, N, d))
    kc, bc = oracle.compress(s, k, lmk)
    pos = list(range(N))
    r = oracle.prefill_rows(s, q, k, v, kc, bc, [(0, 0, i) for i in pos])
    assert np.all(r["nsel"] == 0)
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_window_candidates_are_the_chunks_before_it():
    """With a window of 3 chunks, a row selects among chunks c < i//S - 2 only, by the same
    surrogate scores as without a window; the window's entry is the exact softmax over keys
    (i//S - 2)*S .. i (checked against brute force)."""
    rng = _rng(37)
    d, S, C, K, nw = 16, 8, 12, 3, 3
    N = C * S
    s1 = oracle.shape(1, 1, 1, d, N=N, S=S, K=K)
    sw = oracle.shape(1, 1, 1, d, N=N, S=S, K=K, W=nw * S)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, C, d))
    q = rng.standard_normal((1, 1, N, d))
    kc, bc = oracle.compress(s1, k, lmk)
    pos = list(range(N))
    r = oracle.prefill_rows(sw, q, k, v, kc, bc, [(0, 0, i) for i in pos])
    tau = 1 / math.sqrt(d)
    for n, i in enumerate(pos):
        P = max(0, i // S - nw + 1)
        full = oracle.row_scores(s1, 0, 0, i, q[0, 0, i], kc=kc, bc=bc)
        cand = oracle.row_scores(sw, 0, 0, i, q[0, 0, i], kc=kc, bc=bc)
        assert cand.size == P
        np.testing.assert_array_equal(cand, full[:P])
        best = sorted(range(P), key=lambda c: (-cand[c], c))[:K]
        assert sorted(r["sel_idx"][n, : r["nsel"][n]].tolist()) == sorted(best)
        j0 = max(0, (i // S - nw + 1) * S)
        z = tau * (k[0, 0, j0 : i + 1] @ q[0, 0, i])
        assert abs(r["lse_own"][n] - (z.max() + math.log(np.exp(z - z.max()).sum()))) < 1e-12


def test_rows_of_first_chunk_are_dense():
    rng = _rng(11)
    d, S = 64, 64
    N = 4 * S
    s = oracle.shape(1, 1, 1, d, N=N, S=S, K=2)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, 4, d))
    q = rng.standard_normal((1, 1, N, d))
    kc, bc = oracle.compress(s, k, lmk)
    pos = list(range(S))
    r = oracle.prefill_rows(s, q, k, v, kc, bc, [(0, 0, i) for i in pos])
    assert np.all(r["nsel"] == 0)
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_chunk_size_one_is_dense():
    """S = 1: k' = k, b' = 0, the surrogate is the exact logit; K >= N gives dense attention."""
    rng = _rng(12)
    d, N = 16, 40
    s = oracle.shape(1, 1, 1, d, N=N, S=1, K=N)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 1, N, d))
    q = rng.standard_normal((1, 1, N, d))
    kc, bc = oracle.compress(s, k, lmk)
    np.testing.assert_allclose(kc[0, 0], k[0, 0], atol=0)
    assert np.all(bc == 0)
    pos = list(range(N))
    r = oracle.prefill_rows(s, q, k, v, kc, bc, [(0, 0, i) for i in pos])
    ref = _dense_causal(q[0, 0], k[0, 0], v[0, 0], pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_qcal_on_the_key_side():
    """Q-Cal as a transform of the chunk rows: q^ . k' = q . (k' + D_h^T (U_h^T k')), so
    the score the oracle computes from the calibrated query (aitrends.kr article,
    "Methodology", Q-Cal module: q^ = q + U_h (D_h q)) equals tau q . k~_hc + b'_c with
    k~_hc = k'_c + D_h^T (U_h^T k'_c), one row per query head even where query heads share
    a landmark head.  This is the reading the GPU scoring passes compute."""
    rng = _rng(29)
    d, S, C, r_ = 32, 16, 10, 8
    N = (C + 1) * S
    s = oracle.shape(1, 4, 2, d, N=N, S=S, K=4, Hl=2, r=r_)
    k = rng.standard_normal((1, 2, N, d))
    lmk = rng.standard_normal((1, 2, C + 1, d))
    q = rng.standard_normal((1, 4, N, d))
    D = rng.standard_normal((4, r_, d)) * 0.3
    U = rng.standard_normal((4, d, r_)) * 0.3
    kc, bc = oracle.compress(s, k, lmk)
    tau = 1 / math.sqrt(d)
    for h in range(4):
        lh = h // 2
        kt = kc[0, lh] + (kc[0, lh] @ U[h]) @ D[h]      # [C + 1, d]: k~ of query head h
        for i in (S, 3 * S + 5, N - 1):
            got = oracle.row_scores(s, 0, h, i, q[0, h, i], kc=kc, bc=bc, D=D, U=U)
            want = tau * (kt[:len(got)] @ q[0, h, i]) + bc[0, lh, :len(got)]
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)
            # and the query-side form, for contrast: one calibrated query against k'
            qh = q[0, h, i] + U[h] @ (D[h] @ q[0, h, i])
            np.testing.assert_allclose(got, tau * (kc[0, lh, :len(got)] @ qh) + bc[0, lh, :len(got)], rtol=0,
                                       atol=1e-11)


def test_qcal_special_cases():
    rng = _rng(13)
    d, S, C, r_ = 32, 16, 12, 32
    N = (C + 1) * S
    s0 = oracle.shape(1, 2, 1, d, N=N, S=S, K=4)
    s1 = oracle.shape(1, 2, 1, d, N=N, S=S, K=4, r=r_)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    lmk = rng.standard_normal((1, 2, C + 1, d))
    q = rng.standard_normal((1, 2, N, d))
    kc, bc = oracle.compress(s0, k, lmk)
    rows = [(0, h, i) for h in range(2) for i in range(0, N, 7)]
    # D = 0: identical to no Q-Cal
    D0 = np.zeros((2, r_, d))
    U0 = rng.standard_normal((2, d, r_))
    a = oracle.prefill_rows(s0, q, k, v, kc, bc, rows)
    b = oracle.prefill_rows(s1, q, k, v, kc, bc, rows, D=D0, U=U0)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])
    np.testing.assert_array_equal(a["o"], b["o"])
    # U D = I: q^ = 2 q for scoring; the attention itself still uses the raw q
    I = np.stack([np.eye(d)] * 2)
    for (bb, h, i) in rows[::5]:
        sc_cal = oracle.row_scores(s1, bb, h, i, q[bb, h, i], kc=kc, bc=bc, D=I, U=I)
        sc_two = oracle.row_scores(s0, bb, h, i, 2 * q[bb, h, i], kc=kc, bc=bc)
        np.testing.assert_allclose(sc_cal, sc_two, rtol=0, atol=1e-12)
    c = oracle.prefill_rows(s1, q, k, v, kc, bc, rows, D=I, U=I)
    for h in range(2):
        ref, _ = _vectorised_hils(q[0, h], k[0, 0], v[0, 0], kc[0, h], bc[0, h], S, 4, 1 / math.sqrt(d),
                                  qs=2 * q[0, h])
        sel_rows = [n for n, (bb, hh, i) in enumerate(rows) if hh == h]
        pos = [rows[n][2] for n in sel_rows]
        np.testing.assert_allclose(c["o"][sel_rows], ref[pos], rtol=0, atol=1e-12)
    # rank-1: q^ = q + u (a . q)
    av = rng.standard_normal(d)
    uv = rng.standard_normal(d)
    D1 = np.zeros((2, r_, d))
    U1 = np.zeros((2, d, r_))
    D1[1, 3] = av
    U1[1, :, 3] = uv
    qq = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.qcal(s1, 1, qq, D1, U1), qq + uv * (av @ qq), atol=1e-13)
    np.testing.assert_allclose(oracle.qcal(s1, 0, qq, D1, U1), qq, atol=0)


def _vectorised_hils(q, k, v, kc, bc, S, K, tau, qs=None):
    """Second formulation: one attention weight matrix W[i, j] for all queries at once.

    W[i, j] = softmax over chunks of the scores (selected past chunks: surrogate,
    own chunk: exact LSE), times the intra-chunk softmax of key j.  o = W v.
    qs (default q) are the vectors that score chunks; q always attends.
    """
    N, d = q.shape
    C = kc.shape[0]
    logits = tau * q @ k.T
    sur = tau * (q if qs is None else qs) @ kc.T + bc[None, :]
    W = np.zeros((N, N))
    for i in range(N):
        ci = i // S
        P = min(ci, C)
        past = list(np.lexsort((np.arange(P), -sur[i, :P]))[:min(K, P)])
        groups = [(c * S, c * S + S, sur[i, c]) for c in past]
        lo, hi = ci * S, i + 1
        zo = logits[i, lo:hi]
        groups.append((lo, hi, zo.max() + math.log(np.exp(zo - zo.max()).sum())))
        sig = np.array([g[2] for g in groups])
        wc = np.exp(sig - sig.max())
        wc /= wc.sum()
        for (a, b, _), w in zip(groups, wc):
            z = logits[i, a:b]
            p = np.exp(z - z.max())
            W[i, a:b] += w * p / p.sum()
    return W @ v, W


def test_second_formulation_tiny():
    rng = _rng(14)
    for (d, S, C, K, extra) in [(16, 8, 9, 3, 5), (32, 16, 6, 2, 0), (8, 4, 20, 6, 3)]:
        N = C * S + extra
        s = oracle.shape(1, 1, 1, d, N=N, S=S, K=K)
        k = rng.standard_normal((1, 1, N, d))
        v = rng.standard_normal((1, 1, N, d))
        lmk = rng.standard_normal((1, 1, C, d))
        q = rng.standard_normal((1, 1, N, d)) * 1.7
        kc, bc = oracle.compress(s, k, lmk)
        r = oracle.prefill_rows(s, q, k, v, kc, bc, [(0, 0, i) for i in range(N)])
        ref, W = _vectorised_hils(q[0, 0], k[0, 0], v[0, 0], kc[0, 0], bc[0, 0], S, K, 1 / math.sqrt(d))
        np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)
        # fusion weights form a probability distribution and outputs are convex combinations
        np.testing.assert_allclose(W.sum(1), 1.0, atol=1e-12)
        assert np.all(r["o"] <= v[0, 0].max(0) + 1e-12) and np.all(r["o"] >= v[0, 0].min(0) - 1e-12)


def test_decode_row_equals_prefill_row():
    """A decode query at cache length L (cache capacity > L) equals prefill row L-1."""
    rng = _rng(15)
    d, S, K = 32, 16, 3
    Ncap, L = 12 * S, 7 * S + 9
    s_cap = oracle.shape(2, 4, 2, d, N=Ncap, S=S, K=K)
    s_pre = oracle.shape(2, 4, 2, d, N=L, S=S, K=K)
    k = rng.standard_normal((2, 2, Ncap, d)).astype(np.float32)
    v = rng.standard_normal((2, 2, Ncap, d)).astype(np.float32)
    lmk = rng.standard_normal((2, 4, Ncap // S, d)).astype(np.float32)
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    kc, bc = oracle.compress(s_cap, k, lmk)
    kp, vp = np.ascontiguousarray(k[:, :, :L]), np.ascontiguousarray(v[:, :, :L])
    kcp, bcp = oracle.compress(s_pre, kp, np.ascontiguousarray(lmk[:, :, :L // S]))
    np.testing.assert_array_equal(kcp, kc[:, :, :L // S])
    rows_b = [b for b in range(2) for h in range(4)]
    rows_h = [h for b in range(2) for h in range(4)]
    dec = oracle.attend(s_cap, rows_b, rows_h, [L - 1] * 8, q.reshape(8, d), k, v, kc, bc)
    qfull = np.zeros((2, 4, L, d), np.float32)
    qfull[:, :, L - 1] = q
    pre = oracle.prefill_rows(s_pre, qfull, kp, vp, kcp, bcp, [(b, h, L - 1) for b in range(2) for h in range(4)])
    np.testing.assert_array_equal(dec["sel_idx"], pre["sel_idx"])
    np.testing.assert_allclose(dec["o"], pre["o"], rtol=0, atol=1e-15)


def test_grouped_heads_use_their_kv_and_landmark_heads():
    """GQA mapping: query head h reads KV head h // G and landmark head h // (Hq / Hl)."""
    rng = _rng(16)
    d, S, C, K = 16, 8, 6, 2
    N = C * S + 3
    B, Hq, Hkv = 2, 4, 2
    s = oracle.shape(B, Hq, Hkv, d, N=N, S=S, K=K)
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    lmk = rng.standard_normal((B, Hq, C, d))
    q = rng.standard_normal((B, Hq, N, d))
    kc, bc = oracle.compress(s, k, lmk)
    for b in range(B):
        for h in range(Hq):
            kvh = h // 2
            s1 = oracle.shape(1, 1, 1, d, N=N, S=S, K=K)
            kc1, bc1 = oracle.compress(s1, k[b:b + 1, kvh:kvh + 1], lmk[b:b + 1, h:h + 1])
            np.testing.assert_array_equal(kc1[0, 0], kc[b, h])
            rows = [(b, h, i) for i in range(0, N, 5)]
            full = oracle.prefill_rows(s, q, k, v, kc, bc, rows)
            one = oracle.prefill_rows(s1, q[b:b + 1, h:h + 1], k[b:b + 1, kvh:kvh + 1],
                                      v[b:b + 1, kvh:kvh + 1], kc1, bc1, [(0, 0, i) for (_, _, i) in rows])
            np.testing.assert_array_equal(full["o"], one["o"])


def test_generator_reproducible_and_rounding():
    a = synth.normal(10001, 5, 2, synth.F32)
    b = synth.normal(10001, 5, 2, synth.F32)
    np.testing.assert_array_equal(a, b)
    assert abs(a.mean()) < 0.05 and abs(a.std() - 1) < 0.05
    c = synth.normal(10001, 6, 2, synth.F32)
    assert not np.array_equal(a, c)
    # bf16 output is the round-to-nearest-even of the float output (checked with torch's conversion)
    h = synth.normal(10001, 5, 2, synth.BF16)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(h, ref)
    # tokens(): element (b,h,n,e) equals the flat stream; planting adds alpha*u on masked tokens
    B, H, N, d = 2, 3, 5, 4
    flat = synth.normal(B * H * N * d, 9, 3, synth.F64).reshape(B, H, N, d)
    t0 = synth.tokens(B, H, N, d, 9, 3, synth.F64)
    np.testing.assert_array_equal(flat, t0)
    u = np.arange(d, dtype=np.float64)
    mask = np.zeros((B, N), np.uint8)
    mask[1, 2] = 1
    t1 = synth.tokens(B, H, N, d, 9, 3, synth.F64, 1.0, u, 3.0, mask)
    diff = t1 - t0
    assert np.all(diff[1, :, 2] == 3.0 * u) and np.count_nonzero(diff) == H * (d - 1)


def test_workload_structure():
    w = synth.scaled(synth.WORKLOADS["prefill_8k"], N=4096)
    x = synth.make_inputs(w, 1234)
    assert x["q"].shape == (1, 16, 4096, 64) and x["k"].shape == (1, 4, 4096, 64)
    assert x["lmk"].shape == (1, 16, 64, 64)
    nd = synth.needle_chunks(64, 0.02, 1234, 0)
    assert len(nd) == 1
    nd = synth.needle_chunks(2048, 0.02, 1234, 0)
    assert len(nd) == 41 and np.all(np.diff(nd) > 0)
    pp = synth.planted_positions(4096, 0.25, 1234, 0)
    assert len(pp) == 1024 and len(np.unique(pp)) == 1024


def _dense_case(seed, B, Hq, Hkv, d, N):
    rng = _rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)) * 1.2
    v = rng.standard_normal((B, Hkv, N, d))
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(0, N, 7)]
    return q, k, v, np.asarray(rows)


def test_dense_baseline_matches_sdpa_grouped_heads():
    """oracle.dense = causal softmax attention, each query head reading KV head h // (Hq/Hkv)."""
    B, Hq, Hkv, d, N = 2, 4, 2, 32, 90
    q, k, v, rows = _dense_case(21, B, Hq, Hkv, d, N)
    s = oracle.shape(B, Hq, Hkv, d, N=N)
    o = oracle.dense(s, rows[:, 0], rows[:, 1], rows[:, 2], q[rows[:, 0], rows[:, 1], rows[:, 2]], k, v)
    for t, (b, h, i) in enumerate(rows):
        kvh = h // (Hq // Hkv)
        ref = _dense_causal(q[b, h, i][None], k[b, kvh], v[b, kvh], [i], 1 / math.sqrt(d))[0]
        np.testing.assert_allclose(o[t], ref, rtol=0, atol=1e-12)


def test_dense_baseline_identical_keys_is_prefix_mean():
    """Identical keys give uniform weights: the output is the mean of v[0..i]."""
    rng = _rng(22)
    d, N = 16, 50
    s = oracle.shape(1, 1, 1, d, N=N)
    k = np.repeat(rng.standard_normal((1, d)), N, axis=0).reshape(1, 1, N, d)
    v = rng.standard_normal((1, 1, N, d))
    q = rng.standard_normal((1, 1, N, d))
    pos = np.arange(N)
    o = oracle.dense(s, np.zeros(N), np.zeros(N), pos, q[0, 0], k, v)
    ref = np.cumsum(v[0, 0], axis=0) / (pos[:, None] + 1)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_dense_baseline_equals_hils_with_exact_scores():
    """With exact chunk LSEs and every past chunk selected, the hierarchical softmax is the dense one."""
    B, Hq, Hkv, d, N = 1, 4, 2, 32, 5 * 64 + 9
    q, k, v, rows = _dense_case(23, B, Hq, Hkv, d, N)
    s = oracle.shape(B, Hq, Hkv, d, N=N, S=64, K=5)
    o = oracle.dense(s, rows[:, 0], rows[:, 1], rows[:, 2], q[rows[:, 0], rows[:, 1], rows[:, 2]], k, v)
    r = oracle.prefill_rows(s, q, k, v, None, None, rows, mode=oracle.EXACT)
    np.testing.assert_allclose(o, r["o"], rtol=0, atol=1e-12)
