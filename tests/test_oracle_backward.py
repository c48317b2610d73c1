"""Pins of the oracle's backward pass (CPU only).

The backward is checked against central finite differences of the oracle's
forward pass with the selection held fixed (the forward is pinned on its own in
test_oracle_pins.py), for every input element of a tiny ragged case, with and
without a local window and Q-Cal; and, where HiLS reduces to dense attention
(a window longer than the sequence), against torch autograd of textbook dense
causal attention in float64.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _case(seed, W, r, N=37, d=8, S=4, K=2, Hq=2, Hkv=1, Hl=None):
    rng = np.random.default_rng(seed)
    Hl = Hq if Hl is None else Hl
    s = oracle.shape(1, Hq, Hkv, d, N=N, S=S, K=K, r=r, W=W, Hl=Hl)
    C = N // S
    x = {
        "q": rng.standard_normal((1, Hq, N, d)),
        "k": rng.standard_normal((1, Hkv, N, d)),
        "v": rng.standard_normal((1, Hkv, N, d)),
        "lmk": rng.standard_normal((1, Hl, C, d)),
        "D": rng.standard_normal((Hq, r, d)) * 0.3 if r else None,
        "U": rng.standard_normal((Hq, d, r)) * 0.3 if r else None,
    }
    rows = [(0, h, i) for h in range(Hq) for i in range(N)]
    R = rng.standard_normal((len(rows), d))
    return s, x, rows, R


def _forward(s, x, rows, sel, kc=None, bc=None):
    if kc is None:
        kc, bc = oracle.compress(s, x["k"], x["lmk"])
    rr = np.asarray(rows)
    qrows = x["q"][rr[:, 0], rr[:, 1], rr[:, 2]]
    return oracle.attend(s, rr[:, 0], rr[:, 1], rr[:, 2], qrows, x["k"], x["v"], kc, bc, D=x["D"], U=x["U"],
                         sel_in=sel)


def _grads(s, x, rows, R):
    kc, bc = oracle.compress(s, x["k"], x["lmk"])
    rr = np.asarray(rows)
    qrows = x["q"][rr[:, 0], rr[:, 1], rr[:, 2]]
    f0 = oracle.attend(s, rr[:, 0], rr[:, 1], rr[:, 2], qrows, x["k"], x["v"], kc, bc, D=x["D"], U=x["U"])
    sel = f0["sel_idx"]
    g = oracle.attend_backward(s, rr[:, 0], rr[:, 1], rr[:, 2], qrows, x["k"], x["v"], kc, bc, x["lmk"], sel, R,
                               D=x["D"], U=x["U"])
    dq = np.zeros_like(x["q"])
    dq[rr[:, 0], rr[:, 1], rr[:, 2]] = g["dq"]
    g["dq_full"] = dq
    return g, sel, kc, bc


@pytest.mark.parametrize("W,r", [(0, 0), (8, 2), (12, 0), (4, 3)])
def test_backward_matches_finite_differences(W, r):
    """Every element of q, k, v, the landmark queries, D, U, k' and b'."""
    _check_finite_differences(*_case(40 + W + r, W, r))


def test_backward_shared_landmark_heads_matches_finite_differences():
    """Two query heads per landmark head, each with its own Q-Cal: the landmark
    gradients gather both heads' score terms."""
    _check_finite_differences(*_case(61, 0, 2, Hq=4, Hkv=2, Hl=2))


def _check_finite_differences(s, x, rows, R):
    g, sel, kc, bc = _grads(s, x, rows, R)
    eps = 1e-6
    loss = lambda **kw: float(np.sum(R * _forward(s, kw.get("x", x), rows, sel, kw.get("kc"), kw.get("bc"))["o"]))
    checks = [("q", "dq_full"), ("k", "dk"), ("v", "dv"), ("lmk", "dlmk")] + ([("D", "dD"), ("U", "dU")] if x["D"] is not None else [])
    for name, gname in checks:
        a = x[name]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp = loss()
            a[idx] = old - eps
            lm = loss()
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=0, atol=2e-7, err_msg=name)
        assert np.abs(fd).max() > 1e-3, name  # the check is not vacuous
    # k' and b' directly (the compression's inputs to the scores)
    for name, arr, gname in (("kc", kc, "dkc"), ("bc", bc, "dbc")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(kc=kc, bc=bc)
            arr[idx] = old - eps
            lm = loss(kc=kc, bc=bc)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=0, atol=2e-7, err_msg=name)
        assert np.abs(fd).max() > 1e-3, name


def test_backward_of_window_covering_sequence_is_dense_attention_backward():
    """With a window longer than the sequence there is no selection: the output is dense
    causal attention, so dq, dk, dv are its gradients (torch autograd, float64)."""
    s, x, rows, R = _case(50, W=64, r=0, N=30, S=4)
    g, sel, _, _ = _grads(s, x, rows, R)
    assert np.all(sel == -1)
    Hq, N, d = 2, 30, 8
    q = torch.tensor(x["q"][0], requires_grad=True)
    k = torch.tensor(x["k"][0, 0], requires_grad=True)
    v = torch.tensor(x["v"][0, 0], requires_grad=True)
    logits = torch.einsum("hnd,md->hnm", q, k) / math.sqrt(d)
    mask = torch.triu(torch.ones(N, N, dtype=torch.bool), 1)
    o = torch.softmax(logits.masked_fill(mask, -math.inf), dim=-1) @ v
    (o.reshape(Hq * N, d) * torch.tensor(R)).sum().backward()
    np.testing.assert_allclose(g["dq_full"][0], q.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"][0, 0], k.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dv"][0, 0], v.grad.numpy(), rtol=0, atol=1e-12)
    assert np.all(g["dlmk"] == 0) and np.all(g["dkc"] == 0)
