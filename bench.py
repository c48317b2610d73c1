"""Benchmark of the HiLS-Attention forward pass on one MI355X.

One step = one full prefill pass of a 7B-like attention layer at 256K context
(B=1, 32 query / 8 KV heads, d=128, S=64, K=32, bf16 I/O, Q-Cal rank 32,
landmark compression in the same call): compression, Q-Cal, chunk scoring +
top-K, intra-chunk attention and fusion, all through hils_attn_prefill.
Inputs are synthetic (seeded, with the planted-direction retrieval structure)
and resident in HBM before timing starts.

Also reported on the same line:
  * decode: one decode step of 8 sequences against a 512K-token KV cache
    (32/8 heads, d=128, K=32), microseconds per step, with its roofline;
  * roofline of the dominant prefill kernel from HIP-event stage times;
  * cpu_baseline: the fp64 oracle on a bounded sample of the same workload;
  * dense: this library's dense causal attention kernel (same MFMA tiles) and
    torch SDPA on the same q/k/v (the pages compare against full attention);
    for decode, this library's dense decode kernel and a torch dense step on the
    same cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-dense]
                       [--no-prefill] [--copy-calibration] [--sweep] [--peaks]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS prefill tokens/s and decode us/step at 128K-512K ctx; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def upload(a, io):
    import torch
    import synth
    if io == synth.BF16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prefill_counts(w):
    """Algorithmic work of one prefill pass (2 flops per MAC, exp/log not counted)."""
    S, d, K, C, N = w.S, w.d, w.K, w.C, w.N
    nw = max(1, w.window // S)                   # chunks of the local window (own included)
    rows_per_head = 0
    score_macs = 0
    intra_macs = 0
    window_macs = 0
    pairs = 0
    for p in range((N + S - 1) // S):            # query chunk p holds rows p*S .. p*S+S-1
        nrow = min(S, N - p * S)
        P = min(C, max(0, p - nw + 1))           # candidates: the chunks before the window
        n = min(K, P)
        score_macs += nrow * P * d
        pairs += nrow * n
        own = sum(i + 1 for i in range(nrow))    # causal own-chunk keys
        win = own + nrow * S * min(nw - 1, p)    # plus the full window chunks before it
        intra_macs += 2 * d * (nrow * n * S + win)
        window_macs += 2 * d * win
        rows_per_head += nrow
    H = w.B * w.Hq
    return {
        "compress_flops": 4.0 * S * d * w.B * w.Hlmk * C,
        "qcal_flops": 4.0 * w.qcal_rank * d * H * rows_per_head,
        "score_flops": 2.0 * score_macs * H,
        "intra_flops": 2.0 * intra_macs * H,
        "window_flops": 2.0 * window_macs * H,
        "pairs": pairs * H,
    }


# Work of each prefill kernel.  "bound" and "work" are the method's own algorithmic counts
# (MFMA kernels: 2 flops per MAC of the products the method defines; memory kernels: the
# bytes the method must move); "design_bytes" are the bytes this implementation's data flow
# moves through memory (per-pair query gathers and partial outputs included), the
# memory-side view of the same launch.
def kernel_work(w, cnt, io_bytes=2):
    d, S, K = w.d, w.S, w.K
    rows = w.B * w.Hq * w.N
    entries = rows * K
    kv_once = w.B * w.Hkv * w.N * d * io_bytes * 2          # every K and V row read once
    compress_bytes = (w.B * w.Hkv * w.C * S * d * io_bytes + w.B * w.Hlmk * w.C * d * io_bytes
                      + w.B * w.Hlmk * w.C * (d + 1) * 4)
    return {
        # K and the landmark queries read once, k' (fp32) and b' written
        "compress": {"bound": "hbm", "work": compress_bytes, "design_bytes": compress_bytes},
        # one q^ . k' product per (query, candidate chunk) + Q-Cal
        "score_threshold": {"bound": "mfma", "work": cnt["score_flops"] + cnt["qcal_flops"]},
        "score_select": {"bound": "mfma", "work": cnt["score_flops"] + cnt["qcal_flops"]},
        # a reorganisation of the selection (no work of the method): read twice, pair ids written
        "bucket": {"bound": "hbm", "work": entries * 4 * 3, "design_bytes": entries * 4 * 3},
        # QK^T and PV of every (query, selected chunk) pair: 4 S d flops per pair; the design
        # gathers the query row and writes an fp16 output row per pair, K/V once per chunk
        "chunk_attend": {"bound": "mfma", "work": cnt["pairs"] * 4.0 * S * d,
                         "design_bytes": cnt["pairs"] * (d * io_bytes + d * 2) + w.B * w.Hkv * w.C * 2 * S * d * io_bytes},
        # the own chunk (or local window) causally: 4 d flops per (query, key); per row q, the
        # fp16 output slot and its LSE, K/V staged once per (KV head, chunk) for its query heads
        "own_attend": {"bound": "mfma", "work": cnt["window_flops"],
                       "design_bytes": rows * (d * io_bytes + d * 2 + 4) + kv_once},
        # per row: its selected chunk outputs + own output (fp16), their scores, the output row
        "fuse": {"bound": "hbm", "work": (cnt["pairs"] + rows) * d * 2 + cnt["pairs"] * 4 + rows * 4 + rows * d * io_bytes,
                 "design_bytes": (cnt["pairs"] + rows) * d * 2 + cnt["pairs"] * 4 + rows * 4 + rows * d * io_bytes},
    }


def roofline_of(kind, amount, ms):
    if kind == "hbm":
        ach = amount / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "algorithmic_bytes": amount, "ms": ms}
    ach = amount / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_flops": amount, "ms": ms}


def stage_roofline(w, cnt, stage_ms):
    out = {}
    for name, wk in kernel_work(w, cnt).items():
        ms = stage_ms.get(name, 0)
        if ms <= 0:
            continue
        r = roofline_of(wk["bound"], wk["work"], ms)
        if "design_bytes" in wk:
            gbs = wk["design_bytes"] / (ms * 1e-3) / 1e9
            r["design_traffic"] = {"bytes": wk["design_bytes"], "GBs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}
        out[name] = r
    return out


# kernel (stage) -> the source file whose hash must match the profiled one
KERNEL_SOURCES = {
    "compress": "compress.hip", "score_threshold": "score_topk.hip", "score_select": "score_topk.hip",
    "bucket": "attend.hip", "chunk_attend": "attend.hip", "own_attend": "attend.hip", "fuse": "attend.hip",
    "decode_scan": "decode.hip", "decode_merge": "decode.hip", "decode_scan_m": "decode.hip",
    "decode_merge_m": "decode.hip", "decode_attend_fused": "decode.hip", "decode_attend_fused_mirror": "decode.hip", "decode_attend": "decode.hip", "decode_combine": "decode.hip",
}


def source_hash(stage):
    import hashlib
    import glob
    csrc = os.path.join(ROOT, "long_context_chunk_amd", "csrc")
    h = hashlib.sha256()
    for f in [os.path.join(csrc, KERNEL_SOURCES[stage])] + sorted(glob.glob(os.path.join(csrc, "*.h"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the same counter's reading for a plain copy of known size),
    or None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals, kern = {}, {}
    for line in open(path):
        t = line.split()
        if not t or t[0].startswith("#"):
            continue
        if t[0] == "kernel" and len(t) >= 8:
            kern[t[1]] = {"fetch_kib": float(t[3]), "write_kib": float(t[5]), "src": t[7]}
        elif len(t) == 2:
            vals[t[0]] = float(t[1])
    k = kern.get(stage)
    if k is None or k["src"] != source_hash(stage) or "copy_bytes" not in vals:
        return None
    fs = vals["copy_bytes"] / (vals["copy_fetch_kib"] * 1024.0)
    ws = vals["copy_bytes"] / (vals["copy_write_kib"] * 1024.0)
    return k["fetch_kib"] * 1024.0 * fs + k["write_kib"] * 1024.0 * ws


def copy_calibration(nbytes=2 << 30, reps=3):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def run_prefill(w, steps, warmup, seed):
    import torch
    import synth
    from long_context_chunk_amd import hils
    t0 = time.time()
    x = synth.make_inputs(w, seed)
    log("prefill inputs generated in %.1fs" % (time.time() - t0))
    dm = hils.dims(w.B, w.Hq, w.Hkv, w.d, w.N, w.K, S=w.S, qcal_rank=w.qcal_rank, io=w.io, window=w.window)
    q, k, v, lmk = (upload(x[n], w.io) for n in ("q", "k", "v", "lmk"))
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    host = x
    o = torch.empty_like(q)
    kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.float32, device="cuda")
    ws = hils.workspace(dm, hils.OP_PREFILL)
    log("prefill workspace %.1f GiB" % (ws.numel() / 2**30))

    def step():
        hils.attn_prefill(dm, q, k, v, o, ws, lmk_q=lmk, kc=kc, bc=bc, qcal_D=D, qcal_U=U, sel_idx=sel,
                          sel_score=scr)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # one event between consecutive steps: the bracketed total gives the mean, the gaps the
    # per-step distribution (recording an event adds no synchronisation)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[steps]) / steps
    per = np.asarray([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    dist = {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)), "p90": float(np.percentile(per, 90))}
    log("prefill: %.3f ms/step (median %.3f, p10 %.3f, p90 %.3f)" % (ms, dist["median"], dist["p10"], dist["p90"]))
    # per-stage times (HIP events recorded by the library on the launch stream)
    stages = {s: 0.0 for s in hils.STAGES}
    nrep = max(1, min(steps, 5))
    for _ in range(nrep):
        r = hils.attn_prefill(dm, q, k, v, o, ws, lmk_q=lmk, kc=kc, bc=bc, qcal_D=D, qcal_U=U, sel_idx=sel,
                              sel_score=scr, timed=True)
        for s_ in stages:
            stages[s_] += r[s_] / nrep
    log("stages (ms): " + ", ".join("%s %.3f" % kv for kv in stages.items()))
    return {"ms": ms, "dist": dist, "stages": stages, "tensors": (q, k, v, o, sel, kc, bc), "host": host, "ws": ws}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, res, target_s=15.0):
    """The fp64 oracle on the host cores: landmark compression of every chunk + a uniform
    sample of query rows, timed and scaled to the full layer.  The sampled rows' oracle
    results are then compared with the benchmarked GPU output (same launch configuration):
    selection bit-exact where the K-th/(K+1)-th gap exceeds 1e-4, and the output error."""
    import oracle
    import torch
    x = res["host"]
    q, k, v, o, sel, kc, bc = res["tensors"]
    s = oracle.shape(w.B, w.Hq, w.Hkv, w.d, w.N, S=w.S, K=w.K, r=w.qcal_rank, W=w.window)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.time()
    kc_o, bc_o = oracle.compress(s, x["k"], x["lmk"])
    t_comp = time.time() - t0
    rng = np.random.default_rng(11)
    total_rows = w.B * w.Hq * w.N
    n = 256
    t_rows, done = 0.0, 0
    rows_all, refs = [], []
    while t_rows < target_s - t_comp and done < total_rows:
        rows = np.stack([rng.integers(w.B, size=n), rng.integers(w.Hq, size=n), rng.integers(w.N, size=n)], 1)
        t1 = time.time()
        r = oracle.prefill_rows(s, x["q"], x["k"], x["v"], kc_o, bc_o, rows, D=x.get("D"), U=x.get("U"))
        t_rows += time.time() - t1
        rows_all.append(rows)
        refs.append(r)
        done += n
        n *= 2
    t_full = t_comp + t_rows * total_rows / done
    cpu = {"value": w.B * w.N / t_full, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
           "sample": "landmark compression of all %d chunks x %d heads (%.1fs) + %d of %d query rows drawn "
                     "uniformly (%.1fs), scaled to the full layer" % (w.C, w.Hlmk, t_comp, done, total_rows, t_rows)}
    # the same rows on the GPU
    rr = np.concatenate(rows_all)
    gap = np.concatenate([r["gap"] for r in refs])
    nsel = np.concatenate([r["nsel"] for r in refs])
    o_ref = np.concatenate([r["o"] for r in refs])
    s_ref = np.concatenate([r["sel_idx"] for r in refs])
    idx = torch.from_numpy(rr).cuda()
    g_sel = sel[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
    g_o = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy()
    slot = np.arange(w.K)[None, :]
    g_sorted = np.sort(np.where(g_sel >= 0, g_sel, -1 - slot), 1)
    o_sorted = np.sort(np.where(slot < nsel[:, None], s_ref, -1 - slot), 1)
    exact = gap > 1e-4
    same = np.all(g_sorted == o_sorted, 1)
    err = np.abs(g_o - o_ref)[exact & same]
    parity = {"rows": int(len(rr)), "gap_rows": int(exact.sum()), "selection_exact": int((exact & same).sum()),
              "near_tie_rows": int((~exact).sum()),
              "max_abs_diff": float(err.max()) if err.size else None, "mean_abs_diff": float(err.mean()) if err.size else None}
    return cpu, parity


def _time_ms(fn, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def dense_flops(w):
    """Useful flops of dense causal attention: 4 d per (query, key <= query) pair."""
    return 4.0 * w.d * w.B * w.Hq * (w.N * (w.N + 1) / 2)


def dense_baseline(res, w, reps=2, sdpa=True):
    """Dense causal attention on the same q/k/v: this library's MFMA kernel
    (hils_dense_attention) and torch SDPA (flash / memory-efficient kernels only)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from long_context_chunk_amd import hils
    q, k, v = res["tensors"][:3]
    out = {}
    o = torch.empty_like(q)
    dm = hils.dims(w.B, w.Hq, w.Hkv, w.d, w.N, w.K, qcal_rank=0, io=w.io)
    ms = _time_ms(lambda: hils.dense_attention(dm, q, k, v, o), reps)
    fl = dense_flops(w)
    out["own"] = {"impl": "hils_dense_attention (same MFMA tiles as the sparse pass)", "ms": ms,
                  "tokens_per_s": w.B * w.N / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12,
                  "mfma_frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del o
    if sdpa:
        G = w.Hq // w.Hkv
        k2 = k.repeat_interleave(G, dim=1).contiguous()
        v2 = v.repeat_interleave(G, dim=1).contiguous()
        f = torch.nn.functional.scaled_dot_product_attention
        with torch.no_grad(), sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            ms2 = _time_ms(lambda: f(q, k2, v2, is_causal=True), reps)
        del k2, v2
        out["torch_sdpa"] = {"impl": "torch SDPA causal, flash/mem-efficient backend, KV heads repeated to Hq",
                             "ms": ms2, "tokens_per_s": w.B * w.N / (ms2 * 1e-3),
                             "tflops": fl / (ms2 * 1e-3) / 1e12}
    return out


def run_sweep(args):
    """HiLS prefill against the dense baseline over N, head layout 16/4, d = 64, K = 16:
    where the sparse pass overtakes dense attention (one JSON line per N)."""
    import torch
    import synth
    base = synth.Workload("sweep", B=1, Hq=16, Hkv=4, d=64, N=8192, K=16)
    for n in (8192, 16384, 32768, 65536, 131072, 262144, 524288):
        w = synth.scaled(base, N=n)
        w.name = "sweep_%dk" % (n // 1024)
        res = run_prefill(w, max(2, args.steps // 2), 1, synth.BASE_SEED + 5)
        dn = dense_baseline(res, w, reps=2, sdpa=n <= 131072)
        row = {"sweep": w.name, "N": n, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "K": w.K,
               "hils_ms": res["ms"], "dense_own_ms": dn["own"]["ms"], "speedup_vs_own_dense": dn["own"]["ms"] / res["ms"],
               "dense_own_tflops": dn["own"]["tflops"], "hils_stages_ms": res["stages"]}
        if "torch_sdpa" in dn:
            row["torch_sdpa_ms"] = dn["torch_sdpa"]["ms"]
        print(json.dumps(row), flush=True)
        res.clear()
        torch.cuda.empty_cache()


def run_peaks():
    """Measured ceilings on this GPU: a plain device copy and a large bf16 GEMM (hipBLASLt)."""
    import torch
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src), 5)
    copy_gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms2 = _time_ms(lambda: torch.matmul(a, b), 20)
    print(json.dumps({"peaks": {"copy_GBs_read_plus_write": copy_gbs, "copy_bytes": nbytes,
                                "bf16_gemm_tflops": 2.0 * n ** 3 / (ms2 * 1e-3) / 1e12, "gemm": "%d^3 torch.matmul" % n,
                                "spec_hbm_GBs": PEAK_HBM_GBS, "spec_bf16_tflops": PEAK_BF16_TFLOPS}}), flush=True)


def run_decode(wd, steps, warmup, seed, dense=False):
    import torch
    import synth
    from long_context_chunk_amd import hils
    t0 = time.time()
    x = synth.make_inputs(wd, seed)
    log("decode inputs generated in %.1fs" % (time.time() - t0))
    dm = hils.dims(wd.B, wd.Hq, wd.Hkv, wd.d, wd.N, wd.K, S=wd.S, qcal_rank=wd.qcal_rank, io=wd.io,
                   window=wd.window)
    kcache, vcache, lmk = (upload(x[n], wd.io) for n in ("k", "v", "lmk"))
    del x["k"], x["v"]
    q = upload(x["q"], wd.io)
    lens = torch.from_numpy(x["seq_lens"]).cuda()
    kc = torch.empty((wd.B, wd.Hlmk, wd.C, wd.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((wd.B, wd.Hlmk, wd.C), dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    hils.landmark_compress(dm, kcache, lmk, kc, bc)
    e1.record()
    torch.cuda.synchronize()
    comp_ms = e0.elapsed_time(e1)
    # the 8-bit landmark mirror (built once per chunk, like k' and b'): the scan reads it
    kcm = torch.empty(hils.mirror_shape(dm), dtype=torch.uint8, device="cuda")
    hils.landmark_mirror(dm, kc, bc, kcm)   # the first launch also loads the kernel: time the second
    e0.record()
    hils.landmark_mirror(dm, kc, bc, kcm)
    e1.record()
    torch.cuda.synchronize()
    mirror_ms = e0.elapsed_time(e1)
    o = torch.empty_like(q)
    sel = torch.empty((wd.B, wd.Hq, wd.K), dtype=torch.int32, device="cuda")
    ws = hils.workspace(dm, hils.OP_DECODE_MIRROR)   # covers both steps
    # evicting by a READ of 512 MB of unrelated data leaves the 256 MB Infinity Cache and the
    # L2s holding clean lines: a write-flush would leave dirty lines whose write-back the
    # next step's first cache-allocating kernel pays for
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def timed_steps(mirror):
        """Per-step times of plain calls (one HIP event pair per step on the launch stream, the
        caches evicted before each), then the stage times of as many timed calls (their own
        events between the stages add a few microseconds, so they are not the step time)."""
        for _ in range(warmup):
            hils.attn_decode(dm, q, kcache, vcache, lens, kc, bc, o, ws, sel_idx=sel, kc_mirror=mirror)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for ea, eb in evs:
            torch.sum(flush, dim=0, out=flush_out)   # evict k' and the KV chunks (untimed)
            ea.record()
            hils.attn_decode(dm, q, kcache, vcache, lens, kc, bc, o, ws, sel_idx=sel, kc_mirror=mirror)
            eb.record()
        torch.cuda.synchronize()
        per = [ea.elapsed_time(eb) * 1e3 for ea, eb in evs]
        stages = {s: 0.0 for s in hils.DECODE_STAGES}
        for _ in range(steps):
            torch.sum(flush, dim=0, out=flush_out)
            r = hils.attn_decode(dm, q, kcache, vcache, lens, kc, bc, o, ws, sel_idx=sel, timed=True,
                                 kc_mirror=mirror)
            for s_ in stages:
                stages[s_] += r[s_] / steps
        dist = {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                "p90": float(np.percentile(per, 90))}
        return float(np.mean(per)), stages, dist

    # the exact fp32 scan (hils_attn_decode), then the mirror scan (hils_attn_decode_mirror):
    # the same step, bit for bit
    us_f, stages_f, dist_f = timed_steps(None)
    sel_f, o_f = sel.clone(), o.clone()
    us, stages, dist = timed_steps(kcm)
    same = bool(torch.equal(sel, sel_f) and torch.equal(o.view(torch.int16), o_f.view(torch.int16)))
    log("decode, fp32 scan: %.1f us/step (stages ms %s)" % (us_f, stages_f))
    # algorithmic bytes per step: q, o; k' and b' of every candidate chunk; the K/V rows of
    # the union of selected chunks per (sequence, KV head) plus the local window (own chunk)
    seln = sel.cpu().numpy()
    G = wd.Hq // wd.Hkv
    nw = max(1, wd.window // wd.S)
    kv_bytes = 0
    for b in range(wd.B):
        L = int(x["seq_lens"][b])
        own = (L - 1) // wd.S
        for g in range(wd.Hkv):
            u = set(seln[b, g * G:(g + 1) * G].ravel().tolist()) - {-1}
            kv_bytes += (len(u) * wd.S + (L - own * wd.S) + min(nw - 1, own) * wd.S) * wd.d * 2 * 2
    Ps = [min(wd.C, max(0, (int(L) - 1) // wd.S - nw + 1)) for L in x["seq_lens"]]
    scan_bytes_f = sum(P * wd.Hlmk * (wd.d + 1) * 4 for P in Ps)          # fp32 k' and b'
    scan_bytes = sum(P * wd.Hlmk * (wd.d + 8) for P in Ps)   # mirror: 8-bit codes of k', fp32 b' and scale
    total_bytes = scan_bytes + kv_bytes + 2 * 2 * wd.B * wd.Hq * wd.d
    step_gbs = total_bytes / (us * 1e-6) / 1e9
    scan_gbs = scan_bytes / (stages["scan"] * 1e-3) / 1e9
    scan_gbs_f = scan_bytes_f / (stages_f["scan"] * 1e-3) / 1e9
    log("decode: %.1f us/step (stages ms %s), same result as the fp32 scan: %s" % (us, stages, same))
    dense_kv = sum(int(L) for L in x["seq_lens"]) * wd.Hkv * wd.d * 2 * 2
    dense_meas = None
    if dense and len(set(int(L) for L in x["seq_lens"])) == 1:
        own, o_own = dense_decode_own(dm, q, kcache, vcache, lens, flush, flush_out)
        own["hils_speedup"] = own["us"] / us
        own["achieved_GBs"] = dense_kv / (own["us"] * 1e-6) / 1e9
        own["frac"] = own["achieved_GBs"] / PEAK_HBM_GBS
        tq, o_t = dense_decode(q, kcache, vcache, int(x["seq_lens"][0]), flush, flush_out)
        tq["hils_speedup"] = tq["us"] / us
        own["max_abs_diff_vs_torch"] = float((o_own.float() - o_t.float().reshape(o_own.shape)).abs().max())
        dense_meas = {"own": own, "torch": tq}
        log("dense decode: own %.1f us (%.0f GB/s), torch %.1f us" % (own["us"], own["achieved_GBs"], tq["us"]))
    return {
        "workload": wd.name, "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "d": wd.d, "ctx": int(max(x["seq_lens"])),
        "K": wd.K, "window": wd.window, "us_per_step": us, "us_per_step_dist": dist,
        "stages_us": {k_: v_ * 1e3 for k_, v_ in stages.items()},
        "scan": "8-bit landmark mirror + exact fp32 rescoring (hils_attn_decode_mirror)",
        "one_off_compress_ms": comp_ms, "one_off_mirror_ms": mirror_ms,
        "roofline": {"bound": "hbm", "achieved": scan_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": scan_gbs / PEAK_HBM_GBS, "kernel": "decode_scan_m",
                     "traffic": measured_traffic("decode_scan_m", wd.name)},
        "step_hbm": {"algorithmic_bytes": total_bytes, "achieved_GBs": step_gbs, "frac": step_gbs / PEAK_HBM_GBS,
                     "kv_union_bytes": kv_bytes, "kprime_bytes": scan_bytes},
        "fp32_scan": {"us_per_step": us_f, "us_per_step_dist": dist_f,
                      "stages_us": {k_: v_ * 1e3 for k_, v_ in stages_f.items()},
                      "roofline": {"bound": "hbm", "achieved": scan_gbs_f, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": scan_gbs_f / PEAK_HBM_GBS, "kernel": "decode_scan",
                                   "traffic": measured_traffic("decode_scan", wd.name)},
                      "kprime_bytes": scan_bytes_f},
        "mirror_result_identical": same,
        "dense_kv_bytes": dense_kv, "dense_us_at_hbm_peak": dense_kv / (PEAK_HBM_GBS * 1e9) * 1e6,
        "dense_measured": dense_meas,
    }


def dense_decode(q, kcache, vcache, L, flush, flush_out, reps=5):
    """Dense attention of the decode queries over the whole cache (torch, bf16 GEMMs with fp32
    softmax): per KV head, S^T = K Q^T of its query heads, softmax over the L keys, O = P V.
    Timed per step after the same cache eviction as the sparse step."""
    import torch
    B, Hq, d = q.shape
    Hkv = kcache.shape[1]
    G = Hq // Hkv
    kk, vv = kcache[:, :, :L], vcache[:, :, :L]
    qt = q.view(B, Hkv, G, d).transpose(-1, -2).contiguous()          # [B, Hkv, d, G], a contiguous right operand
    tau = 1.0 / math.sqrt(d)

    def step():
        st = torch.matmul(kk, qt).float() * tau                      # [B, Hkv, L, G]
        p = torch.softmax(st, dim=2).to(torch.bfloat16).transpose(-1, -2).contiguous()   # [B, Hkv, G, L]
        return torch.matmul(p, vv)                                     # [B, Hkv, G, d]

    out = step()
    per = []
    for _ in range(reps):
        torch.sum(flush, dim=0, out=flush_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3)
    return ({"impl": "torch: bf16 matmuls K Q^T and P V with an fp32 softmax, per KV head", "us": float(np.median(per)),
             "us_p10": float(np.percentile(per, 10)), "us_p90": float(np.percentile(per, 90))}, out)


def dense_decode_own(dm, q, kcache, vcache, lens, flush, flush_out, reps=5):
    """hils_dense_decode over the whole cache (every key read once per KV group), timed per
    step after the same cache eviction as the sparse step."""
    import torch
    from long_context_chunk_amd import hils
    ws = hils.workspace(dm, hils.OP_DENSE_DECODE)
    o = torch.empty_like(q)
    hils.dense_decode(dm, q, kcache, vcache, lens, o, ws)
    per = []
    for _ in range(reps):
        torch.sum(flush, dim=0, out=flush_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        hils.dense_decode(dm, q, kcache, vcache, lens, o, ws)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3)
    return ({"impl": "hils_dense_decode (splits of 2048 keys, one K/V read per KV group, split merge)",
             "us": float(np.median(per)), "us_p10": float(np.percentile(per, 10)),
             "us_p90": float(np.percentile(per, 90))}, o)


def backward_flops(w, cnt):
    """Algorithmic MFMA work of the backward: per (row, selected chunk) pair and per window key,
    the five products S = q K^T, dP = g V^T, dq = dS K, dk = dS^T q, dv = P^T g (2 d flops each
    per (row, key)); the score, Q-Cal and compression gradients are small beside them."""
    pair_keys = cnt["pairs"] * w.S
    window_keys = cnt["window_flops"] / (4.0 * w.d)  # the forward's 4 d flops per (row, window key)
    return 10.0 * w.d * (pair_keys + window_keys)


def run_backward(w, steps, warmup, seed):
    """Times hils_attn_prefill_backward on the forward's own outputs (selection, k', o) with a
    seeded standard-normal output gradient."""
    import torch
    import synth
    from long_context_chunk_amd import hils
    x = synth.make_inputs(w, seed)
    dm = hils.dims(w.B, w.Hq, w.Hkv, w.d, w.N, w.K, S=w.S, qcal_rank=w.qcal_rank, io=w.io, window=w.window)
    q, k, v, lmk = (upload(x[n], w.io) for n in ("q", "k", "v", "lmk"))
    D = upload(x["D"], w.io) if w.qcal_rank else None
    U = upload(x["U"], w.io) if w.qcal_rank else None
    del x
    o = torch.empty_like(q)
    kc = torch.empty((w.B, w.Hlmk, w.C, w.d), dtype=torch.float32, device="cuda")
    bc = torch.empty((w.B, w.Hlmk, w.C), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.int32, device="cuda")
    scr = torch.empty((w.B, w.Hq, w.N, w.K), dtype=torch.float32, device="cuda")
    ws = hils.workspace(dm, hils.OP_PREFILL)
    hils.attn_prefill(dm, q, k, v, o, ws, lmk_q=lmk, kc=kc, bc=bc, qcal_D=D, qcal_U=U, sel_idx=sel, sel_score=scr)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 77)
    dO = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv, dlmk = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(lmk)
    dD = torch.empty_like(D) if D is not None else None
    dU = torch.empty_like(U) if U is not None else None
    wsb = hils.workspace(dm, hils.OP_BACKWARD)
    log("backward workspace %.1f GiB" % (wsb.numel() / 2**30))

    def step():
        hils.attn_prefill_backward(dm, q, k, v, lmk, kc, sel, scr, o, dO, dq, dk, dv, dlmk, wsb, qcal_D=D, qcal_U=U,
                                   dD=dD, dU=dU)

    ms = _time_ms(step, steps)  # one untimed call first
    cnt = prefill_counts(w)
    fl = backward_flops(w, cnt)
    ach = fl / (ms * 1e-3) / 1e12
    log("backward: %.2f ms/step" % ms)
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_flops": fl, "kernel": "whole backward"}}


def with_window(w, window):
    """The workload with a local window of `window` tokens (named apart from the plain one)."""
    import synth
    if window <= w.S:
        return w
    return synth.scaled(w, window=window, name="%s_w%d" % (w.name, window))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_256k_qcal")
    ap.add_argument("--decode-workload", default="decode_512k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--window", type=int, default=0,
                    help="local window in tokens (a multiple of 64; 0 = the own chunk only) for prefill and decode")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true", help="skip the 128K and 8K prefill lines")
    ap.add_argument("--no-prefill", action="store_true", help="decode step only (for profiling it alone)")
    ap.add_argument("--backward", action="store_true",
                    help="only the backward pass (gradients of the prefill output) at --workload")
    ap.add_argument("--sweep", action="store_true",
                    help="HiLS prefill against the dense baseline over N = 8K..512K (16/4 heads, d = 64, K = 16)")
    ap.add_argument("--peaks", action="store_true", help="only measure a device copy and a large bf16 GEMM")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 2 GiB device copy (counter calibration for the traffic figures)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the HiLS path here runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from long_context_chunk_amd import hils
    if args.copy_calibration:
        copy_calibration()
        return
    if args.peaks:
        run_peaks()
        return
    hils.load()
    if args.sweep:
        run_sweep(args)
        return
    hils.load()
    assert torch.cuda.is_available()
    w = with_window(synth.WORKLOADS[args.workload], args.window)
    seed = synth.BASE_SEED + 5
    if args.backward:
        print(json.dumps({"backward": run_backward(w, args.steps, args.warmup, seed)}), flush=True)
        return
    if args.no_prefill:
        wd = with_window(synth.WORKLOADS[args.decode_workload], args.window)
        print(json.dumps({"decode": run_decode(wd, max(args.steps, 20), args.warmup, seed + 1)}), flush=True)
        return
    res = run_prefill(w, args.steps, args.warmup, seed)
    cnt = prefill_counts(w)
    roof = stage_roofline(w, cnt, res["stages"])
    dom = max(roof, key=lambda s_: roof[s_]["ms"])
    total_flops = cnt["compress_flops"] + cnt["qcal_flops"] + cnt["score_flops"] + cnt["intra_flops"]
    whole = total_flops / (res["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    line = {
        "metric": METRIC,
        "value": w.B * w.N / (res["ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms"],
        "ms_per_step_dist": res["dist"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; planted-direction needle chunks and queries)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "seq_len": w.N, "S": w.S,
                   "K": w.K, "qcal_rank": w.qcal_rank, "window": w.window, "compression": "in the same call"},
        # the dominant (longest) kernel against its own bound: algorithmic MFMA flops for the
        # attention and scoring kernels; counter traffic (HBM bytes per launch) beside it
        "roofline": dict(roof[dom], kernel=dom, traffic=measured_traffic(dom, w.name), whole_step_frac=whole),
        "stages_ms": res["stages"],
        "stage_rooflines": roof,
        "algorithmic_tflops_per_step": total_flops / 1e12,
        "mfma_frac_whole_step": whole,
    }
    if not args.no_dense:
        try:
            dn = dense_baseline(res, w)
            dn["hils_speedup_vs_own_dense"] = dn["own"]["ms"] / res["ms"]
            if "torch_sdpa" in dn:
                dn["hils_speedup_vs_torch_sdpa"] = dn["torch_sdpa"]["ms"] / res["ms"]
            line["dense"] = dn
            log("dense: own %.1f ms, SDPA %.1f ms" % (dn["own"]["ms"], dn.get("torch_sdpa", {}).get("ms", -1)))
        except Exception as ex:  # report, never hide
            line["dense"] = {"error": repr(ex)}
    if not args.no_cpu:
        t0 = time.time()
        line["cpu_baseline"], line["sampled_parity"] = cpu_baseline(w, res)
        log("cpu baseline done in %.1fs; sampled parity %s" % (time.time() - t0, line["sampled_parity"]))
    else:
        line["cpu_baseline"] = None
    res.clear()
    torch.cuda.empty_cache()
    if not args.no_other_configs:
        line["other_configs"] = {}
        for name in ("prefill_128k", "prefill_8k"):
            wo = with_window(synth.WORKLOADS[name], args.window)
            r2 = run_prefill(wo, max(args.steps, 20), max(args.warmup, 2), seed)
            c2 = prefill_counts(wo)
            fl2 = c2["compress_flops"] + c2["qcal_flops"] + c2["score_flops"] + c2["intra_flops"]
            line["other_configs"][name] = {
                "tokens_per_s": wo.B * wo.N / (r2["ms"] * 1e-3), "ms_per_step": r2["ms"], "ms_per_step_dist": r2["dist"],
                "mfma_frac_whole_step": fl2 / (r2["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "stages_ms": r2["stages"],
                "config": {"B": wo.B, "Hq": wo.Hq, "Hkv": wo.Hkv, "d": wo.d, "seq_len": wo.N, "K": wo.K,
                           "qcal_rank": wo.qcal_rank, "window": wo.window}}
            r2.clear()
            torch.cuda.empty_cache()
    if not args.no_decode:
        wd = with_window(synth.WORKLOADS[args.decode_workload], args.window)
        line["decode"] = run_decode(wd, max(args.steps, 20), args.warmup, seed + 1, dense=not args.no_dense)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
