"""Benchmark of the qmm hot path on one MI355X.

One step = the single-token (N = 1) decode pass over Llama-3-8B-shaped projections
-- fused QKV 4096->6144, O 4096->4096, gate+up 4096->2x14336 with the SwiGLU
epilogue, down 14336->4096 (fed with the gate+up output), LM head 4096->128256 --
once with Q8_0 weights and once with Q4_0 weights.  Inputs are seeded synthetic
tensors resident in HBM before timing starts.  The step streams 1.21 GB of
weights, more than the 256 MB Infinity Cache, so every launch reads from HBM.

value = algorithmic bytes of one step (raw weight blocks + x + y) / step time, the
median of 7 trials of K steps each (the pages' own protocol: "alpaca.swift",
Results, median of 7 runs).

The same run also times, each as the median of 7 trials:
  * the single 576 x 576 Q8_0 GEMV with seed 0 (latency-bound; its 352 KB stay in
    the caches);
  * the prefill GEMM (fp16 activations, fp32 output) at 4096->14336 and
    14336->4096 for T in {128, 2048, 4096}, Q8_0 and Q4_0, with the weights rotated
    through copies totalling >= 512 MB so that every call streams them from HBM;
    TFLOP/s = 2 T M K / time;
  * a SmolLM2-135M-shaped decode step (30 layers + LM head), with its weights
    rotated through >= 512 MB of copies, and on one resident set (labelled);
  * small-batch decode (N in {1, 2, 4, 8, 16}), replayed as HIP graphs of rotated
    calls so that host launch overhead stays out;
  * the float64 CPU oracle per workload on bounded samples (unpack and matmul
    timed apart; reported baseline only).
Further sections (timing only): the decode step with the RMSNorm prologues and
residual epilogues fused in, expand-then-GEMM prefill against the fused GEMM,
the quantised embedding row gather, measured ceilings, and the decode step and
prefill route of the Q4_1 / Q5_0 / Q5_1 formats.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials 7] [--no-cpu] [--suite PATH]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--trials", type=int, default=7, help="timed trials per figure; the median is reported")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-smollm", action="store_true")
    p.add_argument("--no-small-batch", action="store_true")
    p.add_argument("--no-next", action="store_true",
                   help="skip the fused-norm/residual step, expand-then-GEMM, row gather and "
                        "Q4_1/Q5_0/Q5_1 sections")
    p.add_argument("--suite", default=None, help="write per-kernel details as JSON to this path")
    p.add_argument("--min-calls", type=int, default=200,
                   help="prefill: at least this many calls per trial (profiling runs pass a few)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (counter calibration)")
    return p.parse_args()


POOL_BYTES = 512 << 20          # rotation pool: 2 x the 256 MB Infinity Cache
# Outputs of the timed calls (copied to the host after timing), re-checked against the
# float64 oracle on sampled rows by the CPU-baseline leg: the single GEMV (all 576
# outputs), the decode step (the first rows of every launch) and every prefill case
# (the first PREFILL_CHECK_ROWS weight rows, all tokens).
TIMED_OUT = {}
PREFILL_CHECK_ROWS = 16
SB_CHECK_ROWS = 64
DECODE_CHECK_ROWS = 512
TOKEN_CHECK = 64  # tokens of the expansion sections' GEMM outputs re-checked


def median_trials(torch, body, trials, per):
    """Median over `trials` of (event time of one call of body()) / per, in ms; the
    device is synchronised before and after every trial."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(trials):
        torch.cuda.synchronize()
        e0.record()
        body()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / per)
    return float(np.median(ts)), ts


def graph_of(torch, body):
    """body() captured once into a HIP graph (on a side stream, as torch requires)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


class Timer:
    """HIP-event timing of individual launches on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, key, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(key, []).append((s, e))

    def ms(self, key):
        return [s.elapsed_time(e) for s, e in self.pairs.get(key, [])]


def decode_workload(torch, qmm, si):
    dev = torch.device("cuda")

    host = {}

    def W(fmt, M, K, seed):
        a = si.weights(fmt, M, K, seed)
        host[(fmt, seed)] = (a, M, K)
        return torch.from_numpy(a).to(dev)

    def X(n, K, seed):
        return torch.from_numpy(si.activations(n, K, seed)).to(dev)

    fmts = {}
    for fmt, base in ((si.FMT_Q8_0, 5000), (si.FMT_Q4_0, 6000)):
        fmts[fmt] = decode_tensors(torch, si, fmt, base, W, X)
    launches = []  # (kernel key, part, bytes, callable)
    for fmt, f in fmts.items():
        launches += decode_launches(qmm, si, fmt, f)
    return fmts, launches, host


def decode_tensors(torch, si, fmt, base, W, X):
    """Weights, input and outputs of the five 8B decode projections in one format."""
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    dev = torch.device("cuda")
    return dict(
        qkv=W(fmt, Q, H, base + 1), o=W(fmt, H, H, base + 2), g=W(fmt, I, H, base + 3),
        u=W(fmt, I, H, base + 4), d=W(fmt, H, I, base + 5), lm=W(fmt, V, H, base + 6),
        x=X(1, H, base + 7), x_host=si.activations(1, H, base + 7), y_qkv=torch.empty(Q, device=dev),
        y_o=torch.empty(H, device=dev), h=torch.empty(I, device=dev), y_d=torch.empty(H, device=dev),
        logits=torch.empty(V, device=dev))


def capture_decode(qmm, si, fmt, f, rows=DECODE_CHECK_ROWS):
    """Host copies for the oracle leg's re-check of a decode step: the outputs, x, and
    the first `rows` rows of every weight matrix (raw blocks, copied back from HBM)."""
    L = si.LLAMA3_8B
    H, I = L["hidden"], L["intermediate"]
    rec = {k: f[k].cpu().numpy() for k in ("y_qkv", "y_o", "h", "y_d", "logits")}
    rec["x"] = f["x"].cpu().numpy()
    rec["w"] = {k: f[k][:rows * qmm.qmm_row_bytes(fmt, I if k == "d" else H)].cpu().numpy()
                for k in ("qkv", "o", "g", "u", "d", "lm")}
    return rec


def decode_launches(qmm, si, fmt, f):
    """(kernel key, part, algorithmic bytes, callable) for each launch of the step."""
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    name = si.FMT_NAMES[fmt]

    def r(K):
        return qmm.qmm_row_bytes(fmt, K)
    launches = [
        (f"gemv_{name}", "qkv", Q * r(H) + 4 * H + 4 * Q,
         lambda f=f, fmt=fmt: qmm.qmm_gemv(fmt, f["qkv"], f["x"], f["y_qkv"], Q, H, 1)),
        (f"gemv_{name}", "o", H * r(H) + 4 * H + 4 * H,
         lambda f=f, fmt=fmt: qmm.qmm_gemv(fmt, f["o"], f["x"], f["y_o"], H, H, 1)),
        (f"gate_up_{name}", "gate_up", 2 * I * r(H) + 4 * H + 4 * I,
         lambda f=f, fmt=fmt: qmm.qmm_gate_up_silu(fmt, f["g"], f["u"], f["x"], f["h"], I, H, 1)),
        (f"gemv_{name}", "down", H * r(I) + 4 * I + 4 * H,
         lambda f=f, fmt=fmt: qmm.qmm_gemv(fmt, f["d"], f["h"], f["y_d"], H, I, 1)),
        (f"gemv_{name}", "lm_head", V * r(H) + 4 * H + 4 * V,
         lambda f=f, fmt=fmt: qmm.qmm_gemv(fmt, f["lm"], f["x"], f["logits"], V, H, 1)),
    ]
    return launches


def more_formats(torch, qmm, si, steps, reps=10):
    """Q4_1, Q5_0 and Q5_1 (the block formats beside Q8_0 / Q4_0): the same 8B decode
    step (per-launch and whole-step HBM rate of the raw blocks + x + y), and prefill
    at 14336 x 4096 with T = 128 and 2048: the fused GEMM, and fp16 expansion followed
    by the F16 GEMM (TFLOP/s = 2 T M K / time)."""
    dev = torch.device("cuda")

    def W(fmt, M, K, seed):
        return torch.from_numpy(si.weights(fmt, M, K, seed)).to(dev)

    def X(n, K, seed):
        return torch.from_numpy(si.activations(n, K, seed)).to(dev)

    out = {}
    for fmt, base in ((si.FMT_Q4_1, 7000), (si.FMT_Q5_0, 8000), (si.FMT_Q5_1, 9000)):
        f = decode_tensors(torch, si, fmt, base, W, X)
        launches = decode_launches(qmm, si, fmt, f)
        nbytes = float(sum(b for _, _, b, _ in launches))
        for _ in range(3):
            for _, _, _, fn in launches:
                fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            for _, _, _, fn in launches:
                fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        timer = Timer(torch)
        for _ in range(steps):
            for key, part, _, fn in launches:
                timer.run(part, fn)
        torch.cuda.synchronize()
        per = {}
        for _, part, b, _ in launches:
            us = 1e3 * float(np.mean(timer.ms(part)))
            per[part] = {"us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1), "bytes": int(b)}
        TIMED_OUT[("decode", fmt)] = capture_decode(qmm, si, fmt, f)
        res = {"step_us": round(ms * 1e3, 2), "step_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "step_bytes": int(nbytes), "launches": per}
        M, K = 14336, 4096
        W16 = torch.empty((M, K), dtype=torch.float16, device=dev)

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms_e = timed(lambda: qmm.qmm_expand_f16(fmt, f["g"], W16, M, K))
        rb = qmm.qmm_row_bytes(fmt, K)
        pf = {"M": M, "K": K, "expand_us": round(ms_e * 1e3, 2),
              "expand_GBps": round((M * rb + 2 * M * K) / (ms_e * 1e-3) / 1e9, 1), "T": []}
        for T in (128, 2048):
            Xh = torch.randn(T, K, device=dev).half()
            Y = torch.empty((T, M), device=dev)
            fl = 2.0 * T * M * K
            ms_f = timed(lambda: qmm.qmm_gemm(fmt, f["g"], Xh, Y, M, K, T))
            ms_x = timed(lambda: (qmm.qmm_expand_f16(fmt, f["g"], W16, M, K), qmm.qmm_gemm(1, W16, Xh, Y, M, K, T)))
            pf["T"].append({"T": T, "fused_TFLOPs": round(fl / (ms_f * 1e-3) / 1e12, 1),
                            "expand_then_gemm_TFLOPs": round(fl / (ms_x * 1e-3) / 1e12, 1)})
            capture_expand(("expand", fmt, M, K, T), fmt, f["g"], W16, Xh, Y, rb)
            del Xh, Y
        res["prefill"] = pf
        out[si.FMT_NAMES[fmt]] = res
        del f, launches, W16
        torch.cuda.empty_cache()
    return out


def config1(torch, qmm, si, trials, calls=400):
    """The single Q8_0 GEMV 576 x 576 (W seed 0, x seed 1), N = 1: time per call as
    back-to-back launches and as a replayed graph of `calls` launches.  Its 352 KB
    of weights stay in the caches between calls: the figure is the launch-and-latency
    time of one small GEMV, not an HBM rate."""
    dev = torch.device("cuda")
    M = K = 576
    W = torch.from_numpy(si.weights(si.FMT_Q8_0, M, K, 0)).to(dev)
    x = torch.from_numpy(si.activations(1, K, 1)).to(dev)
    y = torch.empty(M, device=dev)
    nbytes = M * qmm.qmm_row_bytes(si.FMT_Q8_0, K) + 4 * K + 4 * M

    def body():
        for _ in range(calls):
            qmm.qmm_gemv(si.FMT_Q8_0, W, x, y, M, K, 1)

    body()
    eager_ms, _ = median_trials(torch, body, trials, calls)
    g = graph_of(torch, body)
    g.replay()
    graph_ms, _ = median_trials(torch, g.replay, trials, calls)
    del g
    TIMED_OUT["single_gemv_576"] = y.cpu().numpy()
    return {"workload": "Q8_0 GEMV 576x576, N=1, W seed 0, x seed 1 (cache-resident, latency-bound)",
            "us_per_call_eager": round(eager_ms * 1e3, 3), "us_per_call_graph": round(graph_ms * 1e3, 3),
            "tok_s_graph": round(1e3 / graph_ms, 1), "GBps_graph": round(nbytes / (graph_ms * 1e-3) / 1e9, 1),
            "bytes": int(nbytes), "calls_per_trial": calls, "trials": trials}


def rotation_pool(torch, make, nbytes):
    """Enough copies (from make(i)) that together they exceed POOL_BYTES."""
    copies = max(1, -(-POOL_BYTES // nbytes))
    return [make(i) for i in range(copies)]


def prefill(torch, qmm, si, trials, min_calls=200):
    """Prefill GEMM cases, weights rotated through >= 512 MB of copies (one call per
    copy in turn), >= min_calls calls and >= 2 ms per trial; median of the trials."""
    dev = torch.device("cuda")
    details = []
    tot_f, tot_ms = 0.0, 0.0
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0):
        for (M, K) in ((14336, 4096), (4096, 14336)):
            base = torch.from_numpy(si.weights(fmt, M, K, 7000 + M % 101 + fmt)).to(dev)
            pool = rotation_pool(torch, lambda i: base.clone(), base.numel())
            for T in (128, 2048, 4096):
                Xt = torch.from_numpy(si.activations(T, K, 7100 + T, dtype=np.float16)).to(dev)
                Yt = torch.empty((T, M), device=dev)
                ws = torch.empty(max(1, qmm.qmm_workspace_size(qmm.QMM_OP_GEMM, fmt, M, K, T)), dtype=torch.uint8,
                                 device=dev)

                def call(i):
                    qmm.qmm_gemm(fmt, pool[i % len(pool)], Xt, Yt, M, K, T, ws)
                for i in range(3):
                    call(i)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call(0)
                e1.record()
                torch.cuda.synchronize()
                calls = min_calls
                if min_calls >= 200:  # timing runs: also >= 2 ms per trial
                    calls = max(calls, int(2.0 / max(e0.elapsed_time(e1), 1e-3)) + 1)

                def body():
                    for i in range(calls):
                        call(i)
                ms, _ = median_trials(torch, body, trials, calls)
                TIMED_OUT[("prefill", fmt, M, K, T)] = Yt[:, :PREFILL_CHECK_ROWS].cpu().numpy()
                fl = 2.0 * T * M * K
                tot_f += fl
                tot_ms += ms
                details.append({"fmt": si.FMT_NAMES[fmt], "M": M, "K": K, "T": T, "us": round(ms * 1e3, 2),
                                "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1),
                                "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                                "copies": len(pool), "calls_per_trial": calls})
                del Xt, Yt, ws
            del pool, base
            torch.cuda.empty_cache()
    tflops = tot_f / (tot_ms * 1e-3) / 1e12
    return {"value": round(tflops, 1), "unit": "TFLOP/s", "peak": FP16_MFMA_PEAK_TFLOPS,
            "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
            "workload": "Q8_0+Q4_0 x {4096->14336, 14336->4096} x T in {128,2048,4096}, fp16 X, fp32 Y; "
                        "weights rotated through >= 512 MB of copies; median of trials",
            "cases": details}


def cpu_baseline(host, si, trials, rows=512):
    """The float64 oracle on the host cores, per workload, on bounded samples (about
    20-30 s of CPU work); each figure is the median of `trials` runs, with the unpack
    (raw blocks -> float64 weights) and the matmul (numpy BLAS on all threads) timed
    apart.  A reported baseline, never a target.
      * single 576 x 576 Q8_0 GEMV (seed 0): whole;
      * Llama-3-8B decode GEMVs, Q8_0 and Q4_0: the first `rows` rows of each of the
        step's matrices (the very bytes the GPU streamed), scaled to whole matrices;
      * SmolLM2-135M decode step: one layer and 1024 LM-head rows, scaled to 30 layers
        and 49152 rows;
      * small-batch GEMV, 16 tokens, on the sampled O rows (F16, Q8_0, Q4_0);
      * prefill GEMM, T in {128, 2048, 4096}, on the sampled rows of 14336 x 4096.
    """
    import oracle

    def timed(fn):
        ts, r = [], None
        for _ in range(trials):
            t0 = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), r

    L, S = si.LLAMA3_8B, si.SMOLLM2_135M
    out = {}
    # single GEMV
    raw = si.weights(si.FMT_Q8_0, 576, 576, 0)
    x = si.activations(1, 576, 1).astype(np.float64)
    tu, W = timed(lambda: oracle.dequant(si.FMT_Q8_0, raw, 576, 576))
    tm, _ = timed(lambda: x @ W.T)
    out["single_q8_0_gemv_576"] = {"unpack_ms": round(tu * 1e3, 3), "matmul_ms": round(tm * 1e3, 4),
                                   "tok_s": round(1.0 / (tu + tm), 1),
                                   "GBps": round(raw.size / (tu + tm) / 1e9, 4)}
    # 8B decode GEMVs (sampled rows)
    step_bytes, step_t, samp_bytes, samp_t = 0.0, 0.0, 0.0, 0.0
    per_fmt = {}
    o_rows = {}
    for (fmt, seed), (a, M, K) in host.items():
        rb = oracle.row_bytes(fmt, K)
        part = a[:rows * rb]
        xs = si.activations(1, K, 4321).astype(np.float64)
        tu, W = timed(lambda: oracle.dequant(fmt, part, rows, K))
        tm, _ = timed(lambda: xs @ W.T)
        pf = per_fmt.setdefault(si.FMT_NAMES[fmt], {"unpack_s": 0.0, "matmul_s": 0.0, "bytes": 0})
        pf["unpack_s"] += tu * M / rows
        pf["matmul_s"] += tm * M / rows
        pf["bytes"] += M * rb
        samp_bytes += part.size
        samp_t += tu + tm
        step_bytes += M * rb
        step_t += (tu + tm) * M / rows
        if M == L["hidden"] and K == L["hidden"]:
            o_rows[fmt] = (part, W)
        if M == L["intermediate"] and K == L["hidden"] and "prefill" not in out:
            out["prefill"] = {"fmt": si.FMT_NAMES[fmt], "rows": rows, "K": K, "cases": []}
            for T in (128, 2048, 4096):
                X = si.activations(T, K, 7100 + T, dtype=np.float16).astype(np.float64)
                tp, _ = timed(lambda: X @ W.T)
                out["prefill"]["cases"].append({"T": T, "matmul_s": round(tp, 4),
                                                "TFLOPs": round(2.0 * T * rows * K / tp / 1e12, 5)})
            out["prefill"]["unpack_s_per_row"] = round(tu / rows, 6)
    for v in per_fmt.values():
        v["GBps"] = round(v["bytes"] / (v["unpack_s"] + v["matmul_s"]) / 1e9, 4)
        v["tok_s"] = round(1.0 / (v["unpack_s"] + v["matmul_s"]), 4)
        v["unpack_s"], v["matmul_s"] = round(v["unpack_s"], 2), round(v["matmul_s"], 3)
    out["llama3_8b_decode_step"] = {"per_format": per_fmt, "step_s_extrapolated": round(step_t, 1),
                                    "GBps": round(step_bytes / step_t / 1e9, 4), "rows_sampled": rows}
    # small batch, 16 tokens, on the sampled O rows
    sb = {}
    X16 = si.activations(16, L["hidden"], 4322).astype(np.float64)
    for fmt, (part, W) in o_rows.items():
        tm, _ = timed(lambda: X16 @ W.T)
        sb[si.FMT_NAMES[fmt]] = {"matmul_ms_16_tokens": round(tm * 1e3, 3), "rows": rows}
    f16 = si.weights(si.FMT_F16, rows, L["hidden"], 4323)
    tu, W = timed(lambda: oracle.dequant(si.FMT_F16, f16, rows, L["hidden"]))
    tm, _ = timed(lambda: X16 @ W.T)
    sb["F16"] = {"unpack_ms": round(tu * 1e3, 3), "matmul_ms_16_tokens": round(tm * 1e3, 3), "rows": rows}
    out["small_batch_16"] = sb
    # SmolLM2-135M step: one layer + 1024 LM-head rows, scaled
    H, I, V, Q = S["hidden"], S["intermediate"], S["vocab"], si.qkv_rows(S)
    sm = {}
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0):
        mats = [(si.weights(fmt, m, k, 8000 + i), m, k) for i, (m, k) in
                enumerate(((Q, H), (H, H), (I, H), (I, H), (H, I), (1024, H)))]
        lay_t, lm_t = 0.0, 0.0
        for j, (a, m, k) in enumerate(mats):
            xs = si.activations(1, k, 77).astype(np.float64)
            tu, W = timed(lambda: oracle.dequant(fmt, a, m, k))
            tm, _ = timed(lambda: xs @ W.T)
            if j < 5:
                lay_t += tu + tm
            else:
                lm_t += (tu + tm) * V / 1024
        step = S["layers"] * lay_t + lm_t
        sm[si.FMT_NAMES[fmt]] = {"step_s_extrapolated": round(step, 3), "tok_s": round(1.0 / step, 3)}
    out["smollm2_135m_decode_step"] = sm
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(samp_bytes / samp_t / 1e9, 5), "unit": "GB/s", "cores": min(cores, threads),
            "kind": "oracle", "cpu_model": model, "trials": trials,
            "parity_of_timed_outputs": timed_parity(oracle, si),
            "sample": f"first {rows} rows of each of the 12 weight matrices of the Llama-3-8B decode step "
                      f"(Q8_0 and Q4_0), float64 numpy unpack + BLAS matmul, median of {trials} runs; "
                      f"per-workload figures in configs",
            "configs": out}


def timed_parity(oracle, si):
    """The timed calls' outputs against the float64 oracle, on the same inputs (the
    weights' first rows and x copied back from the device where the section drew them
    at random): the single 576 x 576 GEMV whole; the first DECODE_CHECK_ROWS rows of
    every 8B decode launch in every block format (down from the GPU's own h, the input
    it consumed), and of the fused step (norm prologues; the two residual adds of one
    call, from the residual before it); the SmolLM2-135M step's last layer and LM head;
    the first SB_CHECK_ROWS rows of every small-batch call; the first PREFILL_CHECK_ROWS
    weight rows of every prefill case over all tokens and, for the expand-then-GEMM
    cases, over the first TOKEN_CHECK tokens, with the fp16 expansion compared bit for
    bit; the first 16 gathered rows of every row gather, bit for bit (NaN where the
    random scale bytes make one); and the first DECODE_CHECK_ROWS rows of every launch
    of the 8-way tensor-parallel shard step (down and gate+up from the GPU's own h).  Each output's error is divided by its bound (2e-3 S
    + 1e-6; the SwiGLU and residual bounds where they apply): every ratio must be <= 1."""
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    worst, n, fails = 0.0, 0, []

    def take(name, got, ref, tol):
        nonlocal worst, n
        r = float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref) / tol))
        n += int(np.size(ref))
        worst = max(worst, r)
        if not r <= 1.0:
            fails.append(name)

    def exact(name, got, ref):
        nonlocal n
        n += int(np.size(ref))
        if not np.array_equal(np.asarray(got), np.asarray(ref), equal_nan=True):
            fails.append(name)

    if "single_gemv_576" in TIMED_OUT:
        raw = si.weights(si.FMT_Q8_0, 576, 576, 0)
        y, S = oracle.matmul_ref(si.FMT_Q8_0, raw, si.activations(1, 576, 1), 576, 576)
        take("single_gemv_576", TIMED_OUT["single_gemv_576"], y[0], oracle.tol_linear(S[0]))
    R = DECODE_CHECK_ROWS
    for key, rec in TIMED_OUT.items():
        if not (isinstance(key, tuple) and key[0] in ("decode", "fused")):
            continue
        kind, fmt = key
        name = f"{kind} {si.FMT_NAMES[fmt]}"
        w, x = rec["w"], rec["x"]
        if kind == "decode":
            for part, M, K, wk, yk, xin in (("qkv", Q, H, "qkv", "y_qkv", x), ("o", H, H, "o", "y_o", x),
                                            ("down", H, I, "d", "y_d", rec["h"]), ("lm_head", V, H, "lm", "logits", x)):
                y, S = oracle.matmul_ref(fmt, w[wk], xin, R, K)
                take(f"{name} {part}", rec[yk][:R], y[0], oracle.tol_linear(S[0]))
            h, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, w["g"], w["u"], x, R, H)
            take(f"{name} gate_up", rec["h"][:R], h[0], oracle.tol_swiglu(g[0], u[0], Sg[0], Su[0]))
        else:
            gm, eps = rec["gamma"], rec["eps"]
            for part, M, wk, yk in (("norm qkv", Q, "qkv", "y_qkv"), ("norm lm_head", V, "lm", "logits")):
                y, S = oracle.rmsnorm_matmul_ref(fmt, w[wk], x, gm, eps, R, H)
                take(f"{name} {part}", rec[yk][:R], y[0], oracle.tol_linear(S[0]))
            h, g, u, Sg, Su = oracle.rmsnorm_gate_up_silu_ref(fmt, w["g"], w["u"], x, gm, eps, R, H)
            take(f"{name} norm gate_up", rec["h"][:R], h[0], oracle.tol_swiglu(g[0], u[0], Sg[0], Su[0]))
            # r2 = (r0 + O x) + D h: both adds, each within its residual bound.
            r1, S1 = oracle.matmul_add_ref(fmt, w["o"], x, np.reshape(rec["r0"], -1)[:R], R, H)
            r2, S2 = oracle.matmul_add_ref(fmt, w["d"], rec["h"], r1[0], R, I)
            take(f"{name} O + down residual", np.reshape(rec["r2"], -1)[:R], r2[0],
                 oracle.tol_residual(S1[0], r1[0]) + oracle.tol_residual(S2[0], r2[0]))
    Sm = si.SMOLLM2_135M
    sH, sI, sV, sQ = Sm["hidden"], Sm["intermediate"], Sm["vocab"], si.qkv_rows(Sm)
    sel = np.arange(R)
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0):
        out = TIMED_OUT.get(("smollm2", fmt))
        if out is None:
            continue
        name, base = si.FMT_NAMES[fmt], out["base"]
        s0 = base + 10 * (Sm["layers"] - 1)
        x = si.activations(1, sH, base + 998)
        for part, i, M, K, key, xin in (("qkv", 0, sQ, sH, "y_qkv", x), ("o", 1, sH, sH, "y_o", x),
                                        ("down", 4, sH, sI, "y_d", out["h"])):
            y, S = oracle.matmul_ref(fmt, si.weights(fmt, M, K, s0 + i), xin, M, K)
            take(f"smollm2 {name} {part}", out[key], y[0], oracle.tol_linear(S[0]))
        h, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, si.weights(fmt, sI, sH, s0 + 2), si.weights(fmt, sI, sH, s0 + 3),
                                                  x, sI, sH)
        take(f"smollm2 {name} gate_up", out["h"], h[0], oracle.tol_swiglu(g[0], u[0], Sg[0], Su[0]))
        y, S = oracle.matmul_ref(fmt, si.weights(fmt, sV, sH, base + 999), x, sV, sH, rows=sel)
        take(f"smollm2 {name} lm_head", out["logits"][sel], y[0], oracle.tol_linear(S[0]))
    for key, rec in TIMED_OUT.items():
        if not isinstance(key, tuple):
            continue
        if key[0] == "small_batch":
            _, fmt, sname = key
            K = rec["K"]
            for (nt, v), got in rec["y"].items():
                xs = rec["x"][:nt * K].reshape(nt, K)
                label = f"small batch {si.FMT_NAMES[fmt]} {sname} N={nt} {v}"
                if sname == "gate_up":
                    h, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, rec["w"][0], rec["w"][1], xs, SB_CHECK_ROWS, K)
                    take(label, got, h, oracle.tol_swiglu(g, u, Sg, Su))
                else:
                    y, S = oracle.matmul_ref(fmt, rec["w"][0], xs, SB_CHECK_ROWS, K)
                    take(label, got, y, oracle.tol_linear(S))
        elif key[0] == "prefill":
            _, fmt, M, K, T = key
            raw = si.weights(fmt, M, K, 7000 + M % 101 + fmt)
            X = si.activations(T, K, 7100 + T, dtype=np.float16)
            y, S = oracle.matmul_ref(fmt, raw, X, M, K, rows=np.arange(PREFILL_CHECK_ROWS))
            take(f"prefill {si.FMT_NAMES[fmt]} {M}x{K} T={T}", rec, y, oracle.tol_linear(S))
        elif key[0] == "expand":
            _, fmt, M, K, T = key
            label = f"expand {si.FMT_NAMES[fmt]} {M}x{K} T={T}"
            exact(label + " fp16 weights",
                  rec["w16"].view(np.uint16), oracle.expand_f16_ref(fmt, rec["w"], PREFILL_CHECK_ROWS, K).view(np.uint16))
            y, S = oracle.matmul_ref(fmt, rec["w"], rec["x"], PREFILL_CHECK_ROWS, K)
            take(label + " GEMM", rec["y"], y, oracle.tol_linear(S))
        elif key[0] == "tp8":
            _, fmt = key
            name = f"tp8 shard {si.FMT_NAMES[fmt]}"
            dims, w = rec["dims"], rec["w"]
            for part, wk, xin in (("qkv", "qkv", rec["x"]), ("o", "o", rec["xo"]), ("down", "d", rec["h"]),
                                  ("lm_head", "lm", rec["x"])):
                M, K = dims[part]
                R = min(M, DECODE_CHECK_ROWS)
                y, S = oracle.matmul_ref(fmt, w[wk], xin, R, K)
                take(f"{name} {part}", np.reshape(rec["y"][part], -1)[:R], y[0], oracle.tol_linear(S[0]))
            I8, H8 = dims["gate_up"]
            R = min(I8, DECODE_CHECK_ROWS)
            hr, g, u, Sg, Su = oracle.gate_up_silu_ref(fmt, w["g"], w["u"], rec["x"], R, H8)
            take(f"{name} gate_up", np.reshape(rec["h"], -1)[:R], hr[0], oracle.tol_swiglu(g[0], u[0], Sg[0], Su[0]))
        elif key[0] == "get_rows":
            _, fmt, nr = key
            m = rec["out"].shape[0]  # 16 gathered rows, or every row of a smaller gather
            with np.errstate(invalid="ignore"):  # NaN rows (random scale bytes) stay NaN in float32
                ref = oracle.get_rows_ref(fmt, rec["w"], m, rec["K"], np.arange(m)).astype(np.float32)
            exact(f"get_rows {si.FMT_NAMES[fmt]} n={nr}", rec["out"], ref)
    if fails:
        print(f"bench: timed outputs outside the oracle bound: {', '.join(fails)}", file=sys.stderr, flush=True)
    return {"outputs_checked": n, "max_err_over_bound": round(worst, 4), "ok": not fails,
            "what": "single 576x576 GEMV whole; the first rows of every 8B decode launch (Q8_0, Q4_0, Q4_1, Q5_0, "
                    "Q5_1) and of the fused step; the SmolLM2-135M step's last layer and LM-head rows; the first "
                    "rows of every small-batch call; the first rows of every prefill and expand-then-GEMM case "
                    "(the expansion bit for bit); the first 16 rows of every row gather, bit for bit; the first rows of "
                    "every launch of the 8-way tensor-parallel shard step"}


def smollm2_step(torch, qmm, si, steps, trials):
    """SmolLM2-135M-shaped decode step (30 layers + LM head), Q8_0 and Q4_0: one step
    per weight set, the sets rotated through >= 512 MB (4 sets of Q8_0, 8 of Q4_0) so
    that each step streams its weights from HBM, eager and as replayed graphs (one per
    set); and on a single resident set (its 76-143 MB stay in the Infinity Cache
    between steps, as in a serving loop of this model alone).  tok/s = 1 / step time."""
    S = si.SMOLLM2_135M
    H, I, V, Q = S["hidden"], S["intermediate"], S["vocab"], si.qkv_rows(S)
    dev = torch.device("cuda")
    out = {}
    for fmt, base in ((si.FMT_Q8_0, 8000), (si.FMT_Q4_0, 8500)):
        layers = []
        for layer in range(S["layers"]):
            s0 = base + 10 * layer
            layers.append([torch.from_numpy(si.weights(fmt, m, k, s0 + i)).to(dev)
                           for i, (m, k) in enumerate(((Q, H), (H, H), (I, H), (I, H), (H, I)))])
        lm = torch.from_numpy(si.weights(fmt, V, H, base + 999)).to(dev)
        nbytes = sum(w.numel() for ws in layers for w in ws) + lm.numel()
        sets = [(layers, lm)] + [([[w.clone() for w in ws] for ws in layers], lm.clone())
                                 for _ in range(max(1, -(-POOL_BYTES // nbytes)) - 1)]
        x = torch.from_numpy(si.activations(1, H, base + 998)).to(dev)
        yq, yo, h, yd, logits = (torch.empty(n, device=dev) for n in (Q, H, I, H, V))

        def step(ws):
            lys, head = ws
            for (wq, wo, wg, wu, wd) in lys:
                qmm.qmm_gemv(fmt, wq, x, yq, Q, H, 1)
                qmm.qmm_gemv(fmt, wo, x, yo, H, H, 1)
                qmm.qmm_gate_up_silu(fmt, wg, wu, x, h, I, H, 1)
                qmm.qmm_gemv(fmt, wd, h, yd, H, I, 1)
            qmm.qmm_gemv(fmt, head, x, logits, V, H, 1)

        n = len(sets) * max(1, steps // len(sets))
        for ws in sets:
            step(ws)

        def rotated():
            for i in range(n):
                step(sets[i % len(sets)])

        def resident():
            for _ in range(n):
                step(sets[0])
        eager_ms, _ = median_trials(torch, rotated, trials, n)
        eager_res_ms, _ = median_trials(torch, resident, trials, n)
        graphs = [graph_of(torch, lambda ws=ws: step(ws)) for ws in sets]

        def g_rotated():
            for i in range(n):
                graphs[i % len(graphs)].replay()

        def g_resident():
            for _ in range(n):
                graphs[0].replay()
        graph_ms, _ = median_trials(torch, g_rotated, trials, n)
        graph_res_ms, _ = median_trials(torch, g_resident, trials, n)
        # The last replays ran set 0: its last layer's outputs and the head's logits.
        TIMED_OUT[("smollm2", fmt)] = {"base": base, "y_qkv": yq.cpu().numpy(), "y_o": yo.cpu().numpy(),
                                       "h": h.cpu().numpy(), "y_d": yd.cpu().numpy(), "logits": logits.cpu().numpy()}
        del graphs, sets
        torch.cuda.empty_cache()
        out[si.FMT_NAMES[fmt]] = {
            "weight_bytes": int(nbytes), "sets_rotated": max(1, -(-POOL_BYTES // nbytes)),
            "hbm": {"eager_tok_s": round(1e3 / eager_ms, 1), "graph_tok_s": round(1e3 / graph_ms, 1),
                    "graph_GBps": round(nbytes / (graph_ms * 1e-3) / 1e9, 1)},
            "cache_resident": {"eager_tok_s": round(1e3 / eager_res_ms, 1),
                               "graph_tok_s": round(1e3 / graph_res_ms, 1)}}
    return out


def small_batch(torch, qmm, si, trials, reps=20):
    """Decode GEMV at N in {1,2,4,8,16} on the Llama-3-8B shapes, F16 / Q8_0 / Q4_0.

    Each (format, shape) rotates through weight copies totalling >= 512 MB, so every
    call streams from HBM rather than the 256 MB Infinity Cache (the weights are random
    bytes with finite scales; the first rows of the last call's weights, x and the
    outputs are copied back for the oracle leg's re-check).  `reps` rotated calls are
    captured as one HIP graph with a preallocated workspace and replayed (the median
    of the trials), so host launch overhead stays out.  Reports weight GB/s of the
    VALU streaming path, of the MFMA path, and of qmm_gemv's own choice, per N, and
    the smallest N at which the MFMA path is faster (the crossover).
    """
    L = si.LLAMA3_8B
    H, I, Q = L["hidden"], L["intermediate"], si.qkv_rows(L)
    shapes = [("qkv", Q, H), ("o", H, H), ("gate_up", I, H), ("down", H, I)]
    dev = torch.device("cuda")
    Ns = (1, 2, 4, 8, 16)
    x = torch.randn(16 * I, device=dev)
    y = torch.empty(16 * I, device=dev)
    out = {}
    for fmt in (si.FMT_F16, si.FMT_Q8_0, si.FMT_Q4_0):
        name = si.FMT_NAMES[fmt]
        res = {v: {n: [0.0, 0.0] for n in Ns} for v in ("valu", "mfma", "auto")}  # bytes, ms
        for sname, M, K in shapes:
            n_mats = 2 if sname == "gate_up" else 1
            op = qmm.QMM_OP_GATE_UP_SILU if sname == "gate_up" else qmm.QMM_OP_GEMV
            nbytes = n_mats * M * qmm.qmm_row_bytes(fmt, K)
            copies = max(1, -(-POOL_BYTES // nbytes))
            pool = [[torch.randint(0, 256, (M * qmm.qmm_row_bytes(fmt, K),), dtype=torch.uint8, device=dev)
                     for _ in range(n_mats)] for _ in range(copies)]
            for w in pool:  # random bytes: clear the scales' top exponent bit (no inf / NaN)
                for m in w:
                    if fmt != si.FMT_F16:
                        bb = qmm.qmm_row_bytes(fmt, 32)
                        m.view(-1, bb)[:, 1] &= 0x3B
                    else:
                        m.view(-1, 2)[:, 1] &= 0x3B
            last = pool[(reps - 1) % copies]  # the weights of the last call of every replay
            sb_key = ("small_batch", fmt, sname)
            TIMED_OUT[sb_key] = {"M": M, "K": K, "x": x[:16 * K].cpu().numpy(),
                                 "w": [m[:SB_CHECK_ROWS * qmm.qmm_row_bytes(fmt, K)].cpu().numpy() for m in last],
                                 "y": {}}
            wsb = max(qmm.qmm_workspace_size(op, fmt, M, K, n, v) for n in Ns for v in (0, 1, 2))
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            for n in Ns:
                for v, code in (("valu", 1), ("mfma", 2), ("auto", 0)):
                    def call(i, n=n, code=code):
                        w = pool[i % copies]
                        if sname == "gate_up":
                            qmm.qmm_gate_up_silu_variant(fmt, w[0], w[1], x, y, M, K, n, code, ws)
                        else:
                            qmm.qmm_gemv_variant(fmt, w[0], x, y, M, K, n, code, ws)
                    for i in range(3):
                        call(i)

                    def body():
                        for i in range(reps):
                            call(i)
                    g = graph_of(torch, body)
                    g.replay()
                    ms, _ = median_trials(torch, g.replay, trials, reps)
                    del g
                    TIMED_OUT[sb_key]["y"][(n, v)] = y[:n * M].view(n, M)[:, :SB_CHECK_ROWS].cpu().numpy()
                    res[v][n][0] += nbytes
                    res[v][n][1] += ms
            del pool, ws
            torch.cuda.empty_cache()
        gbs = {v: {n: round(b / (ms * 1e-3) / 1e9, 1) for n, (b, ms) in d.items()} for v, d in res.items()}
        cross = next((n for n in Ns if gbs["mfma"][n] > gbs["valu"][n]), None)
        out[name] = {"weight_GBps": gbs, "mfma_faster_from_N": cross}
    return out


def fused_decode(torch, qmm, si, fmts, steps):
    """The decode step with the neighbouring steps fused in: attention norm + QKV,
    O + residual, FFN norm + gate+up+SwiGLU, down + residual, final norm + LM head,
    on the same weights as the plain step.  Bytes add gamma (4 K per norm) and the
    residual read (4 M per add) to the plain step's."""
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    dev = torch.device("cuda")
    gamma = torch.from_numpy((1.0 + 0.1 * si.activations(1, H, 4242)[0]).astype(np.float32)).to(dev)
    resid = torch.from_numpy(si.activations(1, H, 4243)).to(dev)
    eps = 1e-5
    out = {}
    for fmt, f in fmts.items():
        r = lambda K: qmm.qmm_row_bytes(fmt, K)
        plain_bytes = (Q * r(H) + 4 * H + 4 * Q) + (H * r(H) + 8 * H) + (2 * I * r(H) + 4 * H + 4 * I) + \
                      (H * r(I) + 4 * I + 4 * H) + (V * r(H) + 4 * H + 4 * V)
        fused_bytes = plain_bytes + 3 * 4 * H + 2 * 4 * H

        def plain(f=f):
            qmm.qmm_gemv(fmt, f["qkv"], f["x"], f["y_qkv"], Q, H, 1)
            qmm.qmm_gemv(fmt, f["o"], f["x"], f["y_o"], H, H, 1)
            qmm.qmm_gate_up_silu(fmt, f["g"], f["u"], f["x"], f["h"], I, H, 1)
            qmm.qmm_gemv(fmt, f["d"], f["h"], f["y_d"], H, I, 1)
            qmm.qmm_gemv(fmt, f["lm"], f["x"], f["logits"], V, H, 1)

        def fused(f=f):
            qmm.qmm_rmsnorm_gemv(fmt, f["qkv"], f["x"], gamma, eps, f["y_qkv"], Q, H, 1)
            qmm.qmm_gemv_add(fmt, f["o"], f["x"], resid, resid, H, H, 1)
            qmm.qmm_rmsnorm_gate_up_silu(fmt, f["g"], f["u"], f["x"], gamma, eps, f["h"], I, H, 1)
            qmm.qmm_gemv_add(fmt, f["d"], f["h"], resid, resid, H, I, 1)
            qmm.qmm_rmsnorm_gemv(fmt, f["lm"], f["x"], gamma, eps, f["logits"], V, H, 1)

        res = {}
        for name, fn, nb in (("plain", plain, plain_bytes), ("fused", fused, fused_bytes)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            res[name] = {"us": round(ms * 1e3, 2), "GBps": round(nb / (ms * 1e-3) / 1e9, 1), "bytes": int(nb)}
        res["fused_over_plain_time"] = round(res["fused"]["us"] / res["plain"]["us"], 4)
        out[si.FMT_NAMES[fmt]] = res
        r0 = resid.cpu().numpy()
        fused()
        rec = capture_decode(qmm, si, fmt, f)
        rec.update(r0=r0, r2=resid.cpu().numpy(), gamma=gamma.cpu().numpy(), eps=eps)
        TIMED_OUT[("fused", fmt)] = rec
    return out


def tp8_shard_decode(torch, qmm, si, trials, reps=20):
    """One GPU's share of the 8B decode step under 8-way tensor parallelism, Q8_0 and
    Q4_0, N = 1: QKV (768 of 6144 rows), gate+up+SwiGLU (1792 of 14336) and the LM head
    (16032 of 128256) split by output rows; O (K = 512 of 4096) and down (K = 1792 of
    14336, fed by this GPU's h) split by K.  The collectives between them are not built
    here.  Weight sets (random bytes with finite scales) rotate through >= 512 MB, one set
    per step.  Reported: the whole step, launched eagerly and replayed as a HIP graph
    (median of `trials`, each over one pass through the sets), and each launch alone
    (a graph of `reps` rotated calls, median of `trials`)."""
    L = si.LLAMA3_8B
    H, I, V, Q = L["hidden"], L["intermediate"], L["vocab"], si.qkv_rows(L)
    q8, o8, i8, v8 = Q // 8, H // 8, I // 8, V // 8
    dev = torch.device("cuda")
    out = {}
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0):
        rb = lambda K: qmm.qmm_row_bytes(fmt, K)
        shapes = {"qkv": (q8, H), "o": (H, o8), "g": (i8, H), "u": (i8, H), "d": (H, i8), "lm": (v8, H)}
        set_bytes = sum(M * rb(K) for M, K in shapes.values())
        copies = max(1, -(-POOL_BYTES // set_bytes))
        bb = rb(32)

        def rand_w(M, K):
            w = torch.randint(0, 256, (M * rb(K),), dtype=torch.uint8, device=dev)
            w.view(-1, bb)[:, 1] &= 0x3B  # finite block scales
            return w
        sets = [{k: rand_w(M, K) for k, (M, K) in shapes.items()} for _ in range(copies)]
        x = torch.from_numpy(si.activations(1, H, 4600 + fmt)).to(dev)
        xo = torch.from_numpy(si.activations(1, o8, 4601 + fmt)).to(dev)
        y_qkv, y_o = torch.empty(q8, device=dev), torch.empty(H, device=dev)
        h, y_d, logits = torch.empty(i8, device=dev), torch.empty(H, device=dev), torch.empty(v8, device=dev)
        parts = [
            ("qkv", q8 * rb(H) + 4 * H + 4 * q8, lambda w: qmm.qmm_gemv(fmt, w["qkv"], x, y_qkv, q8, H, 1)),
            ("o", H * rb(o8) + 4 * o8 + 4 * H, lambda w: qmm.qmm_gemv(fmt, w["o"], xo, y_o, H, o8, 1)),
            ("gate_up", 2 * i8 * rb(H) + 4 * H + 4 * i8,
             lambda w: qmm.qmm_gate_up_silu(fmt, w["g"], w["u"], x, h, i8, H, 1)),
            ("down", H * rb(i8) + 4 * i8 + 4 * H, lambda w: qmm.qmm_gemv(fmt, w["d"], h, y_d, H, i8, 1)),
            ("lm_head", v8 * rb(H) + 4 * H + 4 * v8, lambda w: qmm.qmm_gemv(fmt, w["lm"], x, logits, v8, H, 1)),
        ]
        step_bytes = float(sum(b for _, b, _ in parts))

        def step(i):
            for _, _, fn in parts:
                fn(sets[i % copies])

        def one_pass():
            for i in range(copies):
                step(i)
        for i in range(copies):
            step(i)
        ms_eager, _ = median_trials(torch, one_pass, trials, copies)
        g = graph_of(torch, one_pass)
        g.replay()
        ms_graph, _ = median_trials(torch, g.replay, trials, copies)
        del g
        per = {}
        for name, b, fn in parts:
            def body(fn=fn):
                for i in range(reps):
                    fn(sets[i % copies])
            gp = graph_of(torch, body)
            gp.replay()
            ms, _ = median_trials(torch, gp.replay, trials, reps)
            per[name] = {"us": round(ms * 1e3, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b)}
            del gp
        # The oracle leg's re-check: one more step on set 0, its outputs and inputs.
        step(0)
        w0 = sets[0]
        TIMED_OUT[("tp8", fmt)] = {
            "x": x.cpu().numpy(), "xo": xo.cpu().numpy(), "h": h.cpu().numpy(),
            "y": {"qkv": y_qkv.cpu().numpy(), "o": y_o.cpu().numpy(), "down": y_d.cpu().numpy(),
                  "lm_head": logits[:DECODE_CHECK_ROWS].cpu().numpy()},
            "w": {k: w0[k][:min(shapes[k][0], DECODE_CHECK_ROWS) * rb(shapes[k][1])].cpu().numpy() for k in shapes},
            "dims": {"qkv": (q8, H), "o": (H, o8), "gate_up": (i8, H), "down": (H, i8), "lm_head": (v8, H)}}
        out[si.FMT_NAMES[fmt]] = {
            "step_us": round(ms_eager * 1e3, 2), "step_GBps": round(step_bytes / (ms_eager * 1e-3) / 1e9, 1),
            "graph_step_us": round(ms_graph * 1e3, 2),
            "graph_step_GBps": round(step_bytes / (ms_graph * 1e-3) / 1e9, 1),
            "step_bytes": int(step_bytes), "weight_sets": copies, "launches": per}
        del sets
        torch.cuda.empty_cache()
    return out


def expand_gemm(torch, qmm, si, reps=10):
    """Expand-then-GEMM prefill (qmm_expand_f16 into a caller-owned fp16 buffer, then
    the F16 qmm_gemm) against the fused LDS-decode GEMM, and the expansion's own HBM
    rate (bytes = raw blocks read + 2 M K written).  Random weight bytes with the
    scale bytes cleared of inf/NaN patterns: timing only."""
    dev = torch.device("cuda")

    def timed(fn, n=reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = []
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0):
        for (M, K) in ((14336, 4096), (4096, 14336)):
            rb = qmm.qmm_row_bytes(fmt, K)
            bb = 34 if fmt == si.FMT_Q8_0 else 18
            W = torch.randint(0, 256, (M * rb,), dtype=torch.uint8, device=dev)
            W.view(M * K // 32, bb)[:, 1] &= 0x3B  # scale exponent below the inf/NaN range
            W16 = torch.empty((M, K), dtype=torch.float16, device=dev)
            ms_e = timed(lambda: qmm.qmm_expand_f16(fmt, W, W16, M, K), 20)
            row = {"fmt": si.FMT_NAMES[fmt], "M": M, "K": K, "expand_us": round(ms_e * 1e3, 2),
                   "expand_GBps": round((M * rb + 2 * M * K) / (ms_e * 1e-3) / 1e9, 1), "T": []}
            for T in (128, 2048, 4096):
                X = torch.randn(T, K, device=dev).half()
                Y = torch.empty((T, M), device=dev)
                fl = 2.0 * T * M * K
                ms_f = timed(lambda: qmm.qmm_gemm(fmt, W, X, Y, M, K, T))
                ms_x = timed(lambda: (qmm.qmm_expand_f16(fmt, W, W16, M, K), qmm.qmm_gemm(1, W16, X, Y, M, K, T)))
                row["T"].append({"T": T, "fused_TFLOPs": round(fl / (ms_f * 1e-3) / 1e12, 1),
                                 "expand_then_gemm_TFLOPs": round(fl / (ms_x * 1e-3) / 1e12, 1)})
                capture_expand(("expand", fmt, M, K, T), fmt, W, W16, X, Y, rb)
            out.append(row)
            del W, W16
    return out


def capture_expand(key, fmt, W, W16, X, Y, rb):
    """Host copies for the re-check of an expand-then-GEMM case: the first
    PREFILL_CHECK_ROWS rows of the raw weights and of their fp16 expansion, and the
    first TOKEN_CHECK tokens of X and of the GEMM output on those rows."""
    R, n = PREFILL_CHECK_ROWS, TOKEN_CHECK
    TIMED_OUT[key] = {"w": W[:R * rb].cpu().numpy(), "w16": W16[:R].cpu().numpy(),
                      "x": X[:n].cpu().numpy(), "y": Y[:n, :R].cpu().numpy()}


def get_rows_bench(torch, qmm, si, reps=20):
    """Quantised embedding gather from the Llama-3-8B token table (128256 x 4096):
    bytes = n rows of raw blocks read + n x 4096 fp32 written."""
    L = si.LLAMA3_8B
    V, H = L["vocab"], L["hidden"]
    dev = torch.device("cuda")
    out = {}
    for fmt in (si.FMT_Q8_0, si.FMT_Q4_0, si.FMT_F16):
        rb = qmm.qmm_row_bytes(fmt, H)
        W = torch.randint(0, 256, (V * rb,), dtype=torch.uint8, device=dev)
        res = {}
        for n in (1, 4096):
            ids = torch.randint(0, V, (n,), dtype=torch.int32, device=dev)
            o = torch.empty((n, H), device=dev)
            for _ in range(3):
                qmm.qmm_get_rows(fmt, W, ids, o, V, H, n)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                qmm.qmm_get_rows(fmt, W, ids, o, V, H, n)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res[f"n{n}"] = {"us": round(ms * 1e3, 2), "GBps": round(n * (rb + 4 * H) / (ms * 1e-3) / 1e9, 1)}
            sel = ids[:16].long()
            TIMED_OUT[("get_rows", fmt, n)] = {"w": W.view(V, rb)[sel].cpu().numpy().reshape(-1),
                                               "out": o[:16].cpu().numpy(), "K": H}
        out[si.FMT_NAMES[fmt]] = res
        del W
    return out


def ceilings(torch, qmm):
    """Achievable ceilings: qmm_stream_read over 2 GiB (the read rate a plain kernel
    with the decode stream's loads reaches; median of 7 trials of 5 calls), and, with
    vendor code never linked into qmm, a 2 GiB device-to-device copy (bytes read + bytes
    written per second) and fp16 torch.matmul at the prefill shapes."""
    dev = torch.device("cuda")
    a = torch.ones(1 << 29, device=dev)  # 2 GiB fp32
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 31) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del b
    sink = torch.empty(qmm.QMM_STREAM_READ_BLOCKS, dtype=torch.int32, device=dev)

    def five_reads():
        for _ in range(5):
            qmm.qmm_stream_read(a, 1 << 31, sink)
    five_reads()
    ms_read, _ = median_trials(torch, five_reads, 7, 5)
    read_gbs = (1 << 31) / (ms_read * 1e-3) / 1e9
    del a, sink
    mm = []
    for (M, K) in ((14336, 4096), (4096, 14336)):
        B = torch.randn(M, K, device=dev).half()
        for T in (128, 2048, 4096):
            A = torch.randn(T, K, device=dev).half()
            for _ in range(3):
                torch.matmul(A, B.t())
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                torch.matmul(A, B.t())
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            mm.append({"M": M, "K": K, "T": T, "TFLOPs": round(2.0 * T * M * K / (ms * 1e-3) / 1e12, 1)})
    return {"stream_read_GBps": round(read_gbs, 1), "copy_read_plus_write_GBps": round(copy_gbs, 1),
            "torch_fp16_matmul": mm}


# Sources the dominant decode kernel is built from; its counter-derived traffic is
# reported only while their combined hash matches the one recorded with the counters.
DOMINANT_KERNEL = "gemv_dma_kernel<8, 1, 1, false, 8, 3, 0>"
DOMINANT_SOURCES = ("gemv_dma.hip", "gemv_block.hpp", "block_decode.hpp", "dma.hpp", "qmm_common.hpp",
                    "qmm_internal.hpp")


def _code_only(text):
    """C++ source with comments removed and whitespace runs collapsed: edits to comments
    or layout leave the kernel, and so this text, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":  # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_digest(files=DOMINANT_SOURCES):
    """sha256 of the dominant kernel's sources, code only (comments and layout removed)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, "block_quantized_weight_gguf_amd", "csrc", f)).read()
        h.update(_code_only(text).encode())
    return h.hexdigest()


def traffic_for(launch_key):
    """HBM bytes per launch from the committed counter summary, if the kernel sources are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
        digest = sources_digest()
        e = rec.get(launch_key)
        if e and e.get("source_sha256") == digest:
            return e["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; each GPU would run its own share of the rows", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_quantized_weight_gguf_amd as qmm
    import seeded_inputs as si

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "copies": 5}))
        return
    fmts, launches, host = decode_workload(torch, qmm, si)
    step_bytes = float(sum(b for _, _, b, _ in launches))
    torch.cuda.synchronize()

    def step(timer=None):
        for key, part, _, fn in launches:
            if timer is None:
                fn()
            else:
                timer.run((key, part), fn)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def k_steps():
        for _ in range(args.steps):
            step()
    # Whole-step timing (no per-launch events inside): the median of the trials, each of
    # K steps between synchronisations.
    ms_per_step, trial_ms = median_trials(torch, k_steps, args.trials, args.steps)
    # The same step captured once as a HIP graph and replayed (the launch path of a
    # serving loop); reported beside the eager figure.
    graph = graph_of(torch, step)
    for _ in range(args.warmup):
        graph.replay()

    def k_replays():
        for _ in range(args.steps):
            graph.replay()
    graph_ms_per_step, _ = median_trials(torch, k_replays, args.trials, args.steps)
    del graph
    # Per-launch timing over the same number of steps, for the roofline of each kernel.
    timer = Timer(torch)
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    for fmt, f in fmts.items():
        TIMED_OUT[("decode", fmt)] = capture_decode(qmm, si, fmt, f)

    per = {}
    for key, part, b, _ in launches:
        ts = timer.ms((key, part))
        per[f"{key}:{part}"] = {"bytes": b, "us_mean": 1e3 * float(np.mean(ts)),
                                "us_median": 1e3 * float(np.median(ts)),
                                "GBps": b / (np.mean(ts) * 1e-3) / 1e9}
    kern = {}
    for key, part, b, _ in launches:
        ts = timer.ms((key, part))
        k = kern.setdefault(key, {"bytes": 0.0, "ms": 0.0, "launches": 0})
        k["bytes"] += b * len(ts)
        k["ms"] += float(np.sum(ts))
        k["launches"] += len(ts)
    # Dominant kernel: the launch that streams the most bytes, and so takes the largest
    # share of the step (one kernel instance, as rocprofv3 names it): the Q8_0 LM-head
    # GEMV.  Chosen by bytes, not by measured time: a short launch's event pair can
    # also time the host when the GPU has run dry, and one stall would then pick it.
    dom = max(per, key=lambda k: per[k]["bytes"])
    dk = per[dom]
    achieved = dk["bytes"] / (dk["us_mean"] * 1e-6) / 1e9

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": "decode GEMV effective HBM GB/s (% of peak) + prefill GEMM TFLOP/s, Q8_0/Q4_0",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "trials": args.trials,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped single-token decode projections (QKV 6144x4096, O 4096x4096, "
                               "gate+up 2x14336x4096 + SwiGLU, down 4096x14336, LM head 128256x4096), "
                               "Q8_0 pass + Q4_0 pass, N=1",
                   "formats": ["Q8_0", "Q4_0"], "tokens": 1, "step_bytes": int(step_bytes),
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "trial_ms_per_step": [round(t, 5) for t in trial_ms],
                   "graph_replay": {"ms_per_step": round(graph_ms_per_step, 5),
                                    "GBps": round(step_bytes / (graph_ms_per_step * 1e-3) / 1e9, 2)}},
        "roofline": {"bound": "hbm",
                     "kernel": (DOMINANT_KERNEL + " (" + dom + ")") if dom == "gemv_Q8_0:lm_head" else dom,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(dom),
                     "avg_launch_us": round(dk["us_mean"], 3), "median_launch_us": round(dk["us_median"], 3),
                     "bytes_per_launch": int(dk["bytes"])},
    }

    line["single_gemv_576"] = config1(torch, qmm, si, args.trials)
    if not args.no_prefill:
        line["prefill_gemm"] = prefill(torch, qmm, si, args.trials, args.min_calls)
    if not args.no_smollm:
        line["smollm2_135m_decode_step"] = smollm2_step(torch, qmm, si, max(10, args.steps), args.trials)
    if not args.no_small_batch:
        line["small_batch_decode"] = small_batch(torch, qmm, si, args.trials)
    if not args.no_next:
        line["fused_decode_step"] = fused_decode(torch, qmm, si, fmts, max(10, args.steps))
        line["expand_then_gemm"] = expand_gemm(torch, qmm, si)
        line["get_rows"] = get_rows_bench(torch, qmm, si)
        line["more_formats"] = more_formats(torch, qmm, si, max(10, args.steps))
        line["tp8_shard_decode"] = tp8_shard_decode(torch, qmm, si, args.trials)
    if not (args.no_prefill or args.no_small_batch):
        line["ceilings"] = ceilings(torch, qmm)
        rd = line["ceilings"]["stream_read_GBps"]
        line["roofline"]["measured_stream_read_GBps"] = rd
        line["roofline"]["frac_of_measured_stream"] = round(achieved / rd, 4)
        line["config"]["frac_of_measured_stream"] = round(value / rd, 4)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(host, si, args.trials)
    if args.suite:
        with open(args.suite, "w") as fh:
            json.dump({"per_launch": per, "per_kernel": kern}, fh, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
