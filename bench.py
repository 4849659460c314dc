#!/usr/bin/env python3
"""Benchmark of jagged GDPA forward + backward (bf16 in, fp32 accumulate) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5|pffn] [--act NAME] [--attn gdpa|softmax]
                    [--norm] [--fp8] [--mx] [--no-per-config]

A step is one forward pass plus one backward pass (as gdpa_bwd runs it: the dK/dV
kernel, then the dQ kernel, or one pass) over the whole batch of the chosen
workload, with inputs resident in HBM.  The default workload is the largest
single-GPU configuration, the windowed long-history self-attention batch (B = 128
samples of uniform length 512..8192, local window |i - j| < 128, H = 4, d = 128,
exact-erf GELU): 1.02 TFLOP of useful work and 6.4 GB of algorithmic traffic per
step, far beyond the 256 MB last-level cache, so consecutive steps do not reuse
each other's data.  Without --steps, K is chosen after the warm-up so that the
timed region lasts at least 1.5 s.

The default run also times every workload (the four bf16 batches and the tiny fp32
one) direction by direction under "per_config": the median of 20 launches of the
forward and of the backward, each launch preceded by a 512 MiB device fill that
evicts the last-level cache, with time, useful TFLOP/s and % of the bf16 MFMA peak,
useful GB/s (forward 2 H d (2 Tq + 2 Tk) bytes, backward 2 H d (3 Tq + 4 Tk)) and %
of the HBM peak, and % of the attainable roofline min(MFMA peak, intensity x HBM
peak).

Prints one JSON line: `value` is useful TFLOP/s over fwd + bwd, counting only
valid (query, key) pairs: 4 H d |V| for the forward and 10 H d |V| for the
backward.  `roofline` describes the slowest kernel against the roof its
arithmetic intensity puts it under: HBM bandwidth for the attention workloads
(algorithmic bytes: each input read once, each output written once), the bf16
MFMA peak for pFFN (algorithmic FLOPs: the products the kernel's algorithm
performs, 4, 8, 6 and 10 H d |V| for the forward, dK/dV, dQ and one-pass
kernels), with the kernel's average duration from HIP events recorded on the
launch stream around each launch.  `cpu_baseline` times the fp64 oracle on the
host cores over a bounded prefix of the same batch.

--attn softmax runs jagged softmax attention (JFA) through the same kernels on the
same batch instead: the forward (also writing the row log-sum-exp), then the dQ
kernel (which also forms each row's D = sum dO * O from a third stationary tile of
O and writes the (LSE, D) pairs) and the dK/dV kernel that reads them; FLOPs are
counted as for GDPA (the exponentials and D are not counted).

--norm runs GDPA with the fused RMSNorm prologue on raw inputs (the tensors the
workload normalises: Q, K, V, or K, V for PMA): the 1/rms pre-pass, then the
forward, dK/dV and dQ kernels that read the raw tensors.  The line also carries the
plain kernels' time on the same batch and the HBM floor of the unfused norm the
prologue replaces (forward: read x, write x^; backward: read x and dx^, write dx).

--fp8 runs the forward with Q and K as fp8 (OCP e4m3, one scale per tensor,
quantised on the host before the timed region) and the backward with Q, K and dO as
fp8 (gdpa_fp8_bwd: plans whose backward is one pass, or d = 128 plans that store
dS; timed as one call); elsewhere the backward in bf16 as gdpa_bwd runs it.
Algorithmic bytes count one byte per element of the fp8 tensors.

--mx runs the forward with Q and K block-scaled (OCP MXFP8: e4m3 elements, one E8M0
scale per 32 head columns of a row, quantised on the host before the timed region)
on the scaled MFMA, the backward as for --fp8; the forward's algorithmic bytes count
one byte per element of Q and K plus their scale bytes (d / 32 per row and head).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "useful TFLOP/s, jagged GDPA fwd+bwd bf16, % of MFMA peak, 1 MI355X"
METRIC_JFA = "useful TFLOP/s, jagged softmax attention (JFA) fwd+bwd bf16, 1 MI355X"
METRIC_FP8 = "useful TFLOP/s, jagged GDPA fwd (fp8 Q, K) + bwd (fp8 Q, K, dO where one pass, else bf16), 1 MI355X"
METRIC_MX = "useful TFLOP/s, jagged GDPA fwd (MXFP8 Q, K) + bwd (bf16), 1 MI355X"
METRIC_NORM = "useful TFLOP/s, jagged GDPA fwd+bwd with fused RMSNorm prologue, bf16, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector (the fp32 path runs no MFMA)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_flops(H, d, pairs, Tq=0, Tk=0, ds=False):
    """Algorithmic FLOPs per launch: the MFMA products each kernel's algorithm performs
    (stat: the JFA pre-pass's dot products dO . O; rstd: the sums of squares of the norm;
    ds: the dQ kernel multiplies the stored dS by K, one product, instead of
    recomputing S and dP)."""
    u = 2.0 * H * d * pairs          # one product over the valid pairs
    return {"fwd": 2 * u, "dkdv": 4 * u, "dq": (1 if ds else 3) * u, "bwd": 5 * u, "stat": 2.0 * H * d * Tq,
            "rstd": 2.0 * H * d * (Tq + 2 * Tk)}


def kernel_bytes(H, d, Tq, Tk, softmax=False, norm="", fp8=False, ds_bytes=0, mx=False, fp8_bwd=False):
    """Algorithmic bytes per launch (bf16): every input read once, every output written
    once; softmax (JFA): plus the fp32 row LSE written by the forward, and the fp32
    (LSE, D) row pair that the pre-pass writes and the gradient kernels read; norm
    (RMSNorm prologue): plus the fp32 1/rms factors (H (Tq + 2 Tk)) that the rstd
    pre-pass writes, after reading the tensors it normalises, and the kernels read;
    ds_bytes (a plan that stores dS): the dK/dV kernel also writes the dS blocks, and
    the dQ kernel reads them and K instead of recomputing the scores; mx (block-scaled
    fp8 Q and K): their d / 32 E8M0 scale bytes per row and head as well; fp8_bwd (the
    backward on fp8 Q, K, dO, one pass or, with ds_bytes, dK/dV storing dS and dQ from
    it, as one "bwd" entry): one byte per element of those."""
    e = 2 * H * d
    lse, st = (4 * H * Tq, 8 * H * Tq) if softmax else (0, 0)
    rs = 4 * H * (Tq + 2 * Tk) if norm else 0
    qk = 0.5 if fp8 else 1.0                           # fp8 Q, K: one byte per element
    dq = (e * (Tq + Tk) + ds_bytes if ds_bytes else   # dS, K -> dQ
          e * (3 * Tq + 2 * Tk) + (e * Tq + lse if softmax else 0) + st + rs)   # Q, dO, K, V (+ O, LSE) -> dQ
    mxs = H * (d // 32) * (Tq + Tk) if mx else 0        # E8M0 scale bytes of Q and K
    return {"fwd": int(e * (qk * Tq + qk * Tk + Tk + Tq)) + lse + rs + mxs,   # Q, K, V (, rstd) -> O (, LSE)
            "dkdv": e * (2 * Tq + 4 * Tk) + st + rs + ds_bytes,   # Q, dO, K, V (, stat or rstd) -> dK, dV (, dS)
            "dq": dq,
            "bwd": (e * (2 * Tq + 4 * Tk) + 2 * ds_bytes if fp8_bwd and ds_bytes  # + K again, dS out and in
                    else int(e * (2 * Tq + 3.5 * Tk)) if fp8_bwd  # fp8 Q, dO, K; bf16 V -> dQ, dK, dV
                    else e * (3 * Tq + 4 * Tk)),         # one-pass backward: Q, dO, K, V -> dQ, dK, dV
            "stat": 2 * e * Tq + lse + st,              # O, dO, LSE -> stat
            "rstd": e * (Tq * ("q" in norm) + Tk * ("k" in norm) + Tk * ("v" in norm)) + rs}


KERNEL_SOURCES = ("device.hpp", "ring.hpp", "fwd_bf16.hip", "bwd_bf16.hip", "bwd_common.hpp", "bwd_fused.hip",
                  "jfa.hip", "norm.hip", "partials.hip", "kernels.hpp", "plan.cpp", "plan.hpp", "api.cpp", "gelu_poly.h",
                  "noalloc.hip", "bwd16.hip")


def kernel_source_digest() -> str:
    """sha256 over the kernel and planner sources and the build script, whose code
    generation options differ per object (identifies the build the counters came from)."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(os.path.dirname(os.path.abspath(__file__)), "recsys_attention_jagged_amd")
    for name in KERNEL_SOURCES + ("../build.py",):
        with open(os.path.normpath(os.path.join(pkg, "csrc", name)), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary of `workload`,
    or None if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes")


def cpu_baseline(inp, budget_s=15.0, softmax=False, norm=""):
    """Time the fp64 oracle (forward + backward; softmax: jfa_fwd + jfa_bwd; norm: the
    RMSNorm-prologue forms) on a prefix of the batch."""
    import numpy as np
    import torch
    from oracle import gdpa_ref as R
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    spent, flops, n, rows = 0.0, 0, 0, 0
    f = lambda t, a, e: t[a:e].to("cpu", torch.float64).numpy()
    for b in range(len(inp.lq)):
        qs, qe = int(inp.q_off[b]), int(inp.q_off[b + 1])
        ks, ke = int(inp.kv_off[b]), int(inp.kv_off[b + 1])
        k, v = f(inp.k, ks, ke), f(inp.v, ks, ke)
        # a long windowless sample is taken in blocks of 2048 query rows (each block
        # against all the sample's keys), so the budget can stop inside it
        step = 2048 if inp.window == 0 else qe - qs
        for a in range(qs, max(qe, qs + 1), max(step, 1)):
            e = min(qe, a + step)
            q, do = f(inp.q, a, e), f(inp.do, a, e)
            qo, ko = np.array([0, e - a]), np.array([0, ke - ks])
            t0 = time.perf_counter()
            if softmax:
                R.jfa_fwd(q, k, v, qo, ko, inp.window)
                R.jfa_bwd(q, k, v, do, qo, ko, inp.window)
            elif norm:
                R.norm_gdpa_fwd(q, k, v, qo, ko, inp.act, inp.window, norm)
                R.norm_gdpa_bwd(q, k, v, do, qo, ko, inp.act, inp.window, norm)
            else:
                R.gdpa_fwd(q, k, v, qo, ko, inp.act, inp.window)
                R.gdpa_bwd(q, k, v, do, qo, ko, inp.act, inp.window)
            spent += time.perf_counter() - t0
            flops += 14 * inp.H * inp.d * R.useful_pairs([e - a], [ke - ks], inp.window)
            rows += e - a
            if spent >= budget_s:
                break
        n += 1
        if spent >= budget_s:
            break
    return {"value": flops / spent / 1e12 if spent > 0 else None, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} query rows of the first {n} of {len(inp.lq)} samples, fp64 numpy/scipy "
                      f"forward+backward, {spent:.1f} s, same seeded inputs"}


def direction_table(cfg: int, seed: int = 0, runs: int = 20, warm: int = 3):
    """Per-direction figures of workload `cfg` (see the module docstring)."""
    import statistics
    import torch
    import recsys_attention_jagged_amd as G
    from gdpa_workloads import WORKLOADS, make_workload
    w = WORKLOADS[cfg]
    inp = make_workload(cfg, seed=seed, device="cuda")
    qo = torch.tensor(inp.q_off, dtype=torch.int32, device="cuda")
    ko = torch.tensor(inp.kv_off, dtype=torch.int32, device="cuda")
    B, H, d, win, act = len(inp.lq), inp.H, inp.d, inp.window, inp.act
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out_rows = {}
    with G.Plan(inp.q_off, inp.kv_off, H, d, win, w["dtype"]) as plan:
        st = plan.stats()
        Tq, Tk, pairs = st["Tq"], st["Tk"], st["valid_pairs"]
        o, dq, dk, dv = (torch.empty_like(t) for t in (inp.q, inp.q, inp.k, inp.v))
        calls = {"fwd": lambda: G.gdpa_fwd(plan.handle, inp.q, inp.k, inp.v, qo, ko, B, H, d, act, win, o, sh),
                 "bwd": lambda: G.gdpa_bwd(plan.handle, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win,
                                           dq, dk, dv, sh)}
        e = 2 * H * d if w["dtype"] == "bf16" else 4 * H * d
        alg_bytes = {"fwd": e * (2 * Tq + 2 * Tk), "bwd": e * (3 * Tq + 4 * Tk)}
        flops = {"fwd": 4.0 * H * d * pairs, "bwd": 10.0 * H * d * pairs}
        for direction in w["directions"]:
            f = calls[direction]
            times = []
            for r in range(warm + runs):
                scrub.fill_(r & 0xFF)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                f()
                b.record(stream)
                b.synchronize()
                if r >= warm:
                    times.append(a.elapsed_time(b))
            ms = statistics.median(times)
            tf = flops[direction] / (ms * 1e-3) / 1e12
            gbs = alg_bytes[direction] / (ms * 1e-3) / 1e9
            peak_tf = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_FP32_VECTOR_TFLOPS
            ai = flops[direction] / alg_bytes[direction]
            attain = min(peak_tf, ai * PEAK_HBM_GBS / 1e3)
            out_rows[direction] = {"ms": round(ms, 4), "useful_TFLOPs": round(tf, 2),
                                   "pct_peak_compute": round(100 * tf / peak_tf, 2),
                                   "useful_GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                                   "attainable_TFLOPs": round(attain, 1),
                                   "pct_attainable": round(100 * tf / attain, 2)}
    del scrub
    torch.cuda.empty_cache()
    return {"workload": w["name"], "compute_peak": "bf16 MFMA" if w["dtype"] == "bf16" else "fp32 vector",
            **out_rows}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: enough for at least 1.5 s of timed work)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="5", choices=["2", "3", "4", "5", "pffn"])
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-workload, per-direction table")
    ap.add_argument("--act", default=None, help="override the workload's activation (e.g. gelu_poly)")
    ap.add_argument("--attn", default="gdpa", choices=["gdpa", "softmax"],
                    help="softmax: jagged softmax attention (JFA) on the same batch")
    ap.add_argument("--norm", action="store_true",
                    help="GDPA with the fused RMSNorm prologue on raw inputs of the same batch")
    ap.add_argument("--fp8", action="store_true",
                    help="forward with fp8 (e4m3) Q and K, backward in bf16, on the same batch")
    ap.add_argument("--mx", action="store_true",
                    help="forward with block-scaled fp8 (MXFP8) Q and K, backward in bf16, on the same batch")
    ap.add_argument("--claim", default="auto", choices=["auto", "bins", "always"],
                    help="how workgroups get items: claimed at run time where the plan decides (auto), "
                         "the planner's bins only, or claimed wherever the kernel runs one-wave teams")
    ap.add_argument("--dq-team", default="auto", choices=["auto", "one_wave"],
                    help="dQ from stored dS in two-wave teams over 64-row q items (auto) or one-wave workgroups")
    ap.add_argument("--slot-time", default="auto", choices=["auto", "off"],
                    help="deal weighted by each bin's dispatch round on its CU where the plan decides (auto), "
                         "or every bin dealt by plain cost")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (reference kernel for "
                         "calibrating the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(GDPA shards by sample with no exchange; see the design notes).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return 0
    import recsys_attention_jagged_amd as G
    from gdpa_workloads import PFFN, WORKLOADS, make_pffn, make_workload

    G.load_library()
    w = PFFN if args.config == "pffn" else WORKLOADS[int(args.config)]
    log(f"generating workload {args.config} ({w['name']}) on cuda:0 ...")
    if args.config == "pffn":   # one sample: every query row against the shared weight rows
        inp = make_pffn(seed=args.seed, device="cuda", act=args.act)
    else:
        inp = make_workload(int(args.config), seed=args.seed, device="cuda", act=args.act, raw=args.norm)
    torch.cuda.synchronize()
    qo = torch.tensor(inp.q_off, dtype=torch.int32, device="cuda")
    ko = torch.tensor(inp.kv_off, dtype=torch.int32, device="cuda")
    B, H, d, win, act = len(inp.lq), inp.H, inp.d, inp.window, inp.act

    sm = args.attn == "softmax"
    if (sm or args.norm) and args.config == "pffn":
        print("--attn softmax and --norm run the attention workloads", file=sys.stderr)
        return 2
    if sum([sm, args.norm, args.fp8, args.mx]) > 1:
        print("--attn softmax, --norm, --fp8 and --mx are separate modes", file=sys.stderr)
        return 2
    if (args.fp8 or args.mx) and args.config == "pffn":
        print("--fp8 and --mx run the attention workloads", file=sys.stderr)
        return 2
    if args.mx and d < 64:
        print("--mx needs d >= 64 (64-wide scaled k blocks)", file=sys.stderr)
        return 2
    norm = w["rms"] if args.norm else ""
    t0 = time.perf_counter()
    plan = G.Plan(inp.q_off, inp.kv_off, H, d, win, "bf16", claim=args.claim, slot_time=args.slot_time,
                  dq_team=args.dq_team)
    plan_ms = (time.perf_counter() - t0) * 1e3
    st = plan.stats()
    Tq, Tk, pairs = st["Tq"], st["Tk"], st["valid_pairs"]

    o = torch.empty_like(inp.q)
    dq = torch.empty_like(inp.q)
    dk = torch.empty_like(inp.k)
    dv = torch.empty_like(inp.v)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    h = plan.handle

    def fwd():
        G.gdpa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, act, win, o, sh)

    def dkdv():
        G.gdpa_bwd_dkdv(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, dk, dv, sh)

    def dqk():
        G.gdpa_bwd_dq(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, dq, sh)

    def bwd():
        G.gdpa_bwd(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, dq, dk, dv, sh)

    if sm:
        act = "softmax"
        lse = torch.empty((H, Tq), dtype=torch.float32, device="cuda")
        stat = torch.empty((H, Tq, 2), dtype=torch.float32, device="cuda")

        def jfwd():
            G.gdpa_jfa_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, win, o, lse, sh)

        def jdkdv():
            G.gdpa_jfa_bwd_dkdv(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, win, stat, dk, dv, sh)

        def jdq():
            G.gdpa_jfa_bwd_dq(h, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, B, H, d, win, stat, dq, sh)

        def jbwd():
            G.gdpa_jfa_bwd(h, inp.q, inp.k, inp.v, o, lse, inp.do, qo, ko, B, H, d, win, stat, dq, dk, dv, sh)

    if norm:
        rstd = torch.empty((H * (Tq + 2 * Tk),), dtype=torch.float32, device="cuda")

        def nrstd():
            G.gdpa_norm_rstd(h, inp.q, inp.k, inp.v, H, d, norm, rstd, sh)

        def nfwd():
            G.gdpa_norm_fwd(h, inp.q, inp.k, inp.v, qo, ko, B, H, d, act, win, norm, rstd, o, sh)

        def ndkdv():
            G.gdpa_norm_bwd_dkdv(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, norm, rstd, dk, dv, sh)

        def ndq():
            G.gdpa_norm_bwd_dq(h, inp.q, inp.k, inp.v, inp.do, qo, ko, B, H, d, act, win, norm, rstd, dq, sh)

    if args.fp8:
        def quant(t):   # per-tensor scale amax / 448, OCP e4m3 bytes (on the host, once)
            x = t.float().cpu()
            sc8 = max(float(x.abs().max()) / 448.0, 1e-30)
            return (x / sc8).to(torch.float8_e4m3fn).view(torch.uint8).to("cuda"), sc8
        q8, sq8 = quant(inp.q)
        k8, sk8 = quant(inp.k)

        def ffwd():
            G.gdpa_fp8_fwd(h, q8, k8, inp.v, qo, ko, B, H, d, act, win, sq8, sk8, o, sh)

        do8, sdo8 = quant(inp.do)

        def fbwd():
            G.gdpa_fp8_bwd(h, q8, k8, inp.v, do8, qo, ko, B, H, d, act, win, sq8, sk8, sdo8, dq, dk, dv, sh)

    if args.mx:
        def quant_mx(t):   # e4m3 bytes [T, H, d] and E8M0 scales [H, T, d / 32] (on the host, once)
            x = t.float().cpu()
            T_, H_, d_ = x.shape
            xb = x.reshape(T_, H_, d_ // 32, 32)
            amax = xb.abs().amax(-1)
            ex = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 8,
                             torch.full_like(amax, -127.0)).clamp(-127, 127)
            q = (xb / torch.exp2(ex)[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).reshape(T_, H_, d_)
            return (q.view(torch.uint8).to("cuda"),
                    (ex + 127).to(torch.uint8).permute(1, 0, 2).contiguous().to("cuda"))
        qm8, qms = quant_mx(inp.q)
        km8, kms8 = quant_mx(inp.k)

        def ffwd():
            G.gdpa_mx_fwd(h, qm8, qms, km8, kms8, inp.v, qo, ko, B, H, d, act, win, o, sh)

    # the backward as gdpa_bwd / gdpa_jfa_bwd run it: one pass, or the dK/dV and dQ
    # kernels (the norm prologue: always the two kernels, after its pre-pass; JFA: one
    # pass only where every Lk <= 32)
    fused = 0 if norm else (int(st["bwd_fused"] == 1) if sm else st["bwd_fused"])
    fp8_bwd = args.fp8 and bool(fused or st["ds_bytes"] > 0)   # plans gdpa_fp8_bwd runs on
    if sm:
        calls = [("fwd", jfwd), ("bwd", jbwd)] if fused else [("fwd", jfwd), ("dq", jdq), ("dkdv", jdkdv)]
    elif norm:
        calls = [("rstd", nrstd), ("fwd", nfwd), ("dkdv", ndkdv), ("dq", ndq)]
    else:
        f0 = ffwd if (args.fp8 or args.mx) else fwd
        if fp8_bwd:   # one call (one pass, or dK/dV storing dS then dQ from it)
            calls = [("fwd", f0), ("bwd", fbwd)]
        else:
            calls = [("fwd", f0), ("bwd", bwd)] if fused else [("fwd", f0), ("dkdv", dkdv), ("dq", dqk)]
    for _ in range(args.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()

    K = args.steps
    if K is None:   # enough steps for 1.5 s of timed work (at least 20)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            for _, c in calls:
                c()
        b.record(stream)
        torch.cuda.synchronize()
        K = max(20, math.ceil(1500.0 / (a.elapsed_time(b) / 3)))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        for j, (_, c) in enumerate(calls):
            c()
            ev[i][j + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / K
    kms = {name: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)) / K
           for j, (name, _) in enumerate(calls)}

    useful = 14.0 * H * d * pairs
    value = useful / (ms_step * 1e-3) / 1e12
    ds_bytes = 0 if (sm or norm or fused) else st["ds_bytes"]   # what gdpa_bwd_dkdv / _dq (or fp8) run with
    kb = kernel_bytes(H, d, Tq, Tk, softmax=sm, norm=norm, fp8=args.fp8 or args.mx, ds_bytes=ds_bytes, mx=args.mx,
                      fp8_bwd=fp8_bwd)
    kf = kernel_flops(H, d, pairs, Tq, Tk, ds=ds_bytes > 0)
    dom = max(kms, key=kms.get)
    trace_name = w["name"] + ("_jfa" if sm else "_norm" if norm else "_fp8" if args.fp8 else "_mx" if args.mx else "")   # its counter record
    # the roof the kernel's arithmetic intensity puts it under (ridge: peak FLOP/s / peak B/s)
    mfma_bound = kf[dom] / kb[dom] > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = kf[dom] / (kms[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "algorithmic_flops": kf[dom], "traffic": measured_traffic(trace_name, dom)}
    else:
        achieved = kb[dom] / (kms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "algorithmic_bytes": kb[dom], "traffic": measured_traffic(trace_name, dom)}
    kernels = {n: {"ms": round(kms[n], 4), "alg_GBps": round(kb[n] / (kms[n] * 1e-3) / 1e9, 1)}
               for n in kms}
    kernels["fwd"]["useful_TFLOPs"] = round(4.0 * H * d * pairs / (kms["fwd"] * 1e-3) / 1e12, 2)
    bwd_ms = kms["bwd"] if "bwd" in kms else kms["dkdv"] + kms["dq"] + kms.get("stat", 0.0)

    out = {
        "metric": (METRIC_JFA if sm else METRIC_NORM if norm else METRIC_FP8 if args.fp8 else
                   METRIC_MX if args.mx else METRIC),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16" if args.fp8 else "mxfp8+bf16" if args.mx else "bf16",
        "data": "synthetic (seeded jagged lengths and N(0,1) values; see gdpa_workloads)",
        "config": {"workload": w["name"], "B": B, "H": H, "d": d,
                   "act": act, "window": win, "Tq": Tq, "Tk": Tk, "valid_pairs": pairs, "ds_bytes": ds_bytes,
                   "bwd_inputs": "fp8 Q, K, dO" if fp8_bwd else "bf16",
                   "claimed_lists": st["claimed"],
                   "slot_weighted_lists": st["slot_weighted"],
                   "dq_team": st["dq_team"],
                   "backward": ("one KV-stationary pass (D formed from P and dP)" if sm and fused else
                                "dQ kernel (also D and the row statistics) + dK/dV kernel" if sm else
                                "dK/dV + dQ kernels (1/rms pre-pass before the forward)" if norm else
                                ["dK/dV + dQ kernels", "one KV-stationary pass", "one Q-stationary pass"][fused])},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_useful_TFLOPs": kernels["fwd"]["useful_TFLOPs"],
        "bwd_useful_TFLOPs": round(10.0 * H * d * pairs / (bwd_ms * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "plan_ms": round(plan_ms, 1),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
    }
    if norm:
        # the plain kernels on the same batch (as gdpa_bwd runs them; timing does not
        # depend on the values), and
        # the HBM floor of an unfused RMSNorm of the same tensors: forward reads x and
        # writes x^, backward reads x and dx^ and writes dx
        pcalls = [fwd, bwd] if st["bwd_fused"] else [fwd, dkdv, dqk]
        for c in pcalls:
            c()
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for _ in range(K):
            for c in pcalls:
                c()
        p1.record(stream)
        torch.cuda.synchronize()
        rows = Tq * ("q" in norm) + Tk * ("k" in norm) + Tk * ("v" in norm)
        out["norm"] = {"tensors": norm, "plain_kernels_ms": round(p0.elapsed_time(p1) / K, 4),
                       "fused_ms": round(ms_step, 4),
                       "unfused_norm_hbm_floor_ms": round(5 * 2 * H * d * rows / (PEAK_HBM_GBS * 1e9) * 1e3, 4)}
    default_mode = not (sm or norm or args.fp8 or args.mx) and args.config != "pffn" and args.act is None
    if default_mode and not args.no_per_config:
        out["per_config"] = {}
        for cfg in sorted(WORKLOADS):
            log(f"per-direction timing of workload {cfg} ...")
            out["per_config"][str(cfg)] = direction_table(cfg, args.seed)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, softmax=sm, norm=norm)
    plan.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
