"""Benchmark of the attention backward hot path on one MI355X.

One step = attn_bwd_preprocess (D = rowsum(dO o O)) + attn_bwd_with_dq (dK, dV
and dQ = scale * sum_j dS K_j rounded to bf16) on the long-sequence causal
workload (B=1, H=8, N=16384, d=128, bf16), with Q, K, V, dO, O and LSE resident in HBM before the timed
region (O and LSE come from attn_fwd_stats, outside the timed region).

Throughput: backward FLOPs of the metric, 10 N^2 d per query head, halved for
a causal mask, divided by the measured time per step.  Prints one JSON line.

Flags: --gpus N (only 1 is supported: the library and this run use one GPU),
--steps K, --warmup W, --workload NAME, --no-cpu-baseline,
--copy-calibration (time a plain 1 GiB device copy instead; its known byte
count calibrates the FETCH_SIZE / WRITE_SIZE counters of rocprofv3).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-backward TFLOP/s (10·N²·d/head) and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
DEFAULT_WORKLOAD = "bf16_causal_b1h8_n16384_d128"
BWD_SOURCES = [os.path.join(ROOT, "flashattention_backward_pass_amd", "csrc", f)
               for f in ("bwd_dkdv.hip", "bwd_dkdv_block.h", "bwd_dq.hip", "bwd_dq_block.h", "mfma_common.h", "philox.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "bwd_mfma.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed after evicting the caches (0: skip); reported beside the warm value")
    return ap.parse_args()


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, launch_bytes_key="bytes_per_launch"):
    """HBM bytes per attn_bwd_with_dq launch from committed rocprofv3 counter runs,
    valid only for the workload they were taken on and while the kernel
    source is the one they were taken on."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha") != source_sha(BWD_SOURCES):
        return None
    return t.get(launch_bytes_key)


def measured_mfma(workload):
    """MFMA instructions per attn_bwd_with_dq launch (SQ_INSTS_MFMA of a
    committed rocprofv3 run), under the same validity rule as the traffic."""
    try:
        t = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha") != source_sha(BWD_SOURCES):
        return None
    return sum(t["mfma_per_launch"].values()), t["flop_per_mfma"]


def copy_calibration(torch):
    n = 1 << 28  # 2^28 float32 = 1 GiB
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": dt * 1e3,
                      "GBs": 2 * n * 4 / dt / 1e9}), flush=True)


def cpu_baseline(w, x, heads=3):
    """The fp64 oracle, untuned, on the first `heads` query heads of batch 0 of
    the workload at full N.  Each head's forward (O, LSE: the backward's
    inputs) runs first, untimed apart; the backward alone is timed, and its
    rate is the metric FLOPs of those heads over the backward time."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    heads = min(heads, w.H)
    group = w.H // w.H_kv
    t_fwd = t_bwd = 0.0
    for h in range(heads):
        q, do = x["Q"][0, h], x["dO"][0, h]
        k, v = x["K"][0, h // group], x["V"][0, h // group]
        zf = oracle.head_dropout(w.dropout, h)
        t0 = time.perf_counter()
        O, L = oracle.forward_head(q, k, v, w.tau, w.causal, w.softcap, w.window, zf)
        t1 = time.perf_counter()
        oracle.backward_head(q, k, v, O, do, L, w.tau, w.causal, w.softcap, w.window, zf)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
    flops = heads * w.flops() / (w.B * w.H)
    return {"value": flops / t_bwd / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{heads} query heads (b=0, h=0..{heads - 1}) of the workload at full N={w.N}: fp64 "
                      f"backward alone, {t_bwd:.1f} s wall (their forward, {t_fwd:.1f} s, timed apart); "
                      f"metric FLOPs of those heads",
            "seconds": round(t_bwd, 3), "forward_seconds": round(t_fwd, 3),
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the backward library is a "
              "single-GPU path (it would shard by whole key/value heads, one share per GPU, with no "
              "communication).", file=sys.stderr)
        sys.exit(2)
    import torch

    import flashattention_backward_pass_amd as fab
    from flashattention_backward_pass_amd import workloads

    if args.copy_calibration:
        copy_calibration(torch)
        return
    w = workloads.WORKLOADS[args.workload]
    fab.load_library()
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("Q", "K", "V", "dO"))
    kw = dict(causal=w.causal, scale=w.tau, softcap=w.softcap, window=w.window)
    o, lse = fab.attention_forward(q, k, v, dropout=w.dropout, **kw)
    B, H, N, d = q.shape
    D = torch.empty(B, H, N, device=dev, dtype=torch.float32)
    acc = torch.empty(B, H, N, d, device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fab.attn_bwd_preprocess(o, do, D, acc, H_kv=w.H_kv, **kw)
        if ev is not None:
            ev[1].record()
        fab.attn_bwd_with_dq(q, k, v, do, lse, D, acc, dq, dk, dv, dropout=w.dropout, **kw)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps, synchronised on both sides.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    # Cold caches: before each of these steps a 512 MiB fill (twice the
    # 256 MB Infinity Cache, far above the L2s) evicts the inputs; only the
    # step itself is timed, with events.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 27, device=dev, dtype=torch.float32)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(float(i))
            step(cev[i])
        torch.cuda.synchronize()
        cms = sorted(e[0].elapsed_time(e[2]) for e in cev)[args.cold_steps // 2]
        cold = {"ms_per_step": round(cms, 4), "tflops": round(w.flops() / (cms * 1e-3) / 1e12, 2),
                "steps": args.cold_steps, "statistic": "median of event-timed steps, each after a 512 MiB fill"}
        del flush

    # The two bandwidth-bound kernels, each timed over back-to-back launches
    # (kernel throughput; the per-step time of the preprocess above also holds
    # the launch gap after the previous step).  attn_bwd_dq_convert (dQ = scale
    # * dQaccum in bf16) is not part of the step (attn_bwd_with_dq stores dQ
    # itself); it runs over the same tensors.
    stream_iters = 20
    dq_conv = torch.empty_like(q)

    def back_to_back(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(stream_iters):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / stream_iters

    pre_b2b = back_to_back(lambda: fab.attn_bwd_preprocess(o, do, D, acc, H_kv=w.H_kv, **kw))
    conv_ms = back_to_back(lambda: fab.attn_bwd_dq_convert(acc, dq_conv, scale=w.tau))
    del dq_conv

    # The forward (attn_fwd_stats) is a support step outside the timed
    # backward step; timed here on its own for reference.
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    fe[0].record()
    for _ in range(5):
        fab.attn_fwd_stats(q, k, v, o, lse, dropout=w.dropout, **kw)
    fe[1].record()
    torch.cuda.synchronize()
    fwd_ms = fe[0].elapsed_time(fe[1]) / 5
    fwd_flops = 0.4 * w.flops()  # 4 N^2 d per head (causal: half; window: 4 d per visible pair)

    flops = w.flops()
    ms = wall / args.steps * 1e3
    value = flops / (ms * 1e-3) / 1e12
    bwd_tflops = flops / (bwd * 1e-3) / 1e12
    esz = 2 if w.dtype == "bf16" else 4
    pre_bytes = 2 * B * H * N * d * esz + B * H * N * 4           # read O, dO; write D
    conv_bytes = B * H * N * d * (4 + esz)                         # read dQaccum; write dQ
    traffic = measured_traffic(w.name)
    mfma = measured_mfma(w.name)
    mfma_issue = None
    if mfma is not None:
        issued = mfma[0] * mfma[1] / (bwd * 1e-3) / 1e12
        mfma_issue = {"instructions_per_launch": mfma[0], "tflops": round(issued, 2),
                      "frac_of_peak": round(issued / PEAK_BF16_TFLOPS, 4),
                      "note": "matrix work the kernels issue (S and dP are computed twice, once per kernel; "
                              "diagonal tiles in full) per measured attn_bwd_with_dq time, against the same peak; "
                              "instruction count from profiles/bwd_mfma.json"}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid normal Q, K, V, dO; O and LSE from attn_fwd_stats)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "d": w.d,
                   "causal": w.causal, "softcap": w.softcap, "tau": w.tau, "window": list(w.window),
                   "dropout_p": w.dropout[0] if w.dropout else 0.0, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(bwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_bwd_with_dq entry point (bf16: bwd_dkdv_kernel + bwd_dq_kernel, "
                               "which writes dQ)",
                     "flops_per_launch": flops, "mfma_issue": mfma_issue,
                     "note": "achieved = metric FLOPs (10 N^2 d per head, halved when causal; with a local window "
                             "10 d per visible (query, key) pair) / measured attn_bwd_with_dq time; the two kernels issue "
                             "14/10 of that as MFMA work because the dQ kernel recomputes S and dP"},
        "kernels_ms": {"bwd_preprocess": round(pre, 4), "bwd_with_dq": round(bwd, 4)},
        "stream_kernels_GBs": {"bwd_preprocess": round(pre_bytes / (pre_b2b * 1e-3) / 1e9, 1),
                               "bwd_dq_convert": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                               "peak": PEAK_HBM_GBS,
                               "frac_of_peak": {"bwd_preprocess": round(pre_bytes / (pre_b2b * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                                "bwd_dq_convert": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                               "bytes": {"bwd_preprocess": pre_bytes, "bwd_dq_convert": conv_bytes},
                               "ms": {"bwd_preprocess": round(pre_b2b, 5), "bwd_dq_convert": round(conv_ms, 5)},
                               "bwd_preprocess_in_step_ms": round(pre, 5),
                               "note": "algorithmic bytes (preprocess: read O, dO, write D; convert: read "
                                       f"dQaccum, write dQ) / duration over {stream_iters} back-to-back launches "
                                       "(events on the launch stream); bwd_preprocess_in_step_ms is the event time "
                                       "of the step's own preprocess call, launch gap included; the step does not "
                                       "run convert"},
        "cold_cache": cold,
        "forward": {"kernel": "attn_fwd_stats (not part of the timed step)", "ms": round(fwd_ms, 4),
                    "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1), "flops": "4/10 of the backward metric FLOPs"},
    }
    try:
        out["git"] = subprocess.run(["git", "rev-parse", "--short", "HEAD"], capture_output=True, text=True,
                                    cwd=ROOT).stdout.strip() or None
    except Exception:
        out["git"] = None
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
