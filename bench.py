"""Benchmark of the fused exact-attention hot path on one MI355X.

A step is one forward and one backward (every stage of the path: tiling,
causal mask, online softmax, dropout, the O+LSE epilogue, the dO.O
preprocess, recomputation and the dQ/dK/dV products) over the training
workload B=4, H=32, N=4096, d=128, bf16, causal, dropout p=0.1, with the
inputs resident in HBM.  The metric is attention TFLOP/s of forward +
backward, counted as 3.5 * F with F = 4 B H N^2 d / 2 (causal), and its
fraction of the bf16 dense matrix-core peak (2516.6 TFLOP/s).

Prints one JSON line.  Besides the headline it reports the dominant
kernel's roofline position (HIP-event timing of its launches over the timed
region), the other stages' timings, secondary workloads, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6        # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2         # 256 CU x 8192 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s fwd & fwd+bwd (bf16, causal, d=128) + % of MFMA peak"
# Sources of the 16-bit kernels each stage runs (the counters in
# profiles/traffic.json are only used while these are unchanged).
KERNEL_SOURCES = {"fwd": "fa_fwd_pp.hip", "bwd_dkdv": "fa_dkdv16.hip", "bwd_dq": "fa_dq16.hpp"}
COPY_BYTES = 1 << 30             # the plain copy used to calibrate the HBM byte counters


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(name: str) -> str:
    path = os.path.join(ROOT, "io_aware_exact_20_amd", "csrc", name)
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "io_aware_exact_20_amd", "csrc", "fa_device.hpp"),
              os.path.join(ROOT, "io_aware_exact_20_amd", "csrc", "fa_kernels.hpp")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def make_problem(fa, w, dev, with_bwd=True):
    q, k, v, do = workloads.draw(w, with_dout=with_bwd)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    do = do.to(dev) if do is not None else None
    return fa.Problem(q, k, v, do, scale=w.softmax_scale, causal=w.causal,
                      dropout_p=w.dropout_p, seed=w.dropout_seed)


def time_steps(prob, steps, warmup, with_bwd=True, per_step=False):
    """Wall time per step plus per-stage HIP-event times (ms, per launch);
    with per_step, also each step's event time (ms) in a list."""
    stages = [("fwd", prob.fwd)]
    if with_bwd:
        stages += [("bwd_prepare", prob.bwd_prepare), ("bwd_dkdv", prob.bwd_dkdv),
                   ("bwd_dq", prob.bwd_dq)]
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    per = {}
    for i, (name, _) in enumerate(stages):
        per[name] = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
    if per_step:
        return wall, per, [ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]
    return wall, per


def decode_line(fa, dev, B=1, H=32, N=16, Nk=65536, d=128, splits=16):
    """Long-context decoding: N query rows over Nk keys per head, one pass
    (B*H*ceil(N/256) workgroups) against the keys split into `splits`
    chunks; HIP-event times and the K+V bytes read per second."""
    w = workloads.Workload("decode", B, H, N, d, "bf16", causal=True, seed=6)
    q, k, v = (t.to(dev) for t in workloads.draw_cross(w, Nk))
    ws = torch.empty(max(fa.load().fa_fwd_splitkv_workspace_bytes(
        __import__("ctypes").byref(fa.make_params(B, H, N, d, fa.BF16, causal=True, Nk=Nk)),
        splits), 16), dtype=torch.uint8, device=dev)
    runs = {"one_pass": lambda: fa.fwd(q, k, v, causal=True),
            "split%d" % splits: lambda: fa.fwd_splitkv(q, k, v, splits, causal=True, workspace=ws)}
    out = {"B": B, "H": H, "N": N, "Nk": Nk, "d": d}
    kv_bytes = 2.0 * B * H * Nk * d * 2
    for name, fn in runs.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        out[name + "_ms"] = round(ms, 4)
        out[name + "_kv_GBs"] = round(kv_bytes / (ms * 1e-3) / 1e9, 1)
    return out


def fp8_lines(fa, dev):
    """The FP8 (e4m3) forward on the long causal shape (1 x 32 x N x 128,
    N = 4096 and 16384) and on the training shape without dropout
    (4 x 32 x 4096 x 128, causal): HIP-event time and TFLOP/s against the
    bf16 and the fp8 dense peaks."""
    out = {}
    for name, (B, H, N) in (("long_causal_4k", (1, 32, 4096)), ("long_causal_16k", (1, 32, 16384)),
                            ("train_shape", (4, 32, 4096))):
        w = workloads.Workload("fp8_" + name, B, H, N, 128, "bf16", causal=True, seed=4)
        args = [t.to(dev) for t in workloads.draw_fp8(w)]
        for _ in range(3):
            fa.fwd_fp8(*args, scale=w.softmax_scale, causal=True)
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fa.fwd_fp8(*args, scale=w.softmax_scale, causal=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = w.flops_fwd() / (ms * 1e-3) / 1e12
        out[name] = {"shape": "%dx%dx%dx128" % (B, H, N), "fwd_ms": round(ms, 4),
                     "fwd_tflops": round(tf, 2), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                     "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2)}
        del args
        torch.cuda.empty_cache()
    return out


def traffic_for(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _err(got, exact):
    """(max-abs, mean-abs) of a GPU tensor against a float64 array."""
    import numpy as np
    e = np.abs(got.detach().double().cpu().numpy() - exact)
    return float(e.max()), float(e.mean())


def oracle_heads(w, q, k, v, do, budget_s, outputs=None, max_heads=None):
    """The fp64 oracle over whole heads of workload w (forward, or forward +
    backward when do is given), head after head until budget_s seconds have
    been spent (at least one head).  Returns (heads done, seconds, errors):
    with `outputs` (the GPU's o, lse[, dq, dk, dv] of the same inputs), the
    max/mean-abs error of each on the heads done."""
    import numpy as np
    import oracle
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    if max_heads:
        heads = heads[:max_heads]
    p = float(np.float32(w.dropout_p))
    done, t_total = [], 0.0
    errs = {}
    names = ("O", "LSE", "dQ", "dK", "dV")
    while len(done) < len(heads) and (not done or t_total < budget_s):
        b, h = heads[len(done)]
        args = [x[b, h] for x in (q, k, v)]
        if do is not None:
            args = [oracle._f64(a) for a in args] + [oracle._f64(do[b, h])]
            t0 = time.perf_counter()
            dq, dk, dv, o, lse = oracle.bwd_one_head(*args, b, h, w.softmax_scale, w.causal, p,
                                                     w.dropout_seed)
            t_total += time.perf_counter() - t0
            exact = (o, lse, dq, dk, dv)
        else:
            t0 = time.perf_counter()
            o, lse = oracle.fwd_rows(q, k, v, b, h, range(w.N), w.softmax_scale, w.causal, p,
                                     w.dropout_seed)
            t_total += time.perf_counter() - t0
            exact = (o, lse)
        done.append((b, h))
        if outputs is not None:
            for nm, got, ex in zip(names, outputs, exact):
                mx, mn = _err(got[b, h], ex)
                cur = errs.setdefault(nm, [0.0, 0.0])
                cur[0] = max(cur[0], mx)
                cur[1] += mn
    for nm in errs:
        errs[nm] = {"max_abs": float("%.3e" % errs[nm][0]),
                    "mean_abs": float("%.3e" % (errs[nm][1] / len(done)))}
    return done, t_total, errs


def cpu_baseline(w, budget_s: float, outputs=None):
    """The fp64 oracle (forward + backward of whole heads of the same
    workload, each with its own (b, h) dropout counters) on the host cores
    for about `budget_s` seconds."""
    import oracle
    q, k, v, do = workloads.draw(w)
    f_head = w.flops_fwd() / (w.B * w.H) * 3.5
    done, t_total, errs = oracle_heads(w, q, k, v, do, budget_s, outputs)
    n = len(done)
    return {"value": f_head * n / t_total / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": "%d of %d heads (fwd+bwd, N=%d, d=%d, fp64), %.1f s; whole workload "
                      "extrapolated: %.1f s" % (n, w.B * w.H, w.N, w.d, t_total,
                                                t_total * w.B * w.H / n),
            "errors_on_sample": errs}


def config_table(fa, dev, budget_s=2.0):
    """Per target workload: GPU time and TFLOP/s (mean of HIP-event timed
    calls), % of the bf16 peak, the fp64 oracle's CPU time on sampled heads
    (extrapolated to the whole workload when sampled) and the GPU's
    max/mean-abs error per output against it on those heads."""
    import numpy as np
    import oracle
    rows = {}
    names = ["single_head_f32", "small_fwd_bf16", "small_fwd_bf16_causal", "mid_fwdbwd_causal",
             "long_causal_4k", "long_causal_16k", "long_causal_64k"]
    for name in names:
        w = workloads.WORKLOADS[name]
        q, k, v, do = workloads.draw(w)
        prob = fa.Problem(q.to(dev), k.to(dev), v.to(dev),
                          do.to(dev) if do is not None else None, scale=w.softmax_scale,
                          causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed)
        reps = 3 if w.N >= 65536 else 10
        wall, per = time_steps(prob, reps, 2, with_bwd=w.backward)
        gpu_ms = sum(per.values())
        F = w.flops_fwd() * (3.5 if w.backward else 1.0)
        row = {"shape": "%dx%dx%dx%d" % (w.B, w.H, w.N, w.d), "dtype": w.dtype,
               "causal": w.causal, "pass": "fwd+bwd" if w.backward else "fwd",
               "gpu_ms": round(gpu_ms, 4), "tflops": round(F / (gpu_ms * 1e-3) / 1e12, 2),
               "pct_peak": round(100 * F / (gpu_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        outs = (prob.o, prob.lse) + ((prob.dq, prob.dk, prob.dv) if w.backward else ())
        if w.N >= 65536:
            # one head is 1.1 TFLOP of fp64: time an evenly spaced sample of
            # its rows (a row's cost is proportional to its visible keys) and
            # scale by the flops of all rows of all heads
            rws = list(range(0, w.N, 64))
            t0 = time.perf_counter()
            eo, el = oracle.fwd_rows(q, k, v, 0, 0, rws, w.softmax_scale, w.causal)
            t = time.perf_counter() - t0
            keys = np.array([(r + 1) if w.causal else w.N for r in rws], dtype=np.float64)
            frac = keys.sum() / (w.N * (w.N + 1) / 2 if w.causal else w.N * w.N)
            row["oracle"] = {"seconds": round(t, 2), "cores": oracle.num_threads(),
                             "sample": "%d rows of head (0,0)" % len(rws),
                             "whole_workload_s_extrapolated": round(float(t / frac) * w.B * w.H, 1)}
            row["errors_on_sample"] = {nm: dict(zip(("max_abs", "mean_abs"),
                                                    [float("%.3e" % x) for x in _err(g[0, 0, rws], e)]))
                                       for nm, g, e in (("O", prob.o, eo), ("LSE", prob.lse, el))}
        else:
            done, t, errs = oracle_heads(w, q, k, v, do if w.backward else None, budget_s,
                                         outputs=outs)
            n, tot = len(done), w.B * w.H
            row["oracle"] = {"seconds": round(t, 3), "cores": oracle.num_threads(),
                             "sample": "%d of %d heads" % (n, tot),
                             ("whole_workload_s" if n == tot else "whole_workload_s_extrapolated"):
                                 round(t * tot / n, 2)}
            row["errors_on_sample"] = errs
        rows[name] = row
        log("config %s %s" % (name, row))
        del prob
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--no-extras", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--profile-workload", default=None, metavar="NAME",
                    help="only run --warmup + --steps steps of the named workload "
                         "(%s) and log per-stage times; for profiler runs.  'fp8:NAME' runs the "
                         "FP8 forward on that workload's shape (d = 128, no dropout)" % ", ".join(workloads.WORKLOADS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of %d bytes three times (the "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)" % COPY_BYTES)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes three times" % COPY_BYTES)
        return

    import io_aware_exact_20_amd as fa
    fa.load()
    if args.profile_workload and args.profile_workload.startswith("fp8:"):
        w0 = workloads.WORKLOADS[args.profile_workload[4:]]
        w = workloads.Workload("fp8_" + w0.name, w0.B, w0.H, w0.N, 128, "bf16", causal=w0.causal,
                               seed=w0.seed)
        xs = [t.to(dev) for t in workloads.draw_fp8(w)]
        for _ in range(args.warmup):
            fa.fwd_fp8(*xs, scale=w.softmax_scale, causal=w.causal)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fa.fwd_fp8(*xs, scale=w.softmax_scale, causal=w.causal)
        e1.record()
        torch.cuda.synchronize()
        log("workload %s: fp8 forward %.4f ms" % (w.name, e0.elapsed_time(e1) / max(1, args.steps)))
        return
    if args.profile_workload:
        w = workloads.WORKLOADS[args.profile_workload]
        prob = make_problem(fa, w, dev, with_bwd=w.backward)
        wall, per = time_steps(prob, args.steps, args.warmup, with_bwd=w.backward)
        log("workload %s: step %.3f ms; stages %s" % (w.name, wall, per))
        return
    w = workloads.WORKLOADS["train_dropout"]
    F = w.flops_fwd()
    log("workload %s: B=%d H=%d N=%d d=%d causal p=%g" % (w.name, w.B, w.H, w.N, w.d, w.dropout_p))
    prob = make_problem(fa, w, dev)
    wall, per, steps_ms = time_steps(prob, args.steps, args.warmup, per_step=True)
    value = 3.5 * F / (wall * 1e-3) / 1e12
    steps_sorted = sorted(steps_ms)
    median_ms = (steps_sorted[(len(steps_sorted) - 1) // 2] + steps_sorted[len(steps_sorted) // 2]) / 2
    log("step %.3f ms  -> %.1f TFLOP/s; stages %s" % (wall, value, per))

    # Algorithmic flops credited to each kernel: the forward's two products;
    # the backward's five (S recompute, dP, dV, dK, dQ) split as the dK/dV
    # kernel's four and the dQ kernel's one -- its own S and dP recompute is
    # extra work of this design and is not credited.
    flops_per_launch = {"fwd": F, "bwd_dkdv": 2.0 * F, "bwd_dq": 0.5 * F}
    dominant = max(flops_per_launch, key=lambda k: per[k])
    bwd_ms = per["bwd_prepare"] + per["bwd_dkdv"] + per["bwd_dq"]
    achieved = flops_per_launch[dominant] / (per[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dominant),
                "traffic_source": "profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE "
                                  "per launch, copy-calibrated, taken on the kernel source "
                                  "whose hash it records (null when the source has changed)",
                "avg_launch_ms": round(per[dominant], 4)}

    extras = {
        "step_ms": {"mean_wall": round(wall, 4), "median_event": round(median_ms, 4),
                    "min_event": round(steps_sorted[0], 4), "max_event": round(steps_sorted[-1], 4)},
        "value_at_median_tflops": round(3.5 * F / (median_ms * 1e-3) / 1e12, 2),
        "value_at_min_tflops": round(3.5 * F / (steps_sorted[0] * 1e-3) / 1e12, 2),
        "fwd_tflops": round(F / (per["fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(2.5 * F / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in per.items()},
    }
    extras["fwd_pct_peak"] = round(100 * extras["fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    extras["bwd_pct_peak"] = round(100 * extras["bwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    # the headline's outputs (last timed step) for the oracle comparison below
    head_outputs = tuple(t.cpu() for t in (prob.o, prob.lse, prob.dq, prob.dk, prob.dv))
    del prob
    torch.cuda.empty_cache()

    if not args.no_extras:
        # Same shape without dropout (the dropout overhead), the long-context
        # forward at N=4096, and the mid-size training shape.
        w0 = workloads.Workload("train_nodropout", w.B, w.H, w.N, w.d, "bf16", causal=True,
                                backward=True, seed=w.seed)
        p0 = make_problem(fa, w0, dev)
        wall0, per0 = time_steps(p0, max(5, args.steps // 2), 2)
        extras["p0_fwd_tflops"] = round(F / (per0["fwd"] * 1e-3) / 1e12, 2)
        extras["p0_bwd_tflops"] = round(2.5 * F / ((per0["bwd_prepare"] + per0["bwd_dkdv"]
                                                    + per0["bwd_dq"]) * 1e-3) / 1e12, 2)
        extras["p0_fwdbwd_tflops"] = round(3.5 * F / (wall0 * 1e-3) / 1e12, 2)
        del p0
        # Long-context causal forward, N swept over 4096, 16384, 65536: per-N
        # throughput and the HBM the call adds (only O and LSE; the library
        # allocates nothing, so the allocator's peak does not move during it).
        longs = {}
        for name in ("long_causal_4k", "long_causal_16k", "long_causal_64k"):
            wl = workloads.WORKLOADS[name]
            before = torch.cuda.memory_allocated()
            pl = make_problem(fa, wl, dev, with_bwd=False)
            out_bytes = pl.o.numel() * pl.o.element_size() + pl.lse.numel() * 4
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            peak0 = torch.cuda.max_memory_allocated()
            reps = 10 if wl.N <= 16384 else 3
            _, perl = time_steps(pl, reps, 2, with_bwd=False)
            longs[str(wl.N)] = {
                "fwd_tflops": round(wl.flops_fwd() / (perl["fwd"] * 1e-3) / 1e12, 2),
                "fwd_ms": round(perl["fwd"], 4),
                "out_bytes": out_bytes,
                "allocated_during_call": torch.cuda.max_memory_allocated() - peak0,
                "score_matrix_bytes": workloads.score_matrix_bytes(wl.N, wl.B * wl.H),
                "inputs_bytes": torch.cuda.memory_allocated() - before - out_bytes,
            }
            del pl
            torch.cuda.empty_cache()
        extras["long_causal"] = longs
        extras["long4k_fwd_tflops"] = longs["4096"]["fwd_tflops"]
        extras["long4k_fwd_pct_peak"] = round(100 * extras["long4k_fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
        # Small forward (2 x 8 x 1024 x 64), non-causal and causal.
        small = {}
        for name in ("small_fwd_bf16", "small_fwd_bf16_causal"):
            ws_ = workloads.WORKLOADS[name]
            ps = make_problem(fa, ws_, dev, with_bwd=False)
            _, pers = time_steps(ps, 20, 3, with_bwd=False)
            small[name] = {"fwd_tflops": round(ws_.flops_fwd() / (pers["fwd"] * 1e-3) / 1e12, 2),
                           "fwd_ms": round(pers["fwd"], 4)}
            del ps
        extras["small_fwd"] = small
        w3 = workloads.WORKLOADS["mid_fwdbwd_causal"]
        p3 = make_problem(fa, w3, dev)
        wall3, _ = time_steps(p3, max(5, args.steps // 2), 2)
        extras["mid_fwdbwd_tflops"] = round(3.5 * w3.flops_fwd() / (wall3 * 1e-3) / 1e12, 2)
        del p3
        torch.cuda.empty_cache()
        # The training shape at the other head dimensions (generic kernels).
        hd = {}
        for d in (32, 64, 96, 256):
            wd = workloads.WORKLOADS["train_d%d" % d]
            pd = make_problem(fa, wd, dev)
            walld, perd = time_steps(pd, 3, 1)
            Fd = wd.flops_fwd()
            hd[str(d)] = {"fwd_tflops": round(Fd / (perd["fwd"] * 1e-3) / 1e12, 2),
                          "fwdbwd_tflops": round(3.5 * Fd / (walld * 1e-3) / 1e12, 2)}
            del pd
            torch.cuda.empty_cache()
        extras["head_dims"] = hd
        extras["decode"] = decode_line(fa, dev)
        extras["fp8_fwd"] = fp8_lines(fa, dev)
        log("extras %s" % extras)

    cpu = cpu_baseline(w, args.cpu_seconds, head_outputs) if args.cpu_seconds > 0 else None
    if cpu:
        log("cpu baseline %s" % cpu)
    if not args.no_extras and args.cpu_seconds > 0:
        # every other target workload: GPU throughput, oracle CPU time and error
        extras["configs"] = config_table(fa, dev, budget_s=2.0)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True,
                   "dropout_p": w.dropout_p, "pass": "fwd+bwd",
                   "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
