#!/usr/bin/env python3
"""Throughput of the INT8 convrot linear on one MI355X.

One step is one pass of the whole hot path over one batch: the rotate +
row-max + quantize + pack kernel over X, then the INT8 MFMA contraction with
the fused reconstruction (scale, weight scale, unscale, bias, output cast).
These are the two launches the fused entry convrot_int8_linear makes; the
benchmark issues them as convrot_quantize_rows + int8_linear, the same
kernels.  For the shared QKV workload a step is one convrot_int8_linear_shared
call.  After the timed steps each kernel is timed on its own (K back-to-back
launches between two HIP events) for the roofline figures.

Warm-up is W steps and at least --warmup-ms of wall time: a GPU that starts
from idle runs these kernels boosted for about 2 ms, then throttles below its
power-limited steady state and recovers over some 20 ms (kernel traces show the
GEMM at 150, then 200, then 150 us), and the timed steps are meant to see the
steady state.

Inputs are seeded synthetic DiT-shaped tensors (workloads.py), resident in
HBM before timing starts.  Several input sets are rotated across steps so that
the activations of a step are not still held in the 256 MiB Infinity Cache
from an earlier step.  Weights are rotated and quantized on the GPU by the
same library (convrot_quantize_rows on W) before timing.

Prints one JSON line.  --gpus above 1 is refused: this build runs on a single
GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s
MALL_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "gemm": os.path.join(ROOT, "int8_hadamard_rotated_amd", "csrc", "gemm_i8.hip"),
    "quantize": os.path.join(ROOT, "int8_hadamard_rotated_amd", "csrc", "quantize.hip"),
}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def quantize_bytes(w: workloads.Workload, n_scales: int = 1) -> int:
    """Algorithmic bytes of the quantization of one step: read X once (and
    the producer's inputs, if any: the gated activation's second tensor, the
    normalization weight, the Modulate scale and shift), write the packed tensor of
    each of the n_scales input scales."""
    esz = 2 if w.x_dtype == workloads.BF16 else 4
    m_pad = (w.M + 3) // 4 * 4
    mod = (8 * w.K if w.modulate else 0) + (4 * w.K if w.rmsnorm or w.norm else 0)
    up = w.M * w.K * esz if w.glu else 0
    return w.M * w.K * esz + up + n_scales * (m_pad * w.K + 4 * m_pad) + mod


def gemm_ops(w: workloads.Workload, n_linears: int) -> int:
    return 2 * w.M * w.N * w.K * n_linears


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the
    kernel source still matches the one that was profiled."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kind]):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_means(path: str, counter: str) -> dict:
    """Mean per-dispatch value (KiB) of one counter, by kernel kind."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            kind = ("gemm" if "gemm_i8_kernel" in name else
                    "quantize" if "quantize_rows" in name else
                    "copy" if "elementwise" in name and "neg" in name else None)
            if kind is not None:
                vals.setdefault((kind, name), []).append(float(r["Counter_Value"]))
    return vals


def write_traffic(w: workloads.Workload, fetch_csv: str, write_csv: str, copy_mib: int) -> int:
    """HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    each scaled by the ratio of the bytes a plain copy of copy_mib MiB moves
    to what the same counter reads for that copy.  Per kernel, the median
    over the dispatches of its most frequent instantiation (which outvotes
    the single quantizer launch that prepares the weights)."""
    if not copy_mib:
        print("--traffic needs the --copy-mib the counter runs used", file=sys.stderr)
        return 2
    known = copy_mib << 20
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _counter_means(path, counter)
        copies = [v for (kind, _), vs in vals.items() if kind == "copy" for v in vs]
        if not copies:
            print(f"no copy kernel in {path}", file=sys.stderr)
            return 1
        copy_kib = float(np.median(copies[-3:]))
        scale = known / (copy_kib * 1024.0)
        for kind in ("gemm", "quantize"):
            inst = [(len(vs), name, vs) for (k, name), vs in vals.items() if k == kind]
            if not inst:
                continue
            _, name, vs = max(inst)
            rec = out.setdefault(kind, {"workload": w.name, "kernel": name,
                                        "source_sha256_16": source_hash(KERNEL_SOURCES[kind])})
            key = "fetch" if counter == "FETCH_SIZE" else "write"
            rec[f"{key}_kib_per_dispatch"] = round(float(np.median(vs)), 1)
            rec[f"{key}_copy_kib"] = round(copy_kib, 1)
            rec[f"{key}_scale"] = round(scale, 4)
            rec[f"{key}_bytes"] = int(float(np.median(vs)) * 1024.0 * scale)
    for kind, rec in out.items():
        rec["hbm_bytes_per_launch"] = rec.get("fetch_bytes", 0) + rec.get("write_bytes", 0)
        path = os.path.join(PROFILE_DIR, f"traffic_{kind}_{w.name}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(path, json.dumps(rec))
    return 0


def to_dev_x(X: np.ndarray, torch):
    if X.dtype == np.uint16:
        return torch.from_numpy(X.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(X).to("cuda:0")


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads for the oracle: the job's CPU share when the environment states
    it (OMP_NUM_THREADS), else every core this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w: workloads.Workload, inp: workloads.Inputs, rows: int) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    the full layer (producer if any, quantize, int32 contraction,
    reconstruction) for the first `rows` rows of X against the full weight
    matrix, each phase timed on its own."""
    import oracle
    threads = host_threads()
    o = oracle.get()
    if w.w_bits == 4:                                                # untimed
        Qw, sw = o.unpack_int4(inp.W[0], w.K), inp.s_w[0]
    else:
        Qw, sw = o.weight_prep(inp.W[0], w.G, threads=threads)
    Qu = su = None
    if w.swiglu:
        Qu, su = o.weight_prep(inp.W[1], w.G, threads=threads)      # untimed
    yd = oracle.BF16 if w.y_dtype == workloads.BF16 else oracle.F32
    X = np.ascontiguousarray(inp.X[:rows])
    alpha = w.input_scales[0]
    t = {}
    t0 = time.perf_counter()
    if w.glu:
        X = o.gated_act_rows(X, np.ascontiguousarray(inp.up[:rows]), w.glu, threads=threads)
    if w.rmsnorm:
        X = o.rmsnorm_rows(X, w.rms_eps, inp.norm_weight, threads=threads)
    if w.norm:
        X = o.norm_rows(X, w.rms_eps, inp.norm_weight, threads=threads)
    if w.modulate:
        X = o.modulate_rows(X, inp.mod_scale, inp.mod_shift, threads=threads)
    t1 = time.perf_counter()
    pk = o.quantize_rows(X, w.G, alpha, threads=threads)
    t2 = time.perf_counter()
    A = o.gemm_i32(pk.q, Qw, threads=threads)
    Au = o.gemm_i32(pk.q, Qu, threads=threads) if w.swiglu else None
    t3 = time.perf_counter()
    if w.swiglu:
        Yg = o.epilogue(A, pk.s, sw, None, alpha, oracle.F32, threads=threads)
        Yu = o.epilogue(Au, pk.s, su, None, alpha, oracle.F32, threads=threads)
        o.gated_act_rows(Yg, Yu, oracle.ACT_SILU, threads=threads)
    elif w.gated:
        Yf = o.epilogue(A, pk.s, sw, inp.b[0], alpha, oracle.F32, threads=threads)
        o.gated_residual(Yf, inp.gate, np.ascontiguousarray(inp.residual[:rows]), 1.0, yd,
                         threads=threads)
    else:
        o.epilogue(A, pk.s, sw, inp.b[0], alpha, yd, threads=threads)
    t4 = time.perf_counter()
    dt = t4 - t0
    n_lin = 2 if w.swiglu else 1
    ops = 2 * rows * w.N * w.K * n_lin
    esz = 2 if w.x_dtype == workloads.BF16 else 4
    m_pad = (rows + 3) // 4 * 4
    q_bytes = rows * w.K * esz + m_pad * w.K + 4 * m_pad
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {w.M} rows of {w.name} ({'gated activation + ' if w.glu else ''}"
                      f"{'RMSNorm + ' if w.rmsnorm else ''}"
                      f"{'Norm + ' if w.norm else ''}"
                      f"{'modulate + ' if w.modulate else ''}"
                      f"quantize + int32 GEMM + reconstruction{' + gated residual' if w.gated else ''}"
                      f"{' for the gate and up weights + SwiGLU' if w.swiglu else ''} "
                      f"against all {w.N}x{w.K} weights), {dt:.2f} s",
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
            "threads_note": "OpenMP threads = OMP_NUM_THREADS when set (the job's CPU share), "
                            "else the cores this process may run on",
            "phases_s": {"producer": round(t1 - t0, 4), "quantize": round(t2 - t1, 4),
                         "gemm_i32": round(t3 - t2, 4), "reconstruction": round(t4 - t3, 4)},
            "quantize_gbs": round(q_bytes / (t2 - t1) / 1e9, 3),
            "gemm_gops": round(ops / (t3 - t2) / 1e9, 3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="after the W warm-up steps, keep stepping (untimed) until this much "
                         "wall time has passed since the warm-up began: a GPU that starts "
                         "from idle boosts for about 2 ms, then throttles below its "
                         "power-limited steady state and takes some 20 ms to recover, so "
                         "timed steps that begin earlier measure that transient")
    ap.add_argument("--workload", default="mlp_up", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated over steps (0: enough to exceed the Infinity Cache)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of X in the CPU oracle sample (0: all of them, one whole step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the MFMA-rate probe (the contraction's power-limited ceiling)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, pass a float32 tensor of this many MiB three times "
                         "through torch.neg (a plain copy kernel of known size that calibrates "
                         "the HBM byte counters)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter_collection CSVs of a FETCH_SIZE and a "
                         "WRITE_SIZE rocprofv3 run of this benchmark (with --copy-mib) into "
                         "profiles/traffic_<kernel>_<workload>.json")
    args = ap.parse_args()
    if args.traffic:
        return write_traffic(workloads.WORKLOADS[args.workload], args.traffic[0],
                             args.traffic[1], args.copy_mib)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the INT8 convrot linear is benchmarked on a "
              "single MI355X (rows shard across GPUs with no exchange); --gpus must be 1",
              file=sys.stderr)
        return 2

    import torch
    import int8_hadamard_rotated_amd as cr

    w = workloads.WORKLOADS[args.workload]
    inp = workloads.make_inputs(w)
    dev = "cuda:0"
    torch.cuda.set_device(0)

    # weights: rotated + quantized on the GPU by the library's own quantizer
    # (4-bit weights are drawn already packed, with their scales)
    lins = []
    for j, (W, b, a) in enumerate(zip(inp.W, inp.b, w.input_scales)):
        if w.w_bits == 4:
            lins.append(dict(Qw=torch.from_numpy(W).to(dev), s_w=torch.from_numpy(inp.s_w[j]).to(dev),
                             bias=torch.from_numpy(b).to(dev), input_scale=a))
            continue
        Wd = torch.from_numpy(W).to(dev)
        packed = cr.convrot_quantize_rows(Wd, w.G)
        Qw, sw = cr.packed_parts(packed, w.N, w.K)
        lins.append(dict(Qw=Qw[: w.N].contiguous(), s_w=sw[: w.N].contiguous(),
                         bias=torch.from_numpy(b).to(dev), input_scale=a))
        del Wd, packed
    torch.cuda.synchronize()

    yd = cr.BF16 if w.y_dtype == workloads.BF16 else cr.F32
    ybytes = 2 if yd == cr.BF16 else 4
    shared = w.n_linears > 1 and not w.swiglu
    scales = sorted(set(w.input_scales), key=w.input_scales.index)   # one pass per distinct scale
    n_packed = len(scales)
    w_bytes = sum(l["Qw"].numel() + 8 * w.N for l in lins)
    set_bytes = (inp.X.nbytes * (2 if w.glu else 1) + cr.convrot_workspace_bytes(w.M, w.K, n_packed)
                 + w.n_linears * w.M * w.N * ybytes + w_bytes)
    n_sets = args.sets or max(1, min(8, math.ceil(2 * MALL_BYTES / set_bytes)))
    # Every input set has its own activations, packed tensors, outputs and a
    # copy of the weights (same values), so that nothing a step reads is
    # still in the 256 MiB Infinity Cache from the step before.
    sets = []
    for s in range(n_sets):
        extra = inp if s == 0 else workloads.make_inputs(w, seed=w.seed + 1000 * s)
        Xd = to_dev_x(extra.X, torch)
        up = to_dev_x(extra.up, torch) if w.glu else None
        ws = torch.empty(cr.convrot_workspace_bytes(w.M, w.K, n_packed), dtype=torch.uint8,
                         device=dev)
        Ys = [torch.empty((w.M, w.N), dtype=torch.bfloat16 if yd == cr.BF16 else torch.float32,
                          device=dev) for _ in range(w.n_linears)]
        if w.gated:                  # the output starts as the residual (updated in place)
            Ys[0].copy_(to_dev_x(inp.residual, torch))
        ls = lins if s == 0 else [dict(l, Qw=l["Qw"].clone(), s_w=l["s_w"].clone(),
                                       bias=l["bias"].clone()) for l in lins]
        slot = cr.convrot_workspace_bytes(w.M, w.K, 1)
        views = [cr.packed_parts(ws[k * slot:(k + 1) * slot], w.M, w.K) for k in range(n_packed)]
        # each linear with its output and, past the first scale, the packed
        # tensor of its own input scale
        calls = []
        for l, Y in zip(ls, Ys):
            c = dict(l, Y=Y)
            k = scales.index(l["input_scale"])
            if k:
                c["Qx"], c["s_x"] = views[k]
            calls.append(c)
        slots = [ws[k * slot:(k + 1) * slot] for k in range(n_packed)]
        sets.append(dict(X=Xd, up=up, ws=ws, Y=Ys, lins=ls, views=views, calls=calls, slots=slots))
    torch.cuda.synchronize()

    mod = (cr.Modulate(torch.from_numpy(inp.mod_scale).to(dev), torch.from_numpy(inp.mod_shift).to(dev))
           if w.modulate else None)
    if w.rmsnorm:
        mod = cr.RMSNormModulate(w.rms_eps, torch.from_numpy(inp.norm_weight).to(dev),
                                 mod.scale if mod else None, mod.shift if mod else None)
    if w.norm:
        mod = cr.NormMul(w.rms_eps, torch.from_numpy(inp.norm_weight).to(dev))
    gate = torch.from_numpy(inp.gate).to(dev) if w.gated else None
    slot = cr.convrot_workspace_bytes(w.M, w.K, 1)

    def quantize(i):
        """The step's quantization: one pass per input scale (plain rows of
        several scales in one call, which reads binary32 X once)."""
        S = sets[i % n_sets]
        if n_packed > 1 and mod is None and not w.glu:
            cr.convrot_quantize_rows_scales(S["X"], w.G, scales, packed=S["slots"])
            return
        for k in range(n_packed):
            ws = S["slots"][k]
            if w.glu:
                cr.convrot_quantize_rows_pre(S["X"], cr.GatedAct(S["up"], w.glu), w.G, scales[k], packed=ws)
            elif mod is not None:
                cr.convrot_quantize_rows_pre(S["X"], mod, w.G, scales[k], packed=ws)
            else:
                cr.convrot_quantize_rows(S["X"], w.G, scales[k], packed=ws)

    def gemm(i):
        """The step's GEMM launch: every linear, each reading the packed tensor
        of its input scale (one grouped launch when there are several)."""
        S = sets[i % n_sets]
        qx, sx = S["views"][0]
        ls = S["calls"]
        l = ls[0]
        if w.gated:
            cr.int8_linear_post(qx, sx, l["Qw"], l["s_w"], l["bias"], l["input_scale"],
                                cr.GatedResidual(gate, l["Y"]), Y=l["Y"], M=w.M)
        elif w.swiglu:
            u = dict(S["lins"][1], Y=S["Y"][1])
            cr.int8_swiglu_linear(qx, sx, l["Qw"], l["s_w"], u["Qw"], u["s_w"], l["input_scale"],
                                  Y=l["Y"], M=w.M)
        elif len(ls) > 1:
            cr.int8_linear_grouped(qx, sx, ls, M=w.M)
        else:
            lin_fn = cr.int4_linear if w.w_bits == 4 else cr.int8_linear
            lin_fn(qx, sx, l["Qw"], l["s_w"], l["bias"], l["input_scale"], Y=l["Y"], M=w.M)

    def step(i):
        # the quantization of every distinct input scale, then one GEMM launch
        # over every linear (the launches of the shared entry, without folding
        # a power-of-two scale into the alpha = 1 pass)
        quantize(i)
        gemm(i)

    def step_folded(i):
        S = sets[i % n_sets]
        cr.convrot_int8_linear_shared_pre(
            S["X"], mod, w.G, [dict(l, Y=Y) for l, Y in zip(S["lins"], S["Y"])], workspace=S["ws"])

    stream = torch.cuda.current_stream()

    def warm(fn):
        t_warm = time.perf_counter()
        for i in range(args.warmup):
            fn(i)
        n = args.warmup
        torch.cuda.synchronize()
        while (time.perf_counter() - t_warm) * 1e3 < args.warmup_ms:
            for _ in range(16):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return n

    def timed(fn, n):
        """Wall time and HIP-event time of n calls (events only at the two ends:
        an event recorded between kernels leaves the GPU idle a few us)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3

    warm_steps = warm(step)
    wall, ev = timed(step, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    ev_step_us = ev * 1e6 / args.steps

    def kernel_us(fn):
        """Average duration of one kernel: K launches of it back to back (same
        input rotation as the steps) between two HIP events on its stream."""
        return timed(fn, args.steps)[1] * 1e6 / args.steps

    def kernel_spread(fn, n=100):
        """p10 / median / p90 of single launches, each between its own pair of
        HIP events (the GPU idles for a few microseconds between them)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        return {"launches": n, "p10": round(float(np.percentile(us, 10)), 3),
                "median": round(float(np.median(us)), 3), "p90": round(float(np.percentile(us, 90)), 3)}

    ops = gemm_ops(w, w.n_linears)
    rec = {
        "metric": "int8 linear TOPS + quantize GB/s (fraction of MI355X roofline), M=4096 K=3072",
        "value": round(ops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if w.w_bits == 8 else "i8 x i4",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: X {w.x_dtype} [{w.M},{w.K}], W {'i4' if w.w_bits == 4 else 'i8'} [{w.N},{w.K}] x "
                               f"{w.n_linears}, G={w.G}, Y {w.y_dtype}, input scales "
                               f"{list(w.input_scales)}"
                               + (", SiLU(X) * up fused" if w.glu == 1 else ", Sigmoid(X) * up fused" if w.glu else "")
                               + (", one dual GEMM with the SwiGLU epilogue (gate, up)" if w.swiglu else "")
                               + (", RMSNorm -> Mul(weight) fused" if w.rmsnorm else "")
                               + (", Norm -> Mul(weight) fused" if w.norm else "")
                               + (", Modulate producer fused" if w.modulate else "")
                               + (", gated residual in place" if w.gated else ""),
                   "M": w.M, "K": w.K, "N": w.N, "G": w.G, "x_dtype": w.x_dtype,
                   "y_dtype": w.y_dtype, "linears": w.n_linears, "input_sets": n_sets,
                   "cold": "every set has its own X, packed tensors, Y and weight copy; "
                           f"{n_sets} sets of {set_bytes / 2**20:.0f} MiB rotate past the "
                           "256 MiB Infinity Cache"},
        "step_us_events": round(ev_step_us, 3),
    }
    # per-kernel figures: the step's quantization (for qkv: one pass for both
    # input scales) and the step's GEMM launch (for qkv: the grouped launch of
    # all four linears over both packed tensors), each launched K times back
    # to back
    tq = kernel_us(quantize) * 1e-6
    tg = kernel_us(gemm) * 1e-6
    g_ops = gemm_ops(w, 2 if w.swiglu else w.n_linears)
    q_bytes = quantize_bytes(w, n_packed)
    q_gbs = q_bytes / tq / 1e9
    g_tops = g_ops / tg / 1e12
    rec["quantize"] = {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                       "us": round(tq * 1e6, 3), "bytes": q_bytes,
                       "traffic": measured_traffic("quantize", w.name),
                       "single_launch_us": kernel_spread(quantize)}
    rec["roofline"] = {"bound": "mfma", "achieved": round(g_tops, 1), "peak": INT8_PEAK_TOPS,
                       "unit": "TOPS", "frac": round(g_tops / INT8_PEAK_TOPS, 4),
                       "traffic": measured_traffic("gemm", w.name),
                       "kernel": "gemm_i8 (contraction + fused reconstruction)"
                                 + (f", one grouped launch of {w.n_linears} linears" if shared else "")
                                 + (f" reading {n_packed} packed tensors (input scales {scales})"
                                    if n_packed > 1 else ""),
                       "ops": g_ops, "us": round(tg * 1e6, 3),
                       "note": "int8 ops: one multiply-add counts as 2",
                       "single_launch_us": kernel_spread(gemm)}
    if n_packed > 1:
        rec["quantize"]["scales"] = (
            f"input scales {scales}: one convrot_quantize_rows_scales call writes a packed tensor "
            "for each, reading X once; bytes count X once and every packed tensor")
    # the quantize pass against a plain copy of the same bytes: the probe
    # kernel reads X ([M, K], bf16 or binary32) with 16-byte loads and writes
    # one byte per element with 16-byte stores, no arithmetic, back to back
    # over the same input sets
    if not w.glu and not args.no_probe and n_packed == 1:
        probe = probe_library()
        esz = 2 if w.x_dtype == workloads.BF16 else 4
        dst = torch.empty((w.M, w.K), dtype=torch.int8, device=dev)

        def copy(i):
            rc = probe.convrot_probe_copy(sets[i % n_sets]["X"].data_ptr(), esz, w.M * w.K,
                                          dst.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"convrot_probe_copy: hip error {rc}")
        copy(0)
        tc = kernel_us(copy) * 1e-6
        cbytes = w.M * w.K * (esz + 1)
        rec["quantize"]["copy_ceiling"] = {
            "what": "probe kernel: the same read of X and write of M x K bytes, 16-byte loads and "
                    "stores, no arithmetic",
            "us": round(tc * 1e6, 3), "gbs": round(cbytes / tc / 1e9, 1),
            "frac": round(cbytes / tc / 1e9 / HBM_PEAK_GBS, 4),
            "quantize_vs_copy": round(tc / tq, 4)}
    # the MFMA rate on these codes with no data movement (the power-limited
    # ceiling of the contraction), in the GEMM's wave shape and occupancy
    if w.w_bits == 8 and not args.no_probe:
        rec["roofline"]["mfma_ceiling"] = mfma_ceiling(cr, torch, sets[0]["views"][0][0],
                                                       sets[0]["lins"][0]["Qw"], g_tops)
    # the vendor library's int8 GEMM on the same operands, for reference: one
    # linear's contraction alone (int32 output, no reconstruction), back to
    # back over the same input sets
    if w.w_bits == 8 and not w.swiglu and not args.no_probe and w.M > 16 and w.N % 8 == 0:
        rec["roofline"]["library_gemm"] = library_gemm(torch, sets, w, args.steps, kernel_us)
    if shared:
        warm(step_folded)
        wall_f, _ = timed(step_folded, args.steps)
        ms_f = wall_f * 1e3 / args.steps
        rec["extension"] = {
            "what": "the same step through convrot_int8_linear_shared, which folds the power-of-two "
                    "input scale into the alpha = 1 pass (one quantize pass, one grouped GEMM launch "
                    "of all linears; an extension beyond the pages)",
            "ms_per_step": round(ms_f, 5), "value": round(ops / (ms_f * 1e-3) / 1e12, 3),
            "unit": "TOPS"}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_rows or w.M)
    print(json.dumps(rec), flush=True)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # one read and one write of each element
        torch.cuda.synchronize()
    return 0


_PROBE = None


def probe_library():
    """libconvrot_probe.so: the measurement kernels (MFMA rate, plain copy)."""
    global _PROBE
    if _PROBE is None:
        from int8_hadamard_rotated_amd import _build
        lib = ctypes.CDLL(_build.PROBE_LIBRARY)
        lib.convrot_probe_mfma.restype = ctypes.c_int
        lib.convrot_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
        lib.convrot_probe_copy.restype = ctypes.c_int
        lib.convrot_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p]
        _PROBE = lib
    return _PROBE


def library_gemm(torch, sets, w, steps: int, kernel_us) -> dict:
    """torch._int_mm (hipBLASLt on ROCm) on the first linear's operands: Q_x
    [M, K] times Q_w^T, int32 out.  Not part of the path: a reference for the
    contraction alone."""
    outs = [torch.empty((w.M, w.N), dtype=torch.int32, device=S["Y"][0].device) for S in sets]

    def run(i):
        S = sets[i % len(sets)]
        torch._int_mm(S["views"][0][0][:w.M], S["lins"][0]["Qw"].t(), out=outs[i % len(sets)])
    run(0)
    torch.cuda.synchronize()
    us = kernel_us(run)
    ops = 2 * w.M * w.N * w.K
    return {"what": "torch._int_mm (hipBLASLt) on the first linear's Q_x and Q_w: int32 output, no "
                    "reconstruction, back to back",
            "us": round(us, 3), "achieved": round(ops / us / 1e6, 1),
            "frac": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)}


def mfma_ceiling(cr, torch, qx, qw, gemm_tops: float) -> dict:
    """Run the probe kernel (libconvrot_probe.so) on the workload's own codes:
    256 workgroups of 8 waves (one per CU), each wave 32 MFMAs per step on
    register-resident fragments, long enough to reach the power-limited clock."""
    lib = probe_library()
    blocks, steps = 256, 2048
    out = torch.empty(blocks * 512, dtype=torch.int32, device=qx.device)
    stream = torch.cuda.current_stream()

    def run():
        rc = lib.convrot_probe_mfma(qx.data_ptr(), qx.numel(), qw.data_ptr(), qw.numel(), steps,
                                    blocks, out.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"convrot_probe_mfma: hip error {rc}")

    for _ in range(20):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record(stream)
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / n
    ops = blocks * 8 * steps * 32 * (2 * 16 * 16 * 64)
    tops = ops / t / 1e12
    return {"what": "probe: the GEMM's wave shape and occupancy (8 waves, one workgroup per CU), "
                    "32 MFMAs per step on fragments of this workload's codes held in registers, no "
                    "loads, LDS traffic or barriers",
            "achieved": round(tops, 1), "frac": round(tops / INT8_PEAK_TOPS, 4),
            "us": round(t * 1e6, 2), "gemm_of_ceiling": round(gemm_tops / tops, 4)}


if __name__ == "__main__":
    sys.exit(main())
