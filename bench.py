"""Throughput of the chunkwise key-only GLA forward on one MI355X.

One step = one pass of the whole hot path over one batch: every call of the
workload (for the 640 px frame: one call per scan direction L2R, R2L, T2B,
B2T), each call doing gate stage, intra/inter-chunk products, state carry,
direction remap and epilogue.  Inputs are resident in HBM before the timed
region; enough distinct input sets rotate through the steps that the 256 MB
last-level cache cannot serve them.  Steps are replayed from HIP graphs and
timed with HIP events on the stream they run on.

Prints one JSON line (metric, value in Gtok*head/s, roofline of the forward
call, CPU-oracle baseline on a bounded sample).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunkwise GLA fwd: µs/call + Gtok·head/s at L=1600; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3  # dense binary32 matrix-core peak
MALL_BYTES = 256 << 20     # last-level (Infinity) cache


def algorithmic_bytes_per_token_head(dk, dv, es, gated, gate_proj=None, heads=1):
    """Compulsory HBM traffic: q, k, v, z (fp32) read, out written, r read if
    gated.  With the gate projection, x (d_model values per token, shared by
    the heads) is read in place of z."""
    gate_in = 4 * dk if gate_proj is None else es * gate_proj["d_model"] / heads
    return es * (2 * dk + dv) + gate_in + es * dv + (es * dv if gated else 0)


def weight_bytes_per_call(spec, es):
    """Per-call parameters: RMSNorm weight if gated, projection weights."""
    n = 4 * spec["dv"] if spec["gated"] else 0
    gp = spec.get("gate_proj")
    if gp:
        nout = spec["NH"] * spec["dk"]
        n += es * gp["rank"] * gp["d_model"] + 4 * nout * gp["rank"] + 4 * nout
    return n


def algorithmic_flops_per_token_head(dk, dv, chunk):
    """Chunkwise causal form: intra-chunk scores and values (dk+dv)(C+1), inter
    output and state update 4 dk dv (multiply-add = 2 flops)."""
    return (dk + dv) * (chunk + 1) + 4 * dk * dv


# Sources each kernel family is built from (its own file and the headers it
# includes); the traffic of a workload is tied to these only.
_COMMON_SOURCES = ("gla_device.h", "gla_launch.h", "gla_geometry.h")
KERNEL_SOURCES = {
    "onepass": ("gla_onepass.hip",) + _COMMON_SOURCES,
    "onepass_proj": ("gla_onepass.hip", "gla_proj.hip") + _COMMON_SOURCES,
    "wide": ("gla_wide.hip", "gla_kernel.hip", "gla_chunk.h") + _COMMON_SOURCES,
    "generic": ("gla_kernel.hip", "gla_chunk.h", "gla_chunk_f16.hip", "gla_chunk_f32.hip",
                "gla_chunk_f16_mixed.hip", "gla_chunk_f32_mixed.hip") + _COMMON_SOURCES,
    "sswiglu": ("gla_sswiglu.hip",) + _COMMON_SOURCES,
    "bwd": ("gla_bwd.hip", "gla_epi.h") + _COMMON_SOURCES,
    "bwd_gated": ("gla_bwd.hip", "gla_epi.h") + _COMMON_SOURCES,
    "proj_bwd": ("gla_proj_bwd.hip", "gla_proj.hip") + _COMMON_SOURCES,
}


def kernel_family(spec):
    if spec.get("kind") == "bwd" and spec.get("gated"):
        return "bwd_gated"
    if spec.get("kind") in ("sswiglu", "bwd", "proj_bwd"):
        return spec["kind"]
    if spec["dtype"] == "f16" and spec["dk"] == 64 and spec["chunk"] == 64:
        return "onepass_proj" if spec.get("gate_proj") else "onepass"
    if spec["dtype"] == "f16" and spec["dk"] == 128 and spec["chunk"] == 64:
        return "wide"
    return "generic"


def kernel_source_hash(family):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_vision_backbone_key_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[family]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, family):
    """HBM bytes per call from committed rocprofv3 counter runs, if they were
    taken on the current sources of the workload's kernels; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(family):
        return None
    return rec.get("hbm_bytes_per_call")


def kernel_label(spec, chunk, staged=False):
    """The kernels one call launches (the plan picks the single pass for
    binary16, d = 64, 64-token chunks; the three passes otherwise)."""
    if spec["dtype"] == "f16" and spec["dk"] == 64 and chunk == 64:
        if spec.get("gate_proj"):
            if staged:
                return "gla_gate_logits_kernel + gla_onepass_kernel (projection staged: two launches)"
            return "gla_onepass_kernel<gate projection fused> (single pass: one launch per call)"
        return "gla_onepass_kernel (single pass: one launch per call)"
    if spec["dtype"] == "f16" and spec["dk"] == 128 and chunk == 64:
        return ("gla_wide_kernel<aggregate> + gla_fold_kernel + gla_wide_kernel<output> "
                "(three launches per call)")
    return "gla_chunk_kernel<aggregate> + gla_fold_kernel + gla_chunk_kernel<output>"


def copy_calibration(mib):
    """A plain device copy of known size (src -> dst, `mib` MiB each way), for
    scaling the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 4}), flush=True)


def traffic_from_pmc(workload, fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, copy_bytes,
                     kernel_substr):
    """HBM bytes per call of one workload from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by the same
    counter's reading for a plain copy of `copy_bytes` bytes; written to
    profiles/traffic_<workload>.json with the kernel source hash."""
    import csv

    def per_kernel(path, substr):
        """Counter sum per dispatch, averaged per kernel name."""
        tot = {}
        for row in csv.DictReader(open(path)):
            name = row["Kernel_Name"]
            # demangled ("gla::...") or mangled ("_ZN3gla...") library kernels
            if (substr in name or "_ZN3gla" in name) and "init" not in name:
                key = (name, row["Dispatch_Id"])
                tot[key] = tot.get(key, 0.0) + float(row["Counter_Value"])
        names = {}
        for (name, _), v in tot.items():
            names.setdefault(name, []).append(v)
        return {n: sum(v) / len(v) for n, v in names.items()}, len(tot)

    cf, _ = per_kernel(calib_fetch_csv, "copy")
    cw, _ = per_kernel(calib_write_csv, "copy")
    fetch_factor = max(cf.values()) * 1024.0 / copy_bytes
    write_factor = max(cw.values()) * 1024.0 / copy_bytes
    kf, nd = per_kernel(fetch_csv, kernel_substr)
    kw, _ = per_kernel(write_csv, kernel_substr)
    # one call = one dispatch of every kernel name of the call
    fetch = sum(kf.values()) * 1024.0 / fetch_factor
    write = sum(kw.values()) * 1024.0 / write_factor
    from recurrent_vision_backbone_key_amd.inputs import WORKLOADS
    family = kernel_family(WORKLOADS[workload])
    rec = {"workload": workload, "kernel": kernel_substr, "kernel_family": family,
           "kernel_source_hash": kernel_source_hash(family),
           "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4),
           "hbm_fetch_bytes_per_call": round(fetch), "hbm_write_bytes_per_call": round(write),
           "hbm_bytes_per_call": round(fetch + write), "dispatches": nd,
           "kernels": sorted(kf)}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(spec, name, seconds):
    import numpy as np  # noqa: F401

    import oracle
    from recurrent_vision_backbone_key_amd.inputs import workload_inputs

    cores = min(16, len(os.sched_getaffinity(0)))
    H, W = spec["H"], spec["W"]
    units_total = spec["B"] * spec["NH"]
    # bounded sample: whole (batch, head) scans of the workload's calls, in call
    # order, until the time budget is spent (inputs drawn before the clock starts)
    per_call_units = min(units_total, max(cores, 1))
    inputs = [workload_inputs(name, call=c) for c in range(len(spec["dirs"]))]
    done_th = 0
    calls = 0
    t0 = time.perf_counter()
    while True:
        call = calls % len(spec["dirs"])
        x = inputs[call]
        u0 = (calls * per_call_units) % units_total
        u1 = min(units_total, u0 + per_call_units)
        z = x["z"]
        if spec.get("gate_proj"):
            z = oracle.gate_logits(x["x"], x["w1"], x["w2"], x["bias"], spec["NH"],
                                   threads=cores)
        if spec.get("kind") == "bwd" and spec.get("gated"):
            oracle.bwd_gated(x["q"], x["k"], x["v"], z, x["r"], x["w"], x["dout"],
                             spec["dirs"][call], H, W, units=(u0, u1), threads=cores)
        elif spec.get("kind") == "bwd":
            oracle.bwd(x["q"], x["k"], x["v"], z, x["dout"], spec["dirs"][call], H, W,
                       units=(u0, u1), threads=cores)
        else:
            oracle.fwd(x["q"], x["k"], x["v"], z, spec["dirs"][call], H, W, r=x["r"],
                       w=x["w"], units=(u0, u1), threads=cores)
        done_th += (u1 - u0) * H * W
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done_th / dt / 1e9, "unit": "Gtok·head/s", "cores": cores,
            "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"{calls} oracle {'backward ' if spec.get('kind') == 'bwd' else ''}calls "
                      f"of {name} ({spec['H']}x{spec['W']}, d={spec['dk']}), "
                      + ("gate logits of every token projected per call, "
                         if spec.get("gate_proj") else "")
                      + f"{per_call_units} of {units_total} (batch, head) scans each, "
                      f"{done_th} token-heads in {dt:.1f} s"}


def time_steps(step, rotate, steps, warmup, args, steps_per_graph):
    """Replay `step(r)` (r = input set) from HIP graphs of G consecutive steps
    each (a replay has a fixed cost of about 15 us on this platform, so several
    steps share one); graph i holds steps on input sets i*G .. i*G+G-1 (mod
    rotate), enough graphs that the sets cycle without repeating back to back.
    Runs `warmup` untimed steps (whole replays, then the remainder as eager
    steps, so that G depends on `steps` only), then times `steps` steps with
    HIP events on the replay stream.  Returns (ms per step, G, whether graphs
    were used)."""
    import torch

    G = 1
    if not args.no_graph:
        G = args.steps_per_graph or steps_per_graph
        G = math.gcd(G, steps) if steps > 0 else 1
    n_graphs = rotate // math.gcd(rotate, G)
    stream = torch.cuda.current_stream()
    graphs = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for r in range(rotate):
                step(r)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for gi in range(n_graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(G):
                    step((gi * G + j) % rotate)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        # i counts graph replays (G steps each) or single eager steps
        if graphs is not None:
            graphs[i % n_graphs].replay()
        else:
            step(i % rotate)

    for i in range(warmup // G):
        run(i)
    for j in range(warmup % G):
        step((warmup // G * G + j) % rotate)
    torch.cuda.synchronize()
    # one event before every replay (or eager step) and one after the last:
    # the whole bracket gives the mean, consecutive pairs give each replay's
    # time for the median and minimum (the pages compare latencies on the
    # median of repeated runs and report minimum and mean beside it)
    n = steps // G
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    for i in range(n):
        evs[i].record(stream)
        run(warmup // G + i)
    evs[n].record(stream)
    torch.cuda.synchronize()
    per_replay = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return evs[0].elapsed_time(evs[n]) / steps, G, graphs is not None, per_replay


def latency_stats(per_replay_ms, steps_per_replay, calls_per_step):
    """Median, minimum and mean microseconds per call over the timed replays."""
    import statistics
    per_call = [1e3 * t / (steps_per_replay * calls_per_step) for t in per_replay_ms]
    return {"median": round(statistics.median(per_call), 3), "min": round(min(per_call), 3),
            "mean": round(statistics.fmean(per_call), 3), "replays": len(per_call),
            "calls_per_replay": steps_per_replay * calls_per_step}


def host_cpu_model():
    """Model name of the host CPU (/proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def algorithmic_flops_bwd_per_token_head(dk, dv, chunk):
    """Chunkwise backward, causal products counted once: forward and reverse
    chunk aggregates (k^T v, q^T dO), the entering state and gradient in dq,
    dk, dv (5 x 2 dk dv), and the intra-chunk scores dO v^T, their products
    with k (dq) and q (dk), the decayed scores q k^T and their product with dO
    (dv): chunk/2 positions on average, chunk (3 dk + 2 dv) flops."""
    return 10 * dk * dv + chunk * (3 * dk + 2 * dv)


def bench_bwd(args, spec, name):
    """One step = one gla_bwd call per direction of the workload, over the
    whole batch; same timing method as the forward."""
    import torch

    from recurrent_vision_backbone_key_amd import gla
    from recurrent_vision_backbone_key_amd.inputs import make_bwd_inputs_device

    B, NH, H, W, d = spec["B"], spec["NH"], spec["H"], spec["W"], spec["dk"]
    dirs = spec["dirs"]
    es = 2 if spec["dtype"] == "f16" else 4
    th_call = B * NH * H * W
    gated = spec["gated"]
    # q, k, v, dO read, dq, dk, dv written (storage type); z read, dz written
    # (binary32); gated: r read and dr written as well, and o recomputed (the
    # forward's flops counted: the gate's derivative needs o)
    bytes_call = th_call * ((9 if gated else 7) * es * d + 8 * d)
    flops_call = th_call * (algorithmic_flops_bwd_per_token_head(d, d, spec["chunk"]) +
                            (algorithmic_flops_per_token_head(d, d, spec["chunk"]) if gated else 0))
    rotate = args.rotate or max(1, math.ceil(2 * MALL_BYTES / (bytes_call * len(dirs))))
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 20
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {name}: {len(dirs)} calls/step, {bytes_call / 1e6:.2f} MB/call, "
          f"{rotate} input sets, steps={steps} warmup={warmup}", file=sys.stderr, flush=True)
    opts = gla.make_opts(B, NH, d, d, gla.F16 if es == 2 else gla.F32)
    ws_bytes = (gla.bwd_gated_workspace_size if gated else gla.bwd_workspace_size)(dirs[0], H, W, opts)
    sets = []
    for r in range(rotate):
        calls = []
        for c, dr in enumerate(dirs):
            x = make_bwd_inputs_device(B, NH, H, W, d, spec["dtype"], spec["z"],
                                       seed=1000 * spec["index"] + 100 * r + c, device=dev,
                                       gated=gated)
            grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]),
                     torch.empty_like(x["z"]))
            if gated:
                grads += (torch.empty_like(x["r"]), torch.empty((d,), dtype=torch.float32, device=dev))
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            calls.append((x, dr, grads, ws))
        sets.append(calls)

    def step(r):
        for x, dr, grads, ws in sets[r]:
            if gated:
                gla.bwd_gated(x["q"], x["k"], x["v"], x["z"], x["r"], x["dout"], dr, H, W,
                              norm_weight=x["w"], grads=grads, workspace=ws)
            else:
                gla.bwd(x["q"], x["k"], x["v"], x["z"], x["dout"], dr, H, W, grads=grads,
                        workspace=ws)

    ms_step, G, graphed, per_replay = time_steps(step, rotate, steps, warmup, args, 10)
    us_call = 1e3 * ms_step / len(dirs)
    tflops = flops_call / (us_call * 1e-6) / 1e12
    gbs = bytes_call / (us_call * 1e-6) / 1e9
    result = {
        "metric": ("chunkwise GLA bwd (output gate included)" if gated else "chunkwise GLA bwd") +
                  f": µs/call + Gtok·head/s at L={H * W}; % of MFMA (fp32) roofline",
        "value": round(len(dirs) * th_call / (ms_step * 1e-3) / 1e9, 4), "unit": "Gtok·head/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "us_per_call": round(us_call, 3),
        "latency_us_per_call": latency_stats(per_replay, G, len(dirs)),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": name, "B": B, "heads": NH, "grid": f"{H}x{W}", "L": H * W,
                   "dk": d, "dv": d, "chunk": spec["chunk"],
                   "dirs": ",".join("L2R R2L T2B B2T".split()[x] for x in dirs),
                   "calls_per_step": len(dirs), "input_sets": rotate, "hip_graph": graphed,
                   "steps_per_graph": G, "workspace_bytes_per_call": ws_bytes,
                   "gated": gated, "accumulate": "f32", "mfma_operands": "f32"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(name, kernel_family(spec)),
                     "kernel": ("gla_bwd_states_kernel<local states> + gla_bwd_fold_kernel<forward> + "
                                "gla_bwd_oepi_kernel (o, the output gate's backward, reverse "
                                "aggregates) + gla_bwd_dw_kernel + gla_bwd_fold_kernel<reverse> + "
                                "gla_bwd_chunk_kernel"
                                if gated else
                                "gla_bwd_states_kernel + gla_bwd_fold_kernel + gla_bwd_chunk_kernel") +
                               " (figures for the whole call)",
                     "algorithmic_flops_per_call": flops_call,
                     "algorithmic_bytes_per_call": bytes_call,
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(spec, name, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_proj_bwd(args, spec, name):
    """One step = one gla_gate_proj_bwd call over every token of the batch;
    same timing method as the forward."""
    import torch

    from recurrent_vision_backbone_key_amd import gla

    B, L, NH, dk = spec["B"], spec["H"] * spec["W"], spec["NH"], spec["dk"]
    dm, rank = spec["d_model"], spec["rank"]
    es = 2 if spec["dtype"] == "f16" else 4
    dt = torch.float16 if es == 2 else torch.float32
    T, nout = B * L, NH * dk
    # dz read, x read, dx written; the weights read and their gradients written
    bytes_call = 4 * T * nout + 2 * es * T * dm + es * rank * dm + 4 * nout * rank + \
        4 * (rank * dm + nout * rank + nout)
    # hp = x W1, dhp = dz W2^T, dx, dW1, dW2 (2 flops per multiply-add), db
    flops_call = 2 * T * rank * (3 * dm + 2 * nout) + T * nout
    rotate = args.rotate or max(1, math.ceil(2 * MALL_BYTES / bytes_call))
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 50
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    sets = []
    for r in range(rotate):
        gen.manual_seed(1000 * spec["index"] + r)
        x = torch.randn((B, L, dm), generator=gen, device=dev).to(dt)
        w1 = (torch.randn((rank, dm), generator=gen, device=dev) / math.sqrt(dm)).to(dt)
        w2 = torch.randn((nout, rank), generator=gen, device=dev) / math.sqrt(rank)
        dz = torch.randn((B, L, NH, dk), generator=gen, device=dev)
        grads = (torch.empty_like(x), torch.empty((rank, dm), dtype=torch.float32, device=dev),
                 torch.empty((nout, rank), dtype=torch.float32, device=dev),
                 torch.empty((nout,), dtype=torch.float32, device=dev))
        need = gla.gate_proj_bwd_workspace_size(gla.make_gate(x, w1, w2, None), T, nout)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        sets.append((x, w1, w2, dz, grads, ws))

    def step(r):
        x, w1, w2, dz, grads, ws = sets[r]
        gla.gate_proj_bwd(x, w1, w2, dz, grads=grads, workspace=ws)

    ms_step, G, graphed, per_replay = time_steps(step, rotate, steps, warmup, args, 10)
    achieved = bytes_call / (ms_step * 1e-3) / 1e9
    tflops = flops_call / (ms_step * 1e-3) / 1e12
    result = {
        "metric": f"gate projection backward: µs/call at {T} tokens; % of HBM roofline",
        "value": round(T / (ms_step * 1e-3) / 1e9, 4), "unit": "Gtok/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "us_per_call": round(1e3 * ms_step, 3),
        "latency_us_per_call": latency_stats(per_replay, G, 1),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": name, "tokens": T, "d_model": dm, "rank": rank, "nout": nout,
                   "input_sets": rotate, "hip_graph": graphed, "steps_per_graph": G,
                   "accumulate": "f32", "mfma_operands": "f32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gla_gate_rank_kernel + 5 gla_pbwd_gemm_kernel + 3 "
                               "gla_pbwd_reduce_kernel (figures for the whole call)",
                     "algorithmic_bytes_per_call": bytes_call,
                     "algorithmic_flops_per_call": flops_call,
                     "mfma_f32_frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        import numpy as np

        import oracle
        from recurrent_vision_backbone_key_amd.inputs import make_gate_proj_inputs
        x = make_gate_proj_inputs(1, L, NH, dk, dm, rank, spec["dtype"], seed=1)
        dz = np.random.default_rng(2).standard_normal((1, L, nout)).astype(np.float32)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.gate_proj_bwd(x["x"], x["w1"], x["w2"], dz)
            n += 1
        dt_s = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(n * L / dt_s / 1e9, 6), "unit": "Gtok/s", "cores": os.cpu_count(),
            "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"{n} oracle calls on one image ({L} tokens) in {dt_s:.1f} s (numpy)"}
    print(json.dumps(result), flush=True)


def bench_sswiglu(args, spec, name):
    """One step = one gla_spatial_swiglu call over the whole batch; same
    timing method as the forward (resident inputs rotating past the last-level
    cache, HIP graphs of several steps, HIP events on the replay stream)."""
    import torch

    from recurrent_vision_backbone_key_amd import gla

    B, H, W, C = spec["B"], spec["H"], spec["W"], spec["C"]
    es = 2 if spec["dtype"] == "f16" else 4
    dt = torch.float16 if es == 2 else torch.float32
    tokens = B * H * W
    bytes_call = 3 * es * tokens * C + 40 * C   # gate, value read; out written; taps, bias
    rotate = args.rotate or max(1, math.ceil(2 * MALL_BYTES / bytes_call))
    steps = args.steps if args.steps is not None else 400
    warmup = args.warmup if args.warmup is not None else 100
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    sets = []
    for r in range(rotate):
        gen.manual_seed(1000 * spec["index"] + r)
        a = torch.randn((B, H * W, C), generator=gen, device=dev).to(dt)
        v = torch.randn((B, H * W, C), generator=gen, device=dev).to(dt)
        w = (torch.rand((C, 3, 3), generator=gen, device=dev) * 2 - 1) / 3
        b = (torch.rand((C,), generator=gen, device=dev) * 2 - 1) / 3
        sets.append((a, v, w, b, torch.empty_like(a)))

    def step(r):
        a, v, w, b, o = sets[r]
        gla.spatial_swiglu(a, v, H, W, w, b, out=o)

    ms_step, G, graphed, per_replay = time_steps(step, rotate, steps, warmup, args, 10)
    achieved = bytes_call / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "Spatial SwiGLU core: µs/call; % of HBM roofline",
        "value": round(tokens * C / (ms_step * 1e-3) / 1e9, 3), "unit": "Gtok·channel/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "us_per_call": round(1e3 * ms_step, 3),
        "latency_us_per_call": latency_stats(per_replay, G, 1),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": name, "B": B, "grid": f"{H}x{W}", "L": H * W, "channels": C,
                   "input_sets": rotate, "hip_graph": graphed, "steps_per_graph": G,
                   "accumulate": "f32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(name, "sswiglu"),
                     "kernel": "gla_sswiglu_kernel (one launch per call)",
                     "algorithmic_bytes_per_call": bytes_call},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        import numpy as np  # noqa: F401

        import oracle
        from recurrent_vision_backbone_key_amd.inputs import make_sswiglu_inputs
        x = make_sswiglu_inputs(1, H, W, C, spec["dtype"], True, seed=1)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.spatial_swiglu(x["a"], x["v"], H, W, x["w"], x["b"])
            n += 1
        dt_s = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(n * H * W * C / dt_s / 1e9, 5), "unit": "Gtok·channel/s", "cores": 1,
            "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"{n} oracle calls on one image ({H}x{W}, {C} channels) in {dt_s:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    from recurrent_vision_backbone_key_amd.inputs import WORKLOADS

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="frame640", choices=sorted(WORKLOADS))
    ap.add_argument("--segment-chunks", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0: enough to exceed 2x MALL)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--steps-per-graph", type=int, default=0,
                    help="steps captured in one HIP graph (0: 10, or 1 for steps over 1 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--staged", action="store_true",
                    help="gate-projection workloads: gla_gate_logits then gla_fwd (unfused)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every length/batch sweep point (one JSON line each)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_MIB"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc counter files")
    args = ap.parse_args()

    if args.traffic_from:
        f, w, cf, cw, mib = args.traffic_from
        spec = WORKLOADS[args.workload]
        sub = "gla::"
        traffic_from_pmc(args.workload, f, w, cf, cw, int(mib) << 20, sub)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.sweep:
        from recurrent_vision_backbone_key_amd.inputs import SWEEP
        for name in SWEEP:
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--no-cpu",
                   "--steps", str(args.steps or 100), "--warmup", str(args.warmup or 20)]
            import subprocess
            subprocess.run(cmd, check=True)
        return

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward would shard across GPUs by batch/head with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from recurrent_vision_backbone_key_amd import gla
    from recurrent_vision_backbone_key_amd.inputs import (make_gate_proj_inputs_device,
                                                          make_inputs_device, tokens_per_call)

    spec = WORKLOADS[args.workload]
    name = args.workload
    if spec.get("kind") == "sswiglu":
        bench_sswiglu(args, spec, name)
        return
    if spec.get("kind") == "bwd":
        bench_bwd(args, spec, name)
        return
    if spec.get("kind") == "proj_bwd":
        bench_proj_bwd(args, spec, name)
        return
    chunk = args.chunk or spec["chunk"]
    dirs = spec["dirs"]
    calls_per_step = len(dirs)
    B, NH, H, W, dk, dv = spec["B"], spec["NH"], spec["H"], spec["W"], spec["dk"], spec["dv"]
    es = 2 if spec["dtype"] == "f16" else 4
    gated = spec["gated"]
    gp = spec.get("gate_proj")
    staged = bool(args.staged and gp)
    th_call = tokens_per_call(spec)
    bytes_call = int(th_call * algorithmic_bytes_per_token_head(dk, dv, es, gated, gp, NH)
                     + weight_bytes_per_call(spec, es))
    flops_call = th_call * algorithmic_flops_per_token_head(dk, dv, chunk)
    step_bytes = bytes_call * calls_per_step
    rotate = args.rotate or max(1, math.ceil(2 * MALL_BYTES / step_bytes))
    big = step_bytes > (1 << 30)
    steps = args.steps if args.steps is not None else (12 if big else 400)
    warmup = args.warmup if args.warmup is not None else (3 if big else 100)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {name}: {calls_per_step} calls/step, {bytes_call / 1e6:.2f} MB/call, "
          f"{rotate} input sets, steps={steps} warmup={warmup}", file=sys.stderr, flush=True)

    # resident inputs, outputs and workspaces
    sets = []
    for r in range(rotate):
        calls = []
        for c, d in enumerate(dirs):
            x = make_inputs_device(B, NH, H, W, dk, dv, spec["dtype"], spec["z"], gated,
                                   seed=1000 * spec["index"] + 100 * r + c, device=dev)
            out = torch.empty((B, H * W, NH, dv), dtype=x["q"].dtype, device=dev)
            opts = gla.make_opts(B, NH, dk, dv, gla.F16 if es == 2 else gla.F32,
                                 segment_chunks=args.segment_chunks)
            if gp:
                # z is not an input: the projection operands replace it (the
                # staged variant writes z into a buffer of its own)
                x["z"] = torch.empty_like(x["z"]) if staged else None
                x.update(make_gate_proj_inputs_device(B, H * W, NH, dk, gp["d_model"], gp["rank"],
                                                      spec["dtype"],
                                                      seed=1000 * spec["index"] + 500 + 100 * r + c,
                                                      device=dev))
            if gp and not staged:
                need = gla.workspace_size_gate_proj(d, H, W, chunk,
                                                    gla.make_gate(x["x"], x["w1"], x["w2"], x["bias"]),
                                                    opts)
            else:
                need = gla.workspace_size(d, H, W, chunk, opts)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            if need:
                gla.workspace_init(ws)
            calls.append((x, d, out, ws))
        sets.append(calls)
    opts_probe = gla.make_opts(B, NH, dk, dv, 0, segment_chunks=args.segment_chunks)
    nseg_bytes = gla.workspace_size(0, H, W, chunk, opts_probe)

    def step(r):
        for x, d, out, ws in sets[r]:
            if gp and not staged:
                gla.fwd_gate_proj(x["q"], x["k"], x["v"], x["x"], x["w1"], x["w2"], x["bias"], d,
                                  H, W, chunk=chunk, r=x["r"], norm_weight=x["w"], eps=1e-6,
                                  out=out, segment_chunks=args.segment_chunks, workspace=ws)
                continue
            if staged:
                gla.gate_logits(x["x"], x["w1"], x["w2"], x["bias"], NH, out=x["z"])
            gla.fwd(x["q"], x["k"], x["v"], x["z"], d, H, W, chunk=chunk, r=x["r"],
                    norm_weight=x["w"], eps=1e-6, out=out, segment_chunks=args.segment_chunks,
                    workspace=ws)

    ms_step, G, graphed, per_replay = time_steps(step, rotate, steps, warmup, args,
                                                 1 if big else 10)
    us_call = 1e3 * ms_step / calls_per_step
    value = calls_per_step * th_call / (ms_step * 1e-3) / 1e9

    achieved = bytes_call / (us_call * 1e-6) / 1e9
    traffic = None if staged else load_traffic(name, kernel_family(dict(spec, chunk=chunk)))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": kernel_label(spec, chunk, staged),
                "algorithmic_bytes_per_call": bytes_call,
                "mfma_frac": round(flops_call / (us_call * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 5)}

    result = {
        "metric": METRIC, "value": round(value, 4), "unit": "Gtok·head/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "us_per_call": round(us_call, 3),
        "latency_us_per_call": latency_stats(per_replay, G, calls_per_step),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": name, "B": B, "heads": NH, "grid": f"{H}x{W}", "L": H * W,
                   "dk": dk, "dv": dv, "chunk": chunk,
                   "dirs": ",".join("L2R R2L T2B B2T".split()[d] for d in dirs),
                   "gated": gated, "calls_per_step": calls_per_step,
                   **({"gate_projection": dict(gp, staged=staged)} if gp else {}),
                   "input_sets": rotate, "hip_graph": graphed,
                   "steps_per_graph": G,
                   "workspace_bytes_per_call": nseg_bytes, "accumulate": "f32"},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(spec, name, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
