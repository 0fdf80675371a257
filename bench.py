"""Benchmark of the Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One "step" is one complete muon_step (momentum, Frobenius normalisation,
Gram Newton–Schulz with 5 quintic steps, weight update) over every matrix of
the workload, with all inputs resident in HBM.  The default workload is the
full Qwen2.5-7B-shaped matrix set: 28 layers × {q, o 3584×3584; k, v
512×3584; gate, up 18944×3584; down 3584×18944} = 196 matrices, 6.53 B
parameters, bf16 weights, fp32 gradients and momentum (seeded synthetic data).

Prints one JSON line: whole-step throughput in algorithmic TFLOP/s (Gram
formulation; symmetric products count their upper triangle only), the
roofline of the dominant kernel (HIP events over the timed region), the
fp64 CPU oracle timed on a bounded sample of the same workload, and (under
"other_configs", unless --no-other-configs) the smaller workloads timed in
the same run: one 256×1024 fp32 matrix, 32 × 1024×4096 bf16, the
176-matrix small-shape mix and one Qwen2.5-7B-shaped layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_F16 = 2500.0   # TFLOP/s, MI355X dense fp16/bf16 MFMA
MFMA_PEAK_F32 = 157.3    # TFLOP/s, MI355X dense fp32 MFMA
HBM_PEAK = 8000.0        # GB/s

METRIC = "Muon step ms & NS TFLOP/s (% MFMA peak), Qwen2.5-7B-shaped matrix set"

KERNEL_SYMBOLS = {"gram256_axpy": "void muon::gemm256_kernel<2, 0>(muon::GemmLaunch)",
                  "gram256_sq": "void muon::gemm256_kernel<1, 0>(muon::GemmLaunch)",
                  "syrk": "void muon::gemm256_kernel<0, 0>(muon::GemmLaunch)",
                  "final": "void muon::gemm256_kernel<3, 1|2>(muon::GemmLaunch)"}


def traffic_for(kind, workload):
    """HBM bytes per launch of the dominant kernel, from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, if it was taken on the current
    kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.traffic.json")
    src = os.path.join(ROOT, "muon_newton_schulz_06_amd", "csrc", "gemm.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def workload_shapes(name):
    import workloads as W
    if name == "qwen_full":
        return W.qwen_model_shapes(28)
    if name == "qwen_layer":
        return W.qwen_model_shapes(1)
    raise SystemExit(f"unknown workload {name}")


def gram_flops(shapes, steps=5):
    tot = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        tot += m * (m + 1) * n + (4 * steps - 3) * m * m * (m + 1) + 2 * m * m * n
    return tot


def cpu_baseline(budget_s=15.0):
    """The oracle as it stands, on a bounded sample of the workload: the
    matrices of layer 0 in the order k, q, down, v, o, gate, up, one full
    muon_step each (momentum, fp64 standard Newton–Schulz, update), until
    about `budget_s` seconds of CPU work have been spent."""
    import numpy as np
    import torch

    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 0) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    layer = W.qwen_model_shapes(1)            # q, k, v, o, gate, up, down
    order = [1, 0, 6, 2, 3, 4, 5]
    shapes = [layer[i] for i in order]
    inp = W.muon_inputs(layer, 5001, device="cpu")
    t0 = time.perf_counter()
    done = []
    for i in order:
        r, c = layer[i]
        oracle.muon_step(inp.params[i].float().numpy(), inp.grads[i].numpy(),
                         inp.momenta[i].numpy(), np.float32(0.95), 0.02, oracle.QUINTIC, 5, 1e-7)
        done.append((r, c))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    fl = gram_flops(done)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"muon_step on {len(done)} of the {len(shapes)} matrices of layer 0 {done} "
                      f"(fp64 numpy, standard NS), {dt:.2f} s; algorithmic Gram flops / time"}


def other_configs(mns, W, torch):
    """ms per call, matrices/s and algorithmic TFLOP/s of the smaller
    workloads (HIP events on the current stream, after one warm-up call)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    def entry(name, ms, shapes, peak, note, ms_graph=None):
        fl = gram_flops(shapes)
        e = {"workload": name, "ms": ms, "matrices_per_s": len(shapes) / (ms / 1e3),
             "tflops": fl / (ms / 1e3) / 1e12, "frac_peak": fl / (ms / 1e3) / 1e12 / peak,
             "note": note}
        if ms_graph is not None:
            e["ms_graph_replay"] = ms_graph
            e["matrices_per_s_graph_replay"] = len(shapes) / (ms_graph / 1e3)
        return e

    def graph_ms(fn, reps):
        """The same call captured once into a HIP graph, then replayed."""
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return timed(g.replay, reps)

    out = []
    x = W.ns_single(device="cuda")
    xo = [torch.empty_like(x)]
    wsx = torch.empty(mns.ns_workspace_size([tuple(x.shape)], dtype=torch.float32),
                      dtype=torch.uint8, device="cuda")
    f1 = lambda: mns.muon_ns_batched([x], outs=xo, steps=5, workspace=wsx)  # noqa: E731
    out.append(entry("single 256x1024 fp32", timed(f1, 50), [(256, 1024)], MFMA_PEAK_F32,
                     "muon_ns_batched, fp32 MFMA, latency-bound", graph_ms(f1, 50)))
    xs = W.ns_uniform_batch(device="cuda")
    outs = [torch.empty_like(t) for t in xs]
    out.append(entry("uniform 32x(1024x4096) bf16",
                     timed(lambda: mns.muon_ns_batched(xs, outs=outs, steps=5), 10),
                     [tuple(t.shape) for t in xs], MFMA_PEAK_F16, "muon_ns_batched"))
    del xs, outs
    ms_ = W.ns_small_mix(device="cuda")
    outs = [torch.empty_like(t) for t in ms_]
    wsm = torch.empty(mns.ns_workspace_size([tuple(t.shape) for t in ms_]), dtype=torch.uint8,
                      device="cuda")
    f3 = lambda: mns.muon_ns_batched(ms_, outs=outs, steps=5, workspace=wsm)  # noqa: E731
    out.append(entry("small mix 176 bf16", timed(f3, 20), [tuple(t.shape) for t in ms_],
                     MFMA_PEAK_F16, "muon_ns_batched", graph_ms(f3, 20)))
    del ms_, outs
    shapes = W.qwen_model_shapes(1)
    inp = W.muon_inputs(shapes, 4001, device="cuda")
    out.append(entry("one Qwen2.5-7B layer muon_step",
                     timed(lambda: mns.muon_step(inp.params, inp.grads, inp.momenta, steps=5), 10),
                     shapes, MFMA_PEAK_F16, "muon_step"))
    del inp
    torch.cuda.empty_cache()
    return out


def selected_step(mns, torch, inp, shapes, stream, fraction, warmup=1, steps=3):
    """The row/column-selected step with error feedback over the same
    matrices (state continues from the main run): ms per step and the
    per-kind HIP-event breakdown; its passes over M, g and W are HBM-bound,
    so the roofline entry is the accumulate pass (B = M + g with row scores)
    against HBM bandwidth."""
    ws = torch.empty(mns.step_selected_workspace_size(shapes, fraction), dtype=torch.uint8,
                     device=inp.params[0].device)

    def step():
        mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=fraction, beta=0.95,
                               lr=0.02, steps=5, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mns.profile_enable(True)
    for k in mns.PROFILE_KINDS:
        mns.profile_read(k)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mns.profile_enable(False)
    kinds = {k: mns.profile_read(k) for k in mns.PROFILE_KINDS}
    ms = (t1 - t0) * 1e3 / steps
    per_kind = {}
    for k, v in kinds.items():
        if v["launches"]:
            e = {"ms_per_step": v["ms"] / steps, "launches_per_step": v["launches"] // steps}
            if k in ("syrk", "gram128", "gram256_sq", "gram256_axpy", "final"):
                e["tflops"] = v["work"] / (v["ms"] / 1e3) / 1e12
            else:
                e["gbs"] = v["work"] / (v["ms"] / 1e3) / 1e9
            per_kind[k] = e
    acc = kinds["sel_accum"]
    gbs = acc["work"] / (acc["ms"] / 1e3) / 1e9
    del ws
    return {"workload": f"muon_step_selected, fraction {fraction}, same {len(shapes)} matrices",
            "ms_per_step": ms, "matrices_per_s": len(shapes) / (ms / 1e3), "steps": steps,
            "roofline": {"bound": "hbm", "kernel": "sel_accum",
                         "symbol": "muon::(anonymous namespace)::sel_accum_kernel(muon::SelLaunch)",
                         "achieved": gbs, "peak": HBM_PEAK, "unit": "GB/s", "frac": gbs / HBM_PEAK,
                         "avg_launch_ms": acc["ms"] / acc["launches"],
                         "algorithmic_bytes_per_launch": acc["work"] / acc["launches"]},
            "breakdown": per_kind}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen_full")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the main workload (profiling runs)")
    ap.add_argument("--no-selected", action="store_true",
                    help="skip the row/column-selected step timing")
    ap.add_argument("--selected-fraction", type=float, default=0.25)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB read + 1 GiB write kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the step shards by matrix across GPUs "
              "but no multi-GPU path is built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import muon_newton_schulz_06_amd as mns
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        # A kernel of known traffic for scaling the FETCH_SIZE / WRITE_SIZE
        # counters: y = 2·x over 2^28 fp32 values reads and writes 1 GiB each.
        x = torch.ones(1 << 28, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 2.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "mul_out", "read_bytes": 1 << 30, "write_bytes": 1 << 30}))
        return
    mns.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = workload_shapes(args.workload)
    seed0 = 5001
    print(f"[bench] generating {len(shapes)} matrices on {dev}", file=sys.stderr, flush=True)
    inp = W.muon_inputs(shapes, seed0, device=dev)
    ws = torch.empty(mns.step_workspace_size(shapes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5,
                      workspace=ws, stream=stream)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done", file=sys.stderr, flush=True)

    mns.profile_enable(True)
    for k in mns.PROFILE_KINDS:
        mns.profile_read(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mns.profile_enable(False)
    kinds = {k: mns.profile_read(k) for k in mns.PROFILE_KINDS}
    ms = (t1 - t0) * 1e3 / args.steps
    F = gram_flops(shapes)
    tflops = F / (ms / 1e3) / 1e12

    gemm_kinds = ("syrk", "gram128", "gram256_sq", "gram256_axpy", "final")
    breakdown = {}
    for k, v in kinds.items():
        if v["launches"] == 0:
            continue
        per_step_ms = v["ms"] / args.steps
        if k in gemm_kinds:
            rate = v["work"] / (v["ms"] / 1e3) / 1e12
            breakdown[k] = {"ms_per_step": per_step_ms, "launches_per_step": v["launches"] // args.steps,
                            "tflops": rate, "frac_peak": rate / MFMA_PEAK_F16}
        else:
            rate = v["work"] / (v["ms"] / 1e3) / 1e9
            breakdown[k] = {"ms_per_step": per_step_ms, "launches_per_step": v["launches"] // args.steps,
                            "gbs": rate, "frac_peak": rate / HBM_PEAK}
    # The dominant kernel: the Gram-space a·Y + B·Y products on 256×256 tiles
    # (gemm256_kernel with the AXPY epilogue), timed alone with HIP events on
    # the launch stream inside the timed region.
    dom = "gram256_axpy" if kinds["gram256_axpy"]["launches"] else max(gemm_kinds, key=lambda k: kinds[k]["ms"])
    d = kinds[dom]
    per_launch = d["work"] / d["launches"]
    avg_s = d["ms"] / d["launches"] / 1e3
    achieved = per_launch / avg_s / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "symbol": KERNEL_SYMBOLS.get(dom),
                "achieved": achieved, "peak": MFMA_PEAK_F16, "unit": "TFLOP/s",
                "frac": achieved / MFMA_PEAK_F16, "traffic": traffic_for(dom, args.workload),
                "avg_launch_ms": avg_s * 1e3, "algorithmic_flops_per_launch": per_launch,
                "launches": d["launches"]}
    selected = None
    if not args.no_selected:
        print("[bench] timing the selected-row step", file=sys.stderr, flush=True)
        selected = selected_step(mns, torch, inp, shapes, stream, args.selected_fraction)
    others = None
    if not args.no_other_configs:
        del inp, ws
        torch.cuda.empty_cache()
        print("[bench] timing the smaller workloads", file=sys.stderr, flush=True)
        others = other_configs(mns, W, torch)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: Qwen2.5-7B-shaped matrix set "
                               f"({len(shapes)} matrices, {sum(r * c for r, c in shapes)} params)",
                   "op": "muon_step", "ns_steps": 5, "coeffs": "quintic (3.4445, -4.775, 2.0315)",
                   "param_dtype": "bf16", "grad_dtype": "f32", "momentum_dtype": "f32",
                   "mfma_operands": "f16 (power-of-two scaled)", "accumulate": "f32",
                   "algorithmic_tflop_per_step": F / 1e12, "parallelism": "single GPU"},
        "frac_mfma_peak": tflops / MFMA_PEAK_F16,
        "matrices_per_s": len(shapes) / (ms / 1e3),
        "elementwise_gbs": {k: breakdown[k]["gbs"] for k in ("momentum", "cast") if k in breakdown},
        "roofline": roofline, "breakdown": breakdown, "cpu_baseline": cpu,
        "selected_step": selected, "other_configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
