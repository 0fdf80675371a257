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
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = kernel_source_sha()
    except OSError:
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def strip_comments(text: str) -> str:
    """C++ source without // and /* */ comments and without blank lines or
    trailing spaces (string literals in these sources hold no comment
    markers), so that edits of comments alone leave the code's hash as it
    was."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_sha():
    """sha256 over the code (comments stripped) of the GEMM kernel sources
    (the template header and its translation units), in name order."""
    import hashlib
    csrc = os.path.join(ROOT, "muon_newton_schulz_06_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(f for f in os.listdir(csrc) if f.startswith("gemm")):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()


def source_ids():
    """git HEAD when the tree is a checkout (else None), and a sha256 over
    every library source, the header and this script, which identifies the
    measured code either way."""
    import hashlib
    import subprocess
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        head = None
    h = hashlib.sha256()
    files = [os.path.join("include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))]
    csrc = os.path.join("muon_newton_schulz_06_amd", "csrc")
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(os.path.join(ROOT, csrc)))]
    files += ["bench.py"]
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return head, h.hexdigest()


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


def parity_probe(mns, W, torch, carried=True):
    """GPU side of the parity figure of the main workload: one muon_step over
    the matrices of layer 0 (the shapes, seeds and kernels of the benchmark;
    each matrix's result does not depend on the batch it is in) with fp32
    weights at zero and zero momentum, so W' = −lr·sc·O exposes the
    orthogonalised update O itself.  With carried operand exponents (the
    benchmark's timed configuration) an identical step first records them,
    weights and momenta are reset, and the measured step has the momentum
    pass write the fp16 operands.  Run outside the timed region."""
    import numpy as np
    layer = W.qwen_model_shapes(1)
    # drawn on the CPU, as the oracle's inputs are (the device generator draws
    # other values), then copied
    inp = W.muon_inputs(layer, 5001, device="cpu", param_dtype=torch.float32)
    inp.params = [torch.zeros_like(p, device="cuda") for p in inp.params]
    inp.grads = [g.cuda() for g in inp.grads]
    inp.momenta = [m.cuda() for m in inp.momenta]
    sx = mns.scale_exp_buffer(len(layer), "cuda") if carried else None
    if carried:
        mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
        for t in inp.params + inp.momenta:
            t.zero_()
    mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
    torch.cuda.synchronize()
    lr32 = float(np.float32(0.02))
    out = []
    for (r, c), p in zip(layer, inp.params):
        sc = (max(1.0, r / c)) ** 0.5
        out.append(-p.double().cpu().numpy() / (lr32 * sc))
    del inp
    torch.cuda.empty_cache()
    return out


def cpu_baseline(probe=None, samples=None, budget_s=15.0, carried=True):
    """The oracle as it stands, on a bounded sample of the workload: the
    matrices of layer 0 in the order k, q, down, v, o, gate, up, one full
    muon_step each (momentum, fp64 standard Newton–Schulz, update), until
    about `budget_s` seconds of CPU work have been spent.

    The same oracle runs also give the parity figures of the line: the
    relative Frobenius error of the GPU's update O (probe, layer 0 in layer
    order) against the oracle's for every matrix timed, and of each smaller
    workload's sampled GPU outputs against the oracle's orthogonalisation of
    the same inputs (samples: name → list of (input, GPU output, steps,
    coefficients, tolerance)).  Returns (baseline, parity)."""
    import numpy as np
    import torch

    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 0) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)  # what the library receives
    layer = W.qwen_model_shapes(1)            # q, k, v, o, gate, up, down
    order = [1, 0, 6, 2, 3, 4, 5]
    shapes = [layer[i] for i in order]
    inp = W.muon_inputs(layer, 5001, device="cpu")
    t0 = time.perf_counter()
    done, errs = [], []
    for i in order:
        r, c = layer[i]
        _, _, O = oracle.muon_step(inp.params[i].float().numpy(), inp.grads[i].numpy(),
                                   inp.momenta[i].numpy(), np.float32(0.95), 0.02, c32, 5, 1e-7)
        done.append((r, c))
        if probe is not None:
            errs.append(float(np.linalg.norm(probe[i] - O) / np.linalg.norm(O)))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    fl = gram_flops(done)
    base = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"muon_step on {len(done)} of the {len(shapes)} matrices of layer 0 {done} "
                      f"(fp64 numpy, standard NS), {dt:.2f} s; algorithmic Gram flops / time"}
    parity = {}
    if probe is not None:
        parity["qwen_full"] = {
            "max_rel_err": max(errs), "tol": 2e-2, "matrices": done,
            "how": "update O of one muon_step from zero momentum, recovered from fp32 weights "
                   "at zero, against the oracle's O (relative Frobenius error), layer-0 matrices"
                   + ("; the step runs as timed (operand exponents carried from an identical earlier step)"
                      if carried else "")}
    for name, items in (samples or {}).items():
        e = []
        for x, out, steps, coeffs, tol in items:
            ref = oracle.muon_orthogonalize(x, tuple(float(np.float32(v)) for v in coeffs), steps, 1e-7)
            e.append(float(np.linalg.norm(out - ref) / np.linalg.norm(ref)))
        parity[name] = {"max_rel_err": max(e), "tol": items[0][4], "matrices": len(items),
                        "how": "muon_ns_batched outputs of sampled matrices against the oracle"}
    return base, parity


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

    def host(t):
        return t.double().cpu().numpy()

    out, samples = [], {}
    Q = mns.QUINTIC
    x = W.ns_single(device="cuda")
    xo = [torch.empty_like(x)]
    wsx = torch.empty(mns.ns_workspace_size([tuple(x.shape)], dtype=torch.float32),
                      dtype=torch.uint8, device="cuda")
    f1 = lambda: mns.muon_ns_batched([x], outs=xo, steps=5, workspace=wsx)  # noqa: E731
    out.append(entry("single 256x1024 fp32", timed(f1, 50), [(256, 1024)], MFMA_PEAK_F32,
                     "muon_ns_batched, fp32 MFMA, latency-bound", graph_ms(f1, 50)))
    samples["single 256x1024 fp32"] = [(host(x), host(xo[0]), 5, Q, 1e-4)]
    xs = W.ns_uniform_batch(device="cuda")
    outs = [torch.empty_like(t) for t in xs]
    out.append(entry("uniform 32x(1024x4096) bf16",
                     timed(lambda: mns.muon_ns_batched(xs, outs=outs, steps=5), 10),
                     [tuple(t.shape) for t in xs], MFMA_PEAK_F16, "muon_ns_batched"))
    samples["uniform 32x(1024x4096) bf16"] = [(host(xs[i]), host(outs[i]), 5, Q, 2e-2) for i in (0, 31)]
    del xs, outs
    ms_ = W.ns_small_mix(device="cuda")
    outs = [torch.empty_like(t) for t in ms_]
    wsm = torch.empty(mns.ns_workspace_size([tuple(t.shape) for t in ms_]), dtype=torch.uint8,
                      device="cuda")
    f3 = lambda: mns.muon_ns_batched(ms_, outs=outs, steps=5, workspace=wsm)  # noqa: E731
    out.append(entry("small mix 176 bf16", timed(f3, 20), [tuple(t.shape) for t in ms_],
                     MFMA_PEAK_F16, "muon_ns_batched", graph_ms(f3, 20)))
    samples["small mix 176 bf16"] = [(host(ms_[i]), host(outs[i]), 5, Q, 2e-2)
                                     for i in range(0, len(ms_), 11)]
    del ms_, outs
    iso = sorted(isolated_calls(mns, W, torch, "small_mix", warm=1, calls=5)["ms_per_call"])
    out[-1]["ms_isolated_call"] = iso[len(iso) // 2]
    shapes = W.qwen_model_shapes(1)
    inp = W.muon_inputs(shapes, 4001, device="cuda")
    plain = timed(lambda: mns.muon_step(inp.params, inp.grads, inp.momenta, steps=5), 10)
    # as a training loop runs it: operand exponents carried from step to step
    # (the untimed first call of `timed` records them)
    sx = mns.scale_exp_buffer(len(shapes), "cuda")
    carried = timed(lambda: mns.muon_step(inp.params, inp.grads, inp.momenta, steps=5, scale_exp=sx), 10)
    out.append(entry("one Qwen2.5-7B layer muon_step", carried, shapes, MFMA_PEAK_F16,
                     "muon_step, operand exponents carried across steps (scale_exp)"))
    out[-1]["ms_without_carried_exponents"] = plain
    del inp
    torch.cuda.empty_cache()
    return out, samples


def isolated_calls(mns, W, torch, which, warm=3, calls=3):
    """Wall time of single muon_ns_batched calls of a smaller workload, each
    started on an idle GPU (synchronisation and a 2 ms pause before it): the
    latency of one call, host submission included."""
    xs = W.ns_small_mix(device="cuda") if which == "small_mix" else W.ns_uniform_batch(device="cuda")
    outs = [torch.empty_like(t) for t in xs]
    ws = torch.empty(mns.ns_workspace_size([tuple(t.shape) for t in xs]), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warm):
        mns.muon_ns_batched(xs, outs=outs, steps=5, workspace=ws)
    torch.cuda.synchronize()
    ms = []
    for _ in range(calls):
        time.sleep(0.002)
        t0 = time.perf_counter()
        mns.muon_ns_batched(xs, outs=outs, steps=5, workspace=ws)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t0) * 1e3)
    return {"isolated": which, "matrices": len(xs), "ms_per_call": ms}


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
    ap.add_argument("--overlap", action="store_true",
                    help="muon_step's overlap option: HBM-bound passes of a later chunk under the "
                         "products of an earlier one")
    ap.add_argument("--no-carried-exponents", action="store_true",
                    help="run the step without scale_exp (every operand cast in its own pass "
                         "after the norm), as a caller without optimiser state would")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB read + 1 GiB write kernel (counter calibration)")
    ap.add_argument("--isolated", choices=["small_mix", "uniform"],
                    help="run only isolated calls of a smaller workload (each after a "
                         "synchronisation and a 2 ms pause; kernel-trace runs)")
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
    if args.isolated:
        print(json.dumps(isolated_calls(mns, W, torch, args.isolated)), flush=True)
        return
    shapes = workload_shapes(args.workload)
    seed0 = 5001
    print(f"[bench] generating {len(shapes)} matrices on {dev}", file=sys.stderr, flush=True)
    inp = W.muon_inputs(shapes, seed0, device=dev)
    ws = torch.empty(mns.step_workspace_size(shapes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    # the optimiser state a training loop carries besides the momenta: one
    # operand exponent per matrix, recorded by each step for the next (the
    # first warm-up step casts every operand in its own pass)
    carried = not args.no_carried_exponents
    sx = mns.scale_exp_buffer(len(shapes), dev) if carried else None

    def step():
        mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5,
                      workspace=ws, stream=stream, overlap=args.overlap, scale_exp=sx)

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
    others, samples = None, None
    del inp, ws
    torch.cuda.empty_cache()
    probe = None
    if not args.no_cpu_baseline and args.workload == "qwen_full":
        probe = parity_probe(mns, W, torch, carried)
    if not args.no_other_configs:
        print("[bench] timing the smaller workloads", file=sys.stderr, flush=True)
        others, samples = other_configs(mns, W, torch)
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample (and the parity figures)", file=sys.stderr,
              flush=True)
        cpu, parity = cpu_baseline(probe, samples, carried=carried)
    git_head, src_sha = source_ids()
    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: Qwen2.5-7B-shaped matrix set "
                               f"({len(shapes)} matrices, {sum(r * c for r, c in shapes)} params)",
                   "op": "muon_step", "ns_steps": 5, "coeffs": "quintic (3.4445, -4.775, 2.0315)",
                   "param_dtype": "bf16", "grad_dtype": "f32", "momentum_dtype": "f32",
                   "mfma_operands": "f16 (power-of-two scaled)", "accumulate": "f32",
                   "operand_exponents": "carried across steps (scale_exp)" if carried else "none",
                   "algorithmic_tflop_per_step": F / 1e12, "parallelism": "single GPU"},
        "frac_mfma_peak": tflops / MFMA_PEAK_F16,
        "matrices_per_s": len(shapes) / (ms / 1e3),
        "elementwise_gbs": {k: breakdown[k]["gbs"] for k in ("momentum", "cast") if k in breakdown},
        "roofline": roofline, "breakdown": breakdown, "cpu_baseline": cpu, "parity": parity,
        "git_head": git_head, "source_sha256": src_sha,
        "selected_step": selected, "other_configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
