"""Launch-configuration autotuning with a cached table.

DMuon's technical summary (gist.science, Korean), §2.4, tunes kernel
configurations per matrix shape when training starts and keeps the winners
in a cache.  Here a Gram group's configuration is its tile edge (fp16
groups: 128 or 256; fp32 groups: 32, 64 or 128) and the order in which its tiles
run (logical tiles per XCD run: 16, 32, 64; tile rows per band: 2, 4, 8),
keyed by the group's size m, largest n, operand type and batch-size class
floor(log2(matrices in the group)) — exactly what `muon_set_tile_table`
takes.  For every group of a workload the knobs are searched one after the
other (tile, then XCD run, then band), each candidate installed and the
whole call timed with HIP events (median of `reps` after a warm-up); the
other groups keep their current choice while one group is being tuned.

    python -m muon_newton_schulz_06_amd.autotune --out tiles.json   # Qwen2.5-7B set
    python -m muon_newton_schulz_06_amd.autotune --apply tiles.json
"""
from __future__ import annotations

import argparse
import json
import math
import sys

CANDIDATES = {"f16": (128, 256), "f32": (32, 64, 128)}
XCD_WINDOWS = (16, 32, 64)
BANDS = (2, 4, 8)


def count_class(count: int) -> int:
    return max(0, int(math.floor(math.log2(max(count, 1)))))


def groups_of(shapes, for_step=True, dtype=None):
    """(m, n_max, op, count, state32) of every Gram group the planner forms."""
    import torch

    from . import describe_plan
    p = describe_plan(shapes, for_step=for_step, dtype=dtype or torch.bfloat16)
    return [(g["m"], g["n_max"], g["op"], g["count"], g["state32"]) for g in p["groups"]]


def save(entries, path, meta=None):
    with open(path, "w") as f:
        json.dump({"meta": meta or {}, "entries": entries}, f, indent=1)


def load_table(path):
    with open(path) as f:
        return json.load(f)["entries"]


def apply(path):
    from . import set_tile_table
    set_tile_table(load_table(path))


def tune(shapes, reps: int = 5, seed: int = 17, device="cuda", log=sys.stderr, run=None):
    """Tune every group of a `muon_step` over `shapes` (bf16 weights, fp32
    gradients), or of the call `run` if given; returns the table entries
    (also installed)."""
    import torch

    from . import muon_step, set_tile_table

    if run is None:
        from .schedule import _inputs
        ps, gs, ms = _inputs(shapes, seed, device)

        def run():
            muon_step(ps, gs, ms)

    def timed():
        run()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    def entries_of(chosen):
        return [dict(m=k[0], n=k[1], op=k[2], count_class=k[3], **v) for k, v in chosen.items()]

    chosen = {}
    set_tile_table([])
    for m, n, op, count, state32 in groups_of(shapes):
        key = (m, n, op, count_class(count))
        conf = {"tile": 0, "xcd_window": 0, "band": 0}
        knobs = [("xcd_window", XCD_WINDOWS), ("band", BANDS)]
        if not state32:  # fp32-state groups are fixed to 128-tiles by the precision policy
            knobs.insert(0, ("tile", CANDIDATES[op]))
        for name, values in knobs:
            best = None
            for v in values:
                trial = dict(chosen)
                trial[key] = dict(conf, **{name: v})
                set_tile_table(entries_of(trial))
                t = timed()
                print(f"[autotune] m={m} n={n} {op} x{count}: {name} {v} -> {t:.3f} ms", file=log,
                      flush=True)
                if best is None or t < best[1]:
                    best = (v, t)
            conf[name] = best[0]
        chosen[key] = conf
    entries = entries_of(chosen)
    set_tile_table(entries)
    return entries


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", help="write the tuned table here (JSON)")
    ap.add_argument("--apply", help="install a saved table and print the resulting plan tiles")
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args(argv)
    from .schedule import QWEN_LAYER
    shapes = QWEN_LAYER * args.layers
    if args.apply:
        apply(args.apply)
        print(json.dumps([{"m": m, "n": n, "op": op, "count": c}
                          for m, n, op, c, _ in groups_of(shapes)]))
        return
    import torch
    entries = tune(shapes, reps=args.reps)
    meta = {"device": torch.cuda.get_device_name(0), "workload": f"{args.layers} Qwen2.5-7B layers",
            "what": "fastest tile, XCD run and band per (m, n, op, count class), whole muon_step timed"}
    if args.out:
        save(entries, args.out, meta)
    print(json.dumps({"meta": meta, "entries": entries}))


if __name__ == "__main__":
    main()
