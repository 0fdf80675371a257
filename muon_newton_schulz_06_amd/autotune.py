"""Tile autotuning with a cached configuration table.

DMuon's technical summary (gist.science, Korean), §2.4, tunes kernel
configurations per matrix shape when training starts and keeps the winners
in a cache.  Here the configuration with a measurable effect is the tile
edge of a Gram group (fp16 groups: 128 or 256; fp32 groups: 64 or 128),
keyed by the group's size m, operand type and batch-size class
floor(log2(matrices in the group)) — exactly what `muon_set_tile_table`
takes.  For every group of a workload each candidate is installed, the whole
call is timed with HIP events (median of `reps` after a warm-up), and the
fastest candidate is kept; the other groups keep their current choice while
one group is being tuned.

    python -m muon_newton_schulz_06_amd.autotune --out tiles.json   # Qwen2.5-7B set
    python -m muon_newton_schulz_06_amd.autotune --apply tiles.json
"""
from __future__ import annotations

import argparse
import json
import math
import sys

CANDIDATES = {"f16": (128, 256), "f32": (64, 128)}


def count_class(count: int) -> int:
    return max(0, int(math.floor(math.log2(max(count, 1)))))


def groups_of(shapes, for_step=True, dtype=None):
    """(m, op, count, state32) of every Gram group the planner forms."""
    import torch

    from . import describe_plan
    p = describe_plan(shapes, for_step=for_step, dtype=dtype or torch.bfloat16)
    return [(g["m"], g["op"], g["count"], g["state32"]) for g in p["groups"]]


def save(entries, path, meta=None):
    with open(path, "w") as f:
        json.dump({"meta": meta or {}, "entries": entries}, f, indent=1)


def load_table(path):
    with open(path) as f:
        return json.load(f)["entries"]


def apply(path):
    from . import set_tile_table
    set_tile_table(load_table(path))


def tune(shapes, reps: int = 5, seed: int = 17, device="cuda", log=sys.stderr):
    """Tune the tile of every group of a `muon_step` over `shapes` (bf16
    weights, fp32 gradients); returns the table entries (also installed)."""
    import torch

    from . import muon_step, set_tile_table
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

    chosen = {}
    set_tile_table([])
    for m, op, count, state32 in groups_of(shapes):
        if state32:
            continue  # fixed to 128 by the precision policy
        key = (m, op, count_class(count))
        best = None
        for tile in CANDIDATES[op]:
            trial = dict(chosen)
            trial[key] = tile
            set_tile_table([{"m": k[0], "op": k[1], "count_class": k[2], "tile": v}
                            for k, v in trial.items()])
            ms_ = timed()
            print(f"[autotune] m={m} {op} x{count}: tile {tile} -> {ms_:.3f} ms", file=log,
                  flush=True)
            if best is None or ms_ < best[1]:
                best = (tile, ms_)
        chosen[key] = best[0]
    entries = [{"m": k[0], "op": k[1], "count_class": k[2], "tile": v} for k, v in chosen.items()]
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
        print(json.dumps([{"m": m, "op": op, "count": c}
                          for m, op, c, _ in groups_of(shapes)]))
        return
    import torch
    entries = tune(shapes, reps=args.reps)
    meta = {"device": torch.cuda.get_device_name(0), "workload": f"{args.layers} Qwen2.5-7B layers",
            "what": "fastest tile per (m, op, count class), whole muon_step timed"}
    if args.out:
        save(entries, args.out, meta)
    print(json.dumps({"meta": meta, "entries": entries}))


if __name__ == "__main__":
    main()
