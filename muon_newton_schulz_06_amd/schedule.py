"""Per-shape cost table and owner assignment for sharding the step by matrix.

DMuon's technical summary (gist.science, Korean), §2.3, balances the Muon
update over owner ranks from measured costs: at start-up every distinct
matrix shape is timed over several batch sizes, and owners are assigned so
that the predicted makespan (the largest per-rank load) is as small as
possible, with a greedy heuristic where an exact search is too large.

This module measures that table on one GPU with the library's own `muon_step`
(so the costs are those of the batched kernels, including what batching
saves), and predicts the per-GPU loads of an assignment:

* `profile_shapes` — times `muon_step` for each distinct shape at each batch
  size (GPU);
* `CostTable` — the table, JSON round trip, and the cost of k matrices of a
  shape (piecewise linear in k between measured batch sizes, extended
  linearly past the last one);
* `assign_greedy` — longest-processing-time-first: matrices in decreasing
  single-matrix cost, each to the rank whose load grows least under the
  batched cost model (ties to the lower rank);
* `assign_round_robin` — the naive assignment, for comparison;
* `loads` / `makespan` — predicted per-rank loads of any assignment.

The per-rank load is modelled as the sum over shapes of cost(shape, count);
`validate_on_one_gpu` measures each rank's share of an assignment on the one
GPU here, which checks that model against the real batched step.

    python -m muon_newton_schulz_06_amd.schedule --profile --out table.json
    python -m muon_newton_schulz_06_amd.schedule --table table.json --gpus 8
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import dataclass, field

Shape = tuple  # (rows, cols)


def _key(shape) -> str:
    return f"{int(shape[0])}x{int(shape[1])}"


def _unkey(k: str) -> Shape:
    r, c = k.split("x")
    return (int(r), int(c))


@dataclass
class CostTable:
    """ms per `muon_step` call for k matrices of one shape: costs[shape][k]."""
    costs: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)

    def add(self, shape, k: int, ms: float):
        self.costs.setdefault(tuple(shape), {})[int(k)] = float(ms)

    def cost(self, shape, k: int) -> float:
        if k <= 0:
            return 0.0
        pts = self.costs.get(tuple(shape))
        if not pts:
            raise KeyError(f"no measurements for shape {tuple(shape)}")
        ks = sorted(pts)
        if k in pts:
            return pts[k]
        if len(ks) == 1:
            return pts[ks[0]] * k / ks[0]
        # (0, 0) is a point of the curve: no matrices cost nothing
        xs = [0] + ks
        if k > xs[-1]:
            x0, x1 = xs[-2], xs[-1]
        else:
            i = next(j for j in range(1, len(xs)) if xs[j] > k)
            x0, x1 = xs[i - 1], xs[i]
        y0, y1 = (0.0 if x0 == 0 else pts[x0]), pts[x1]
        return y0 + (y1 - y0) * (k - x0) / (x1 - x0)

    def to_json(self) -> str:
        return json.dumps({"meta": self.meta,
                           "costs_ms": {_key(s): {str(k): v for k, v in sorted(p.items())}
                                        for s, p in self.costs.items()}}, indent=1)

    @staticmethod
    def from_json(text: str) -> "CostTable":
        d = json.loads(text)
        t = CostTable(meta=d.get("meta", {}))
        for sk, pts in d["costs_ms"].items():
            for k, v in pts.items():
                t.add(_unkey(sk), int(k), float(v))
        return t


def loads(shapes, owners, n_ranks: int, table: CostTable) -> list:
    """Predicted per-rank load: Σ over shapes of cost(shape, matrices of that
    shape the rank owns)."""
    counts = [dict() for _ in range(n_ranks)]
    for s, o in zip(shapes, owners):
        if not 0 <= o < n_ranks:
            raise ValueError(f"owner {o} outside 0..{n_ranks - 1}")
        counts[o][tuple(s)] = counts[o].get(tuple(s), 0) + 1
    return [sum(table.cost(s, k) for s, k in c.items()) for c in counts]


def makespan(shapes, owners, n_ranks: int, table: CostTable) -> float:
    return max(loads(shapes, owners, n_ranks, table))


def assign_round_robin(shapes, n_ranks: int) -> list:
    return [i % n_ranks for i in range(len(shapes))]


def assign_greedy(shapes, n_ranks: int, table: CostTable) -> list:
    """Longest-processing-time first under the batched cost model."""
    if n_ranks <= 0:
        raise ValueError("n_ranks must be positive")
    order = sorted(range(len(shapes)), key=lambda i: (-table.cost(shapes[i], 1), i))
    counts = [dict() for _ in range(n_ranks)]
    load = [0.0] * n_ranks
    owners = [-1] * len(shapes)
    for i in order:
        s = tuple(shapes[i])
        best, best_load = 0, None
        for r in range(n_ranks):
            k = counts[r].get(s, 0)
            new = load[r] + table.cost(s, k + 1) - table.cost(s, k)
            if best_load is None or new < best_load - 1e-12:
                best, best_load = r, new
        owners[i] = best
        counts[best][s] = counts[best].get(s, 0) + 1
        load[best] = best_load
    return owners


def lower_bound(shapes, n_ranks: int, table: CostTable) -> float:
    """max(max_i c(s_i, 1), Σ_s c(s, N_s) / R): a bound on every assignment's
    makespan when each cost curve is non-decreasing (a rank that owns a
    matrix pays at least its single cost) and subadditive (splitting a shape
    over ranks never costs less in total than batching it on one)."""
    by_shape = {}
    for s in shapes:
        by_shape[tuple(s)] = by_shape.get(tuple(s), 0) + 1
    single = max((table.cost(s, 1) for s in by_shape), default=0.0)
    total = sum(table.cost(s, k) for s, k in by_shape.items())
    return max(single, total / n_ranks)


# ------------------------------------------------------------------ GPU side
# One Qwen2.5-7B decoder layer's 2-D weights (rows, cols): q, k, v, o, gate,
# up, down.
QWEN_LAYER = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584),
              (18944, 3584), (3584, 18944)]


def _inputs(shapes, seed, device):
    """Seeded synthetic step inputs: bf16 weights N(0, 0.02²), fp32 gradients
    N(0, 0.01²), zero fp32 momentum."""
    import torch
    gen = torch.Generator(device=device)
    ps, gs, ms = [], [], []
    for j, s in enumerate(shapes):
        gen.manual_seed(seed + j)
        ps.append((torch.randn(s, generator=gen, device=device) * 0.02).to(torch.bfloat16))
        gs.append(torch.randn(s, generator=gen, device=device) * 0.01)
        ms.append(torch.zeros(s, device=device))
    return ps, gs, ms


def profile_shapes(shapes, batch_sizes=(1, 2, 4, 8), reps: int = 3, seed: int = 7,
                   steps: int = 5, device="cuda") -> CostTable:
    """Time one `muon_step` call over k matrices of each distinct shape
    (bf16 weights, fp32 gradients and momentum, seeded synthetic values),
    median of `reps` calls after one warm-up, with HIP events."""
    import torch

    from . import muon_step

    table = CostTable(meta={"device": torch.cuda.get_device_name(0), "reps": reps,
                            "ns_steps": steps, "what": "ms per muon_step call, median"})
    distinct = []
    for s in shapes:
        if tuple(s) not in distinct:
            distinct.append(tuple(s))
    for s in distinct:
        for k in batch_sizes:
            ps, gs, ms = _inputs([s] * k, seed, device)
            muon_step(ps, gs, ms, steps=steps)
            times = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                muon_step(ps, gs, ms, steps=steps)
                e1.record()
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            table.add(s, k, sorted(times)[len(times) // 2])
            print(f"[profile] {s} x{k}: {table.costs[s][k]:.3f} ms", file=sys.stderr, flush=True)
            del ps, gs, ms
            torch.cuda.empty_cache()
    return table


def validate_on_one_gpu(shapes, owners, n_ranks: int, reps: int = 3, seed: int = 11,
                        device="cuda") -> list:
    """Measured ms of each rank's share (one `muon_step` over the matrices it
    owns), run one rank after another on this GPU."""
    import torch

    from . import muon_step

    out = []
    for r in range(n_ranks):
        mine = [tuple(s) for s, o in zip(shapes, owners) if o == r]
        if not mine:
            out.append(0.0)
            continue
        ps, gs, ms = _inputs(mine, seed, device)
        muon_step(ps, gs, ms)
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            muon_step(ps, gs, ms)
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        out.append(sorted(times)[len(times) // 2])
        print(f"[validate] rank {r}: {len(mine)} matrices, {out[-1]:.2f} ms", file=sys.stderr,
              flush=True)
        del ps, gs, ms
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--profile", action="store_true", help="measure the table on this GPU")
    ap.add_argument("--out", help="write the table here (JSON)")
    ap.add_argument("--table", help="read the table from here (JSON)")
    ap.add_argument("--gpus", type=int, default=8, help="ranks to assign owners over")
    ap.add_argument("--layers", type=int, default=28, help="Qwen2.5-7B-shaped layers")
    ap.add_argument("--batch-sizes", default="1,2,4,8,16")
    ap.add_argument("--validate", action="store_true",
                    help="measure each rank's share of both assignments on this GPU")
    args = ap.parse_args(argv)
    shapes = QWEN_LAYER * args.layers
    if args.profile:
        table = profile_shapes(shapes, tuple(int(x) for x in args.batch_sizes.split(",")))
        if args.out:
            with open(args.out, "w") as f:
                f.write(table.to_json())
    elif args.table:
        with open(args.table) as f:
            table = CostTable.from_json(f.read())
    else:
        ap.error("give --profile or --table")
    res = {"ranks": args.gpus, "matrices": len(shapes)}
    for name, owners in (("round_robin", assign_round_robin(shapes, args.gpus)),
                         ("greedy", assign_greedy(shapes, args.gpus, table))):
        ld = loads(shapes, owners, args.gpus, table)
        res[name] = {"predicted_makespan_ms": max(ld), "predicted_loads_ms": ld}
        if args.validate:
            meas = validate_on_one_gpu(shapes, owners, args.gpus)
            res[name]["measured_loads_ms"] = meas
            res[name]["measured_makespan_ms"] = max(meas)
    res["lower_bound_ms"] = lower_bound(shapes, args.gpus, table)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
