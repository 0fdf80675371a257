"""Scheduling options of muon_step_ex, through the C ABI: the overlapped
schedule of large calls (two chunks, HBM-bound passes on the library's side
stream under the previous chunk's products), the default one-stream
schedule, and the workspace budget (chunks run one after another in one
region) must all give the same weights and momenta bit for bit, step after
step, and the overlapped schedule must replay from a captured HIP graph."""
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

# 16 gate/down-shaped matrices + 8 k-shaped ones: 1.10e9 elements (≥ 2^30, so
# the overlap option splits the call), two Gram groups of m = 3584 and 512
LARGE = [(18944, 3584)] * 8 + [(512, 3584)] * 8 + [(3584, 18944)] * 8


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mns():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import muon_newton_schulz_06_amd as m
    m.load()
    return m


def clone(inp):
    return ([p.clone() for p in inp.params], [g.clone() for g in inp.grads],
            [m.clone() for m in inp.momenta])


def assert_same(a, b, what):
    for j, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), (what, j, tuple(x.shape))


def test_overlapped_equals_one_stream_bitwise(mns):
    assert sum(r * c for r, c in LARGE) >= 1 << 30
    base = W.muon_inputs(LARGE, 6101, device="cuda")
    p1, g1, m1 = clone(base)
    p2, g2, m2 = clone(base)
    del base
    for step in range(2):
        if step:
            g1 = W.fresh_grads(LARGE, 6101, step, device="cuda")
            g2 = [g.clone() for g in g1]
        say("overlapped step", step)
        mns.muon_step(p1, g1, m1, overlap=True)
        say("one-stream step", step)
        mns.muon_step(p2, g2, m2)
        torch.cuda.synchronize()
        assert_same(p1, p2, "weights")
        assert_same(m1, m2, "momentum")


def test_budget_chunks_equal_one_plan_bitwise(mns):
    """A Qwen2.5-7B-shaped layer under a budget of what its largest matrix
    needs alone (every matrix its own chunk, one shared region) against one
    plan, over two steps."""
    shapes = W.qwen_layer_shapes()
    budget = max(mns.step_workspace_size([s]) for s in shapes)
    assert budget < mns.step_workspace_size(shapes)
    base = W.muon_inputs(shapes, 6201, device="cuda")
    p1, g1, m1 = clone(base)
    p2, g2, m2 = clone(base)
    for step in range(2):
        if step:
            g1 = W.fresh_grads(shapes, 6201, step, device="cuda")
            g2 = [g.clone() for g in g1]
        say("budget", budget, "step", step)
        ws = torch.empty(budget, dtype=torch.uint8, device="cuda")
        mns.muon_step(p1, g1, m1, workspace=ws, max_workspace_bytes=budget)
        mns.muon_step(p2, g2, m2)
        torch.cuda.synchronize()
        assert_same(p1, p2, "weights")
        assert_same(m1, m2, "momentum")
    with pytest.raises(mns.MuonError) as ei:
        mns.muon_step(p1, g1, m1, max_workspace_bytes=budget // 4)
    assert ei.value.status_name == "WORKSPACE"


def test_budget_chunks_of_fp32_groups_equal_one_plan_bitwise(mns):
    """Small nearly square matrices run fp32 products on tiles chosen by m
    alone, so chunks of fewer matrices pick the tiles of the whole call and
    the weights match one plan bit for bit."""
    shapes = [(128, 128), (256, 300), (200, 200)] * 4 + [(700, 800)] * 2
    plan = mns.describe_plan(shapes, for_step=True)
    assert {g["m"]: g["op"] for g in plan["groups"]} == {128: "f32", 256: "f32", 200: "f32", 700: "f32"}
    budget = max(mns.step_workspace_size([s]) for s in shapes)
    assert budget < mns.step_workspace_size(shapes)
    base = W.muon_inputs(shapes, 6301, device="cuda")
    p1, g1, m1 = clone(base)
    p2, g2, m2 = clone(base)
    for step in range(2):
        if step:
            g1 = W.fresh_grads(shapes, 6301, step, device="cuda")
            g2 = [g.clone() for g in g1]
        say("fp32 groups, budget", budget, "step", step)
        ws = torch.empty(budget, dtype=torch.uint8, device="cuda")
        mns.muon_step(p1, g1, m1, workspace=ws, max_workspace_bytes=budget)
        mns.muon_step(p2, g2, m2)
        torch.cuda.synchronize()
        assert_same(p1, p2, "weights")
        assert_same(m1, m2, "momentum")


def test_fp32_64_and_128_tiles_give_the_same_bits(mns):
    """The built-in tile of an fp32 group with m > 256 depends on its matrix
    count (64-tiles for small groups, 128 otherwise), which a chunked call
    changes; both kernels add each element's products in the same order, so
    the results must not depend on the choice."""
    xs = [W.gaussian((512, 1024), 31, device="cuda"), W.gaussian((700, 900), 32, device="cuda")]
    res = {}
    try:
        for tile in (64, 128):
            mns.set_tile_table([{"m": 512, "op": "f32", "count_class": 0, "tile": tile},
                                {"m": 700, "op": "f32", "count_class": 0, "tile": tile}])
            p = mns.describe_plan([tuple(x.shape) for x in xs], for_step=False, dtype=torch.float32)
            assert all(g["tile"] == tile for g in p["groups"]), p["groups"]
            say("fp32 groups on", tile, "tiles")
            res[tile] = [o.clone() for o in mns.muon_ns_batched(xs, steps=5)]
            torch.cuda.synchronize()
    finally:
        mns.set_tile_table([])
    for a, b in zip(res[64], res[128]):
        assert torch.equal(a, b), tuple(a.shape)


def test_overlapped_step_graph_replays_match_eager(mns):
    """The overlapped schedule forks to the library's stream and joins back
    with events; captured into a graph (the stream exists after the first
    eager call), three replays equal three eager steps bit for bit."""
    base = W.muon_inputs(LARGE, 6301, device="cuda")
    ws = torch.empty(mns.step_workspace_size(LARGE), dtype=torch.uint8, device="cuda")
    ep, eg, em = clone(base)
    eager = []
    for _ in range(3):
        mns.muon_step(ep, eg, em, workspace=ws, overlap=True)
        eager.append(([p.clone() for p in ep], [m.clone() for m in em]))
    torch.cuda.synchronize()
    del ep, em
    gp, gg, gm = clone(base)
    del base
    torch.cuda.synchronize()
    say("capturing the overlapped step")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_step(gp, gg, gm, workspace=ws, overlap=True)
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        say("replay", step)
        assert_same(gp, eager[step][0], "weights")
        assert_same(gm, eager[step][1], "momentum")


def test_schedules_with_carried_exponents_bitwise(mns):
    """With carried operand exponents too, a matrix's result depends only on
    its own exponent and its Gram group's configuration: the budgeted
    chunks (every matrix its own chunk) and the overlapped schedule equal one
    plan bit for bit over three steps (the first casts, the later two take the
    fused operand), exponents included."""
    shapes = W.qwen_layer_shapes()
    budget = max(mns.step_workspace_size([s]) for s in shapes)
    base = W.muon_inputs(shapes, 6401, device="cuda")
    runs = {name: (clone(base), mns.scale_exp_buffer(len(shapes), "cuda"))
            for name in ("one plan", "budget", "overlap")}
    for step in range(3):
        g = base.grads if step == 0 else W.fresh_grads(shapes, 6401, step, device="cuda")
        for name, ((p, _, m), sx) in runs.items():
            say(name, "step", step)
            kw = {}
            if name == "budget":
                kw = dict(workspace=torch.empty(budget, dtype=torch.uint8, device="cuda"),
                          max_workspace_bytes=budget)
            elif name == "overlap":
                kw = dict(overlap=True)
            mns.muon_step(p, [x.clone() for x in g], m, scale_exp=sx, **kw)
        torch.cuda.synchronize()
        (p0, _, m0), x0 = runs["one plan"]
        for name in ("budget", "overlap"):
            (p, _, m), sx = runs[name]
            assert_same(p, p0, name + " weights")
            assert_same(m, m0, name + " momentum")
            assert torch.equal(sx, x0), (name, "exponents", step)
