"""Concurrent lanes through the C ABI: a call's results do not depend on how
its matrices are split over the library's streams (MUON_LANES = 1 … 4 give
the same bits, for muon_ns_batched and muon_step, over two steps), the
default split of an under-filled call matches the oracle, and a call that
forks lanes replays bitwise from a captured HIP graph."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

Q32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)


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


@pytest.fixture(autouse=True)
def _env():
    old = os.environ.pop("MUON_LANES", None)
    yield
    os.environ.pop("MUON_LANES", None)
    if old is not None:
        os.environ["MUON_LANES"] = old


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_ns_batched_lane_counts_bitwise(mns):
    xs = W.ns_small_mix(device="cuda", tall_every_other=True)
    ref = None
    for lanes in ("1", "2", "3", "4"):
        os.environ["MUON_LANES"] = lanes
        say("small mix, lanes", lanes)
        outs = mns.muon_ns_batched(xs, steps=5)
        torch.cuda.synchronize()
        if ref is None:
            ref = outs
            continue
        for j, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (lanes, j, tuple(a.shape))


def test_default_lanes_match_oracle(mns):
    shapes = [(512, 2048)] * 6 + [(256, 1024)] * 5 + [(1100, 300), (96, 4000)]
    assert len(mns.describe_plan(shapes, for_step=False)["lanes"]) >= 2
    xs = [W.gaussian(s, 7100 + i, dtype=torch.bfloat16, device="cuda") for i, s in enumerate(shapes)]
    say("default lanes", len(mns.describe_plan(shapes, for_step=False)["lanes"]))
    outs = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for i in (0, 5, 6, 10, 11, 12):
        want = oracle.muon_orthogonalize(xs[i].float().cpu().numpy(), Q32, 5, 1e-7)
        e = rel(outs[i].float().cpu().numpy(), want)
        say("matrix", i, shapes[i], "rel err", e)
        assert e <= 2e-2


def test_step_lane_counts_bitwise_two_steps(mns):
    shapes = W.qwen_layer_shapes()
    base = W.muon_inputs(shapes, 7200, device="cuda")
    g2 = W.fresh_grads(shapes, 7200, 1, device="cuda")
    ref = None
    for lanes in ("1", "2", "3"):
        os.environ["MUON_LANES"] = lanes
        say("one Qwen layer, lanes", lanes)
        ps = [p.clone() for p in base.params]
        ms = [m.clone() for m in base.momenta]
        mns.muon_step(ps, base.grads, ms)
        mns.muon_step(ps, g2, ms)
        torch.cuda.synchronize()
        if ref is None:
            ref = (ps, ms)
            continue
        for j in range(len(shapes)):
            assert torch.equal(ps[j], ref[0][j]), ("weights", lanes, j)
            assert torch.equal(ms[j], ref[1][j]), ("momentum", lanes, j)


def test_lanes_graph_replays_match_eager(mns):
    """The uniform batch forks two lanes by default; after an eager call has
    created the lanes' streams, a captured call replays bitwise equal to the
    eager result three times, with other work between the replays."""
    xs = W.ns_uniform_batch(count=32, device="cuda")
    assert len(mns.describe_plan([tuple(x.shape) for x in xs], for_step=False)["lanes"]) == 2
    need = mns.ns_workspace_size([tuple(x.shape) for x in xs])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    eager = [torch.empty_like(x) for x in xs]
    mns.muon_ns_batched(xs, outs=eager, steps=5, workspace=ws)
    torch.cuda.synchronize()
    outs = [torch.empty_like(x) for x in xs]
    say("capturing a two-lane call")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_ns_batched(xs, outs=outs, steps=5, workspace=ws)
    for r in range(3):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        say("replay", r)
        for j, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (r, j)
