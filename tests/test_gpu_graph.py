"""The entry points enqueue only kernel launches on the caller's stream (no
allocation, no memset, no host synchronisation), so a whole muon_step can be
captured into a HIP graph and replayed.  Each replay is checked bitwise
against the eager step it stands for, with eager work and synchronisations
between the replays."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mns():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import muon_newton_schulz_06_amd as m
    m.load()
    return m


def test_muon_step_graph_replays_match_eager(mns):
    shapes = [(256, 1024), (1024, 256), (128, 128), (512, 3584), (300, 700)]
    base = W.muon_inputs(shapes, 123, device="cuda")
    ws = torch.empty(mns.step_workspace_size(shapes), dtype=torch.uint8, device="cuda")

    def clone(inp):
        return ([p.clone() for p in inp.params], [g.clone() for g in inp.grads],
                [m.clone() for m in inp.momenta])

    # eager reference: three steps with the same gradients
    ep, eg, em = clone(base)
    eager = []
    for _ in range(3):
        mns.muon_step(ep, eg, em, workspace=ws, nesterov=True, weight_decay=0.01)
        eager.append(([p.clone() for p in ep], [m.clone() for m in em]))
    torch.cuda.synchronize()

    gp, gg, gm = clone(base)
    ws2 = torch.empty_like(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_step(gp, gg, gm, workspace=ws2, nesterov=True, weight_decay=0.01)
    # capture records the launches without running them
    assert all(torch.equal(p, q) for p, q in zip(gp, base.params))
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for j in range(len(shapes)):
            assert torch.equal(gp[j], eager[step][0][j]), ("weights", step, j)
            assert torch.equal(gm[j], eager[step][1][j]), ("momentum", step, j)


def test_selected_step_graph_replays_match_eager(mns):
    """muon_step_selected also enqueues kernels only (score pass, top-k,
    gather, the batched pipeline, scatter): three graph replays equal three
    eager steps bit for bit."""
    shapes = [(256, 1024), (1024, 256), (300, 700), (64, 64)]
    base = W.selected_inputs(shapes, 321, device="cuda", m_std=1e-2)
    ws = torch.empty(mns.step_selected_workspace_size(shapes, 0.25), dtype=torch.uint8, device="cuda")

    def clone(inp):
        return ([p.clone() for p in inp.params], [g.clone() for g in inp.grads],
                [m.clone() for m in inp.momenta])

    ep, eg, em = clone(base)
    eager = []
    for _ in range(3):
        mns.muon_step_selected(ep, eg, em, fraction=0.25, workspace=ws)
        eager.append(([p.clone() for p in ep], [m.clone() for m in em]))
    torch.cuda.synchronize()

    gp, gg, gm = clone(base)
    ws2 = torch.empty_like(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_step_selected(gp, gg, gm, fraction=0.25, workspace=ws2)
    assert all(torch.equal(p, q) for p, q in zip(gp, base.params))
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for j in range(len(shapes)):
            assert torch.equal(gp[j], eager[step][0][j]), ("weights", step, j)
            assert torch.equal(gm[j], eager[step][1][j]), ("buffer", step, j)


def test_muon_step_with_carried_exponents_graph_replays_match_eager(mns):
    """With scale_exp the call reads and rewrites the exponent array on the
    device only, so the captured step carries the exponents from replay to
    replay: three replays (the first casts, the later two take the fused
    operand) equal three eager steps bit for bit, exponents included."""
    shapes = [(256, 1024), (1024, 256), (128, 128), (512, 3584), (3584, 512), (300, 700)]
    base = W.muon_inputs(shapes, 124, device="cuda")
    ws = torch.empty(mns.step_workspace_size(shapes), dtype=torch.uint8, device="cuda")

    def clone(inp):
        return ([p.clone() for p in inp.params], [g.clone() for g in inp.grads],
                [m.clone() for m in inp.momenta])

    ep, eg, em = clone(base)
    ex = mns.scale_exp_buffer(len(shapes), "cuda")
    eager = []
    for _ in range(3):
        mns.muon_step(ep, eg, em, workspace=ws, scale_exp=ex)
        eager.append(([p.clone() for p in ep], [m.clone() for m in em], ex.clone()))
    torch.cuda.synchronize()

    gp, gg, gm = clone(base)
    gx = mns.scale_exp_buffer(len(shapes), "cuda")
    ws2 = torch.empty_like(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_step(gp, gg, gm, workspace=ws2, scale_exp=gx)
    assert all(torch.equal(p, q) for p, q in zip(gp, base.params))
    assert int(gx[0]) == mns.SCALE_EXP_UNKNOWN
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(gx, eager[step][2]), ("exponents", step)
        for j in range(len(shapes)):
            assert torch.equal(gp[j], eager[step][0][j]), ("weights", step, j)
            assert torch.equal(gm[j], eager[step][1][j]), ("momentum", step, j)
