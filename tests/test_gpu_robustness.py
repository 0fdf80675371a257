"""Robustness of the HIP path, through the C ABI:

  * guard canaries: the library writes nothing outside each output matrix
    and nothing beyond the workspace size it asked for, on every planner
    branch (fp32 products, fp32-state 128-tiles, state-free 256-tiles, tall
    and wide, 1×n and n×1);
  * the stored Gram-space iterates are exactly symmetric where they are
    stored symmetric (diagonal blocks of the block-upper iterates, the last
    Q in full, every iterate of a 128-tile group);
  * the serialised-launch debugging mode (MUON_DEBUG_SYNC=1) gives the same
    bits as the default asynchronous mode;
  * a step resumed from saved weights and momentum (through torch.save /
    torch.load, and through the optimiser's state_dict) equals an
    uninterrupted run bit for bit.
"""
import io
import os
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

BRANCH_SHAPES = [(600, 1500), (1536, 1536), (300, 500), (1500, 600), (1, 77), (77, 1), (257, 1025)]
GUARD = 4096  # elements before and after every matrix


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


def guarded(shapes, dtype, sentinel):
    """One buffer holding every matrix with GUARD elements on either side,
    filled with `sentinel`; returns (buffer, views, [(lo, hi)] of the views)."""
    total = sum(GUARD + r * c for r, c in shapes) + GUARD
    buf = torch.full((total,), sentinel, dtype=dtype, device="cuda")
    views, spans, off = [], [], GUARD
    for r, c in shapes:
        views.append(buf[off:off + r * c].view(r, c))
        spans.append((off, off + r * c))
        off += r * c + GUARD
    return buf, views, spans


def guards_intact(buf, spans, sentinel):
    mask = torch.ones(buf.numel(), dtype=torch.bool, device=buf.device)
    for lo, hi in spans:
        mask[lo:hi] = False
    return bool(torch.all(buf[mask] == sentinel))


def test_guard_canaries_ns_batched(mns):
    plan = mns.describe_plan(BRANCH_SHAPES, for_step=False)
    kinds = {(g["op"], g["tile"], g["state32"]) for g in plan["groups"]}
    assert ("f16", 256, False) in kinds and ("f16", 128, True) in kinds and ("f32", 64, False) in kinds
    xs = [W.gaussian(s, 9300 + i, dtype=torch.bfloat16, device="cuda") for i, s in enumerate(BRANCH_SHAPES)]
    buf, outs, spans = guarded(BRANCH_SHAPES, torch.bfloat16, -7.0)
    need = mns.ns_workspace_size(BRANCH_SHAPES)
    ws_all = torch.full((need + 65536,), 0xA5, dtype=torch.uint8, device="cuda")
    say("muon_ns_batched with guarded outputs", BRANCH_SHAPES, "workspace", need)
    mns.muon_ns_batched(xs, outs=outs, steps=5, workspace=ws_all[:need])
    torch.cuda.synchronize()
    assert guards_intact(buf, spans, -7.0), "an output was written outside its matrix"
    assert bool(torch.all(ws_all[need:] == 0xA5)), "workspace written beyond its size"
    ref = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


def test_guard_canaries_step(mns):
    shapes = BRANCH_SHAPES
    inp = W.muon_inputs(shapes, 9400, device="cuda")
    pbuf, params, pspans = guarded(shapes, torch.bfloat16, 3.0)
    mbuf, moms, mspans = guarded(shapes, torch.float32, -5.0)
    for p, q in zip(params, inp.params):
        p.copy_(q)
    for m in moms:
        m.zero_()
    need = mns.step_workspace_size(shapes)
    ws_all = torch.full((need + 65536,), 0x5A, dtype=torch.uint8, device="cuda")
    say("muon_step with guarded weights and momenta", shapes)
    mns.muon_step(params, inp.grads, moms, workspace=ws_all[:need])
    torch.cuda.synchronize()
    assert guards_intact(pbuf, pspans, 3.0), "a weight was written outside its matrix"
    assert guards_intact(mbuf, mspans, -5.0), "a momentum was written outside its matrix"
    assert bool(torch.all(ws_all[need:] == 0x5A)), "workspace written beyond its size"
    ref_p = [p.clone() for p in inp.params]
    ref_m = [m.clone() for m in inp.momenta]
    mns.muon_step(ref_p, inp.grads, ref_m)
    torch.cuda.synchronize()
    for a, b in zip(params, ref_p):
        assert torch.equal(a, b)
    for a, b in zip(moms, ref_m):
        assert torch.equal(a, b)


def _iterate(ws, off, mp, dtype=torch.float16):
    n = mp * mp * torch.finfo(dtype).bits // 8
    return ws[off:off + n].view(dtype).view(mp, mp)


@pytest.mark.parametrize("steps", [1, 4, 5])
def test_stored_iterates_exactly_symmetric(mns, steps):
    """256-tile group (m = 600, Mp = 768): diagonal 256-blocks of the A, B and
    P·A copies and the whole last Q are exactly symmetric; 128-tile group
    (m = 1536, fp32 state): every fp16 iterate copy is exactly symmetric."""
    shapes = [(600, 1500), (1536, 1536)]
    xs = [W.gaussian(s, 9500 + i, dtype=torch.bfloat16, device="cuda") for i, s in enumerate(shapes)]
    plan = mns.describe_plan(shapes, for_step=False, steps=steps)
    need = mns.ns_workspace_size(shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    mns.muon_ns_batched(xs, steps=steps, workspace=ws)
    torch.cuda.synchronize()
    qlast = (steps - 1) & 1
    for g in plan["groups"]:
        mp = g["Mp"]
        say("group m", g["m"], "tile", g["tile"], "steps", steps)
        Q = _iterate(ws, g["offQh"][qlast], mp)
        assert torch.equal(Q, Q.t()), "last Q not exactly symmetric"
        assert float(Q.float().abs().max()) > 0
        bufs = [g["offBh"]] + ([g["offAh"], g["offPAh"]] if steps >= 2 else [g["offAh"]])
        for off in bufs:
            Y = _iterate(ws, off, mp)
            if g["tile"] == 256:
                for b in range(mp // 256):
                    blk = Y[256 * b:256 * b + 256, 256 * b:256 * b + 256]
                    assert torch.equal(blk, blk.t()), ("diagonal block", off, b)
            else:
                assert torch.equal(Y, Y.t()), ("iterate", off)


def test_debug_sync_mode_matches_async(mns):
    shapes = [(96, 200), (1536, 1536), (600, 1500), (300, 500)]
    inp = W.muon_inputs(shapes, 9600, device="cuda")
    p1, m1 = [p.clone() for p in inp.params], [m.clone() for m in inp.momenta]
    p2, m2 = [p.clone() for p in inp.params], [m.clone() for m in inp.momenta]
    mns.muon_step(p1, inp.grads, m1)
    torch.cuda.synchronize()
    os.environ["MUON_DEBUG_SYNC"] = "1"
    try:
        say("serialised launches")
        mns.muon_step(p2, inp.grads, m2)
        outs = mns.muon_ns_batched([p.float() for p in inp.params], steps=5)
    finally:
        del os.environ["MUON_DEBUG_SYNC"]
    torch.cuda.synchronize()
    ref = mns.muon_ns_batched([p.float() for p in inp.params], steps=5)
    torch.cuda.synchronize()
    for a, b in zip(p1, p2):
        assert torch.equal(a, b)
    for a, b in zip(m1, m2):
        assert torch.equal(a, b)
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


def test_resume_from_saved_state_bitwise(mns):
    shapes = [(512, 3584), (3584, 512), (700, 700), (300, 1000)]
    inp = W.muon_inputs(shapes, 9700, device="cuda")
    g2 = W.fresh_grads(shapes, 9700, 1, device="cuda")
    # uninterrupted: two steps
    pa, ma = [p.clone() for p in inp.params], [m.clone() for m in inp.momenta]
    mns.muon_step(pa, inp.grads, ma)
    mns.muon_step(pa, g2, ma)
    # interrupted: one step, save to bytes on the host, reload into new tensors, one step
    pb, mb = [p.clone() for p in inp.params], [m.clone() for m in inp.momenta]
    mns.muon_step(pb, inp.grads, mb)
    torch.cuda.synchronize()
    blob = io.BytesIO()
    torch.save({"params": [p.cpu() for p in pb], "momenta": [m.cpu() for m in mb]}, blob)
    del pb, mb
    blob.seek(0)
    st = torch.load(blob, weights_only=True)
    pc = [p.cuda() for p in st["params"]]
    mc = [m.cuda() for m in st["momenta"]]
    say("resumed step")
    mns.muon_step(pc, g2, mc)
    torch.cuda.synchronize()
    for a, b in zip(pa, pc):
        assert torch.equal(a, b)
    for a, b in zip(ma, mc):
        assert torch.equal(a, b)


def test_optimizer_state_dict_resume_bitwise(mns):
    shapes = [(256, 1024), (1024, 256), (512, 512)]
    inp = W.muon_inputs(shapes, 9800, device="cuda", param_dtype=torch.float32)
    g2 = W.fresh_grads(shapes, 9800, 1, device="cuda")

    def make(ps):
        ws = [torch.nn.Parameter(p.clone()) for p in ps]
        return ws, mns.Muon(ws, lr=0.02, momentum=0.95, nesterov=True, weight_decay=0.01)

    wa, oa = make(inp.params)
    for g in (inp.grads, g2):
        for w, gg in zip(wa, g):
            w.grad = gg.clone()
        oa.step()
    wb, ob = make(inp.params)
    for w, gg in zip(wb, inp.grads):
        w.grad = gg.clone()
    ob.step()
    torch.cuda.synchronize()
    blob = io.BytesIO()
    torch.save({"w": [w.detach().cpu() for w in wb], "opt": ob.state_dict()}, blob)
    blob.seek(0)
    st = torch.load(blob, weights_only=True)
    wc, oc = make([w.cuda() for w in st["w"]])
    oc.load_state_dict(st["opt"])
    for w, gg in zip(wc, g2):
        w.grad = gg.clone()
    say("optimiser resumed from its state_dict")
    oc.step()
    torch.cuda.synchronize()
    for a, b in zip(wa, wc):
        assert torch.equal(a.detach(), b.detach())
