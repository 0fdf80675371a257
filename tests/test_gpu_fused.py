"""Carried operand exponents (muon_step_ex opts.scale_exp), through the C ABI.

With scale_exp the momentum pass of a matrix on the fp16 256-tile path writes
the MFMA operand u·2^e itself; the norm finish keeps it when ‖u‖·2^e lies in
[2^9, 2^14] and otherwise the matrix is cast as without scale_exp.  These
tests check what the call records and how it falls back:
  * after a step every fusable entry holds the exponent that puts the
    momentum's norm (computed here in fp64) in [2^12, 2^13); entries of
    other paths and of empty matrices are left as they were;
  * a known, an out-of-range (both directions) and an unknown exponent give
    bitwise identical momenta; the three fallbacks give bitwise identical
    weights, and the fused step agrees with them to the 2e-2 tolerance of the
    orthogonalised update (its weight change against theirs);
  * a zero momentum records "unknown" and leaves the weights unchanged;
  * two runs from the same state and exponents are bitwise identical.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

# wide and tall 256-tile shapes, an fp32 group (384², nearly square and
# small), a 128-tile group with fp32 state (1536²) and an empty matrix
SHAPES = [(300, 1200), (1100, 256), (384, 384), (1536, 1536), (0, 7), (2304, 512)]
FUSABLE = [0, 1, 5]
OTHER = [2, 3, 4]


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


def _state(seed):
    inp = W.muon_inputs(SHAPES, seed, device="cuda", param_dtype=torch.float32)
    return inp


def _clone(ts):
    return [t.clone() for t in ts]


def _step(mns, params, grads, momenta, sx):
    mns.muon_step(params, grads, momenta, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
    torch.cuda.synchronize()


def test_exponents_are_recorded(mns):
    inp = _state(5100)
    sx = mns.scale_exp_buffer(len(SHAPES), "cuda")
    sx[4] = 77  # empty matrix: its entry is never touched
    say("one step from unknown exponents over", SHAPES)
    _step(mns, inp.params, inp.grads, inp.momenta, sx)
    e = sx.cpu().tolist()
    for j in FUSABLE:
        nrm = float(np.linalg.norm(inp.momenta[j].double().cpu().numpy()))
        x = math.ldexp(nrm, e[j])
        say("matrix", SHAPES[j], "exponent", e[j], "norm·2^e", x)
        assert 2.0**12 * (1 - 1e-6) <= x < 2.0**13 * (1 + 1e-6)
    assert e[2] == e[3] == mns.SCALE_EXP_UNKNOWN
    assert e[4] == 77


def test_fallbacks_agree_and_fused_step_follows(mns):
    inp = _state(5200)
    sx = mns.scale_exp_buffer(len(SHAPES), "cuda")
    _step(mns, inp.params, inp.grads, inp.momenta, sx)  # records the exponents
    known = sx.clone()
    grads = W.fresh_grads(SHAPES, 5200, 1, device="cuda")
    P0, M0 = _clone(inp.params), _clone(inp.momenta)
    runs = {}
    for name, fill in [("known", None), ("high", 100), ("low", -100), ("unknown", mns.SCALE_EXP_UNKNOWN)]:
        e = known.clone()
        if fill is not None:
            for j in FUSABLE:
                e[j] = fill
        P, M = _clone(P0), _clone(M0)
        say("second step with", name, "exponents", e.cpu().tolist())
        _step(mns, P, grads, M, e)
        runs[name] = (P, M, e.cpu().tolist())
    base_P, base_M, base_e = runs["known"]
    for name in ("high", "low", "unknown"):
        P, M, e = runs[name]
        for j in range(len(SHAPES)):
            assert torch.equal(M[j], base_M[j]), ("momentum", name, j)
        # rejected or unknown: cast as without scale_exp, so all three agree
        # bit for bit, and each records the same next exponent
        for j in range(len(SHAPES)):
            assert torch.equal(P[j], runs["unknown"][0][j]), ("fallback weights", name, j)
        assert e == base_e, (name, e, base_e)
    for j in FUSABLE:
        d_fused = (base_P[j] - P0[j]).double()
        d_cast = (runs["unknown"][0][j] - P0[j]).double()
        r = float(torch.linalg.norm(d_fused - d_cast) / torch.linalg.norm(d_cast))
        say("matrix", SHAPES[j], "fused vs cast update rel diff", r)
        assert r <= 2e-2
    # paths that never fuse: identical in all four runs
    for j in OTHER:
        assert torch.equal(base_P[j], runs["unknown"][0][j]), ("non-fusable", j)


def test_zero_momentum_records_unknown(mns):
    shapes = [(256, 1024), (1024, 256)]
    P = [torch.randn(r, c, device="cuda") * 0.02 for r, c in shapes]
    P0 = _clone(P)
    G = [torch.zeros(r, c, device="cuda") for r, c in shapes]
    M = [torch.zeros(r, c, device="cuda") for r, c in shapes]
    sx = torch.tensor([5, -3], dtype=torch.int32, device="cuda")
    say("zero gradients and momenta, exponents", sx.cpu().tolist())
    mns.muon_step(P, G, M, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
    torch.cuda.synchronize()
    assert sx.cpu().tolist() == [mns.SCALE_EXP_UNKNOWN] * 2
    for p, p0 in zip(P, P0):
        assert torch.isfinite(p).all()
        assert torch.equal(p, p0)


def test_run_to_run_bitwise(mns):
    inp = _state(5300)
    sx = mns.scale_exp_buffer(len(SHAPES), "cuda")
    _step(mns, inp.params, inp.grads, inp.momenta, sx)
    grads = W.fresh_grads(SHAPES, 5300, 1, device="cuda")
    outs = []
    for r in range(2):
        P, M, e = _clone(inp.params), _clone(inp.momenta), sx.clone()
        say("fused step, run", r)
        _step(mns, P, grads, M, e)
        outs.append((P, M, e))
    for j in range(len(SHAPES)):
        assert torch.equal(outs[0][0][j], outs[1][0][j])
        assert torch.equal(outs[0][1][j], outs[1][1][j])
    assert torch.equal(outs[0][2], outs[1][2])
