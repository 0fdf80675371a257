"""Parity of every planner branch with the fp64 oracle, through the C ABI.

The planner sends a Gram group to one of four kernel configurations:
  * fp32 MFMA (small, nearly square matrices: m ≤ 1024, n ≤ 2m);
  * fp16 operands with fp32 copies of A and P·A on 128×128 tiles (a group
    with 1024 < m ≤ 2048 that holds a nearly square matrix);
  * fp16 operands, state-free, 256×256 tiles (every other group);
  * fp16 operands, state-free, 128×128 tiles (only when a tile table or the
    MUON_TILE override asks for it).
Each is compared here with the oracle at 1, 2 and 5 Newton–Schulz steps,
through muon_ns_batched (bf16 in and out) and through muon_step with fp32
weights that start at zero, so the update −lr·sc·O itself is exposed
(the final product's update epilogue of that configuration included).
Bound: relative Frobenius error ≤ 2e-2 per matrix (half-precision products,
fp32 accumulation).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
Q32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)

# A 1536-group holding a square and a wide matrix, a 2048 square alone, and
# an 1100-group holding a nearly square matrix in both orientations.
STATE32_SHAPES = [(1536, 1536), (2048, 2048), (1100, 2000), (2000, 1100), (1536, 6000)]
# Wide (n > 2m) matrices with m = 600 and m = 2300: state-free groups.
FORCED128_SHAPES = [(600, 1500), (4700, 2300), (600, 1500)]


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


def rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def groups_of(plan):
    return {g["m"]: g for g in plan["groups"]}


def check_ns(mns, shapes, seed0, steps):
    xs = [W.gaussian(s, seed0 + i, dtype=torch.bfloat16) for i, s in enumerate(shapes)]
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=steps)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        ref = oracle.muon_orthogonalize(x.double().numpy(), Q32, steps, 1e-7)
        e = rel(o.double().cpu().numpy(), ref)
        say("ns", tuple(x.shape), "steps", steps, "rel err", e)
        assert e <= TOL_BF16, (tuple(x.shape), steps, e)


def check_step_update(mns, shapes, seed0, steps):
    inp = W.muon_inputs(shapes, seed0, device="cuda", param_dtype=torch.float32)
    for p in inp.params:
        p.zero_()
    host_g = [g.cpu().numpy() for g in inp.grads]
    mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=steps)
    torch.cuda.synchronize()
    for j, (r, c) in enumerate(shapes):
        lrsc = float(np.float32(0.02)) * oracle.lr_shape_scale(r, c)
        O_gpu = -inp.params[j].double().cpu().numpy() / lrsc
        O = oracle.muon_orthogonalize(host_g[j].astype(np.float64), Q32, steps, 1e-7)
        e = rel(O_gpu, O)
        say("step", (r, c), "steps", steps, "rel err of update", e)
        assert e <= TOL_BF16, ((r, c), steps, e)


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_state32_groups_ns(mns, steps):
    plan = mns.describe_plan(STATE32_SHAPES, for_step=False, steps=steps)
    g = groups_of(plan)
    for m in (1536, 2048, 1100):
        assert g[m]["state32"] and g[m]["tile"] == 128 and g[m]["op"] == "f16", g[m]
    assert g[1536]["count"] == 2
    say("fp32-state groups", STATE32_SHAPES, "steps", steps)
    check_ns(mns, STATE32_SHAPES, 8100 + 10 * steps, steps)


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_state32_groups_step_update(mns, steps):
    plan = mns.describe_plan(STATE32_SHAPES, for_step=True, steps=steps)
    g = groups_of(plan)
    for m in (1536, 2048, 1100):
        assert g[m]["state32"] and g[m]["tile"] == 128, g[m]
    say("fp32-state groups through muon_step", STATE32_SHAPES, "steps", steps)
    check_step_update(mns, STATE32_SHAPES, 8200 + 10 * steps, steps)


def _force_128(mns):
    # count classes of the groups below: m = 600 holds 2 matrices (class 1),
    # m = 2300 holds 1 (class 0)
    mns.set_tile_table([{"m": 600, "op": "f16", "count_class": 1, "tile": 128},
                        {"m": 2300, "op": "f16", "count_class": 0, "tile": 128}])
    g = groups_of(mns.describe_plan(FORCED128_SHAPES, for_step=False))
    assert g[600]["tile"] == 128 and not g[600]["state32"], g[600]
    assert g[2300]["tile"] == 128 and not g[2300]["state32"], g[2300]


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_forced_128_tile_state_free_ns(mns, steps):
    try:
        _force_128(mns)
        say("state-free fp16 groups forced onto 128-tiles", FORCED128_SHAPES, "steps", steps)
        check_ns(mns, FORCED128_SHAPES, 8300 + 10 * steps, steps)
    finally:
        mns.set_tile_table([])


@pytest.mark.parametrize("steps", [1, 5])
def test_forced_128_tile_state_free_step_update(mns, steps):
    try:
        _force_128(mns)
        say("state-free 128-tile groups through muon_step", FORCED128_SHAPES, "steps", steps)
        check_step_update(mns, FORCED128_SHAPES, 8400 + 10 * steps, steps)
    finally:
        mns.set_tile_table([])


def test_default_plan_matches_the_documented_policy(mns):
    """The three-way operand policy as the header states it."""
    shapes = [(512, 900), (1024, 1024), (300, 2000), (1536, 1536), (1536, 6000), (2304, 2304),
              (3584, 18944)]
    g = groups_of(mns.describe_plan(shapes, for_step=True))
    assert g[512]["op"] == "f32" and g[1024]["op"] == "f32"          # m ≤ 1024, n ≤ 2m
    assert g[300]["op"] == "f16" and g[300]["tile"] == 256            # wide: state-free
    assert g[1536]["state32"] and g[1536]["tile"] == 128              # 1024 < m ≤ 2048, square
    assert not g[2304]["state32"] and g[2304]["tile"] == 256          # m > 2048
    assert not g[3584]["state32"] and g[3584]["tile"] == 256
