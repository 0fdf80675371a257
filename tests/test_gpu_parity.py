"""Parity of the HIP path with the fp64 CPU oracle, through the C ABI.

Bounds: relative Frobenius error per matrix ≤ 1e-4 for fp32 storage (fp32
MFMA), ≤ 2e-2 for bf16 storage (half-precision MFMA, fp32 accumulation).
Weights after a step: every bf16 value is the correct rounding of an update
within the elementwise band of the oracle's (see weights_consistent), and the
update itself is checked in Frobenius norm through fp32 weights.  Momentum:
within 1 fp32 ulp.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from checks import weights_consistent

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


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


def rel(gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy() if torch.is_tensor(gpu) else gpu
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm(g - ref)
    n = np.linalg.norm(ref)
    return d / n if n > 0 else d


def oracle_ns(x_cpu, steps=5, coeffs=oracle.QUINTIC, eps=1e-7):
    c32 = tuple(float(np.float32(v)) for v in coeffs)  # what the library receives
    return oracle.muon_orthogonalize(x_cpu.to(torch.float64).numpy(), c32, steps, eps)


# ------------------------------------------------------------------ fp32 path
def test_fp32_single_quintic(mns):
    say("fp32 256x1024 quintic 5 steps")
    x = W.ns_single()
    out = mns.muon_ns_batched([x.cuda()], steps=5)[0]
    torch.cuda.synchronize()
    e = rel(out, oracle_ns(x))
    say("rel err", e)
    assert e <= TOL_F32


def test_fp32_single_cubic_vs_svd(mns):
    say("fp32 256x1024 cubic 30 steps vs SVD")
    x = W.ns_single()
    out = mns.muon_ns_batched([x.cuda()], steps=30, coeffs=mns.CUBIC)[0]
    torch.cuda.synchronize()
    e_svd = rel(out, oracle.polar_svd(x.double().numpy()))
    e_ns = rel(out, oracle_ns(x, steps=30, coeffs=oracle.CUBIC))
    say("rel err vs svd", e_svd, "vs oracle NS", e_ns)
    assert e_svd <= TOL_F32 and e_ns <= TOL_F32


def test_fp32_ragged_tall_wide(mns):
    shapes = [(200, 333), (333, 200), (130, 130), (1, 77), (77, 1), (257, 1025)]
    say("fp32 ragged", shapes)
    xs = [W.gaussian(s, 50 + i) for i, s in enumerate(shapes)]
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=5)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        e = rel(o, oracle_ns(x))
        say(tuple(x.shape), e)
        assert e <= TOL_F32


def test_fp32_split_contraction_tiles(mns):
    """fp32 groups with m ≤ 256 run on 32-tiles whose contraction is split
    over four waves: several tiles per matrix, ragged m padded to 64, long
    SYRK contractions (n up to 4096), a tall input and a 40-matrix group (one
    launch over many matrices), each matrix against the oracle."""
    shapes = [(250, 3000), (96, 4096), (256, 256), (1000, 160), (33, 70)] + [(64, 200)] * 40
    plan = mns.describe_plan(shapes, for_step=False, dtype=torch.float32)
    assert all(g["tile"] == 32 for g in plan["groups"]), plan["groups"]
    say("fp32 32-tile path", shapes[:5], "+ 40 x (64, 200)")
    xs = [W.gaussian(s, 900 + i) for i, s in enumerate(shapes)]
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=5)
    torch.cuda.synchronize()
    for i, (x, o) in enumerate(zip(xs, outs)):
        if i >= 5 and i % 13:
            continue  # a sample of the group
        e = rel(o, oracle_ns(x))
        say(tuple(x.shape), e)
        assert e <= TOL_F32


# ------------------------------------------------------------------ bf16 path
def test_bf16_ragged_mixed_batch(mns):
    shapes = [(300, 700), (700, 300), (129, 129), (1, 513), (513, 1), (64, 4096),
              (4096, 64), (384, 1000), (255, 256), (256, 255)]
    say("bf16 ragged mix", shapes)
    xs = [W.gaussian(s, 100 + i, dtype=torch.bfloat16) for i, s in enumerate(shapes)]
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=5)
    torch.cuda.synchronize()
    worst = 0
    for x, o in zip(xs, outs):
        e = rel(o.float(), oracle_ns(x.float()))
        say(tuple(x.shape), e)
        worst = max(worst, e)
        assert e <= TOL_BF16
    say("worst", worst)


def test_bf16_square_without_fp32_state(mns):
    """Gram size above the fp32-state limit (2048): the 256-tile, state-free
    path on a square matrix, the worst-conditioned Gram case."""
    say("bf16 2304x2304 square, state-free Gram path")
    x = W.gaussian((2304, 2304), 77, dtype=torch.bfloat16)
    o = mns.muon_ns_batched([x.cuda()], steps=5)[0]
    torch.cuda.synchronize()
    e = rel(o.float(), oracle_ns(x.float()))
    say("rel err", e)
    assert e <= TOL_BF16


def test_row_vector_closed_form(mns):
    """m = 1: O = φ^5(1)·x/‖x‖ (one singular value, equal to 1)."""
    say("fp32 row/column vector closed form")
    x = W.gaussian((1, 300), 7)
    phi5 = oracle.scalar_map(1.0, oracle.QUINTIC, 5)
    want = phi5 * x.double().numpy() / np.linalg.norm(x.double().numpy())
    o1, o2 = mns.muon_ns_batched([x.cuda(), x.t().contiguous().cuda()], steps=5)
    torch.cuda.synchronize()
    assert rel(o1, want) <= TOL_F32
    assert rel(o2, want.T) <= TOL_F32


def test_uniform_batch_sampled_and_batch_invariant(mns):
    say("bf16 32x(1024x4096) batch")
    xs = W.ns_uniform_batch(device="cuda")
    outs = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for i in (0, 13, 31):
        e = rel(outs[i].float(), oracle_ns(xs[i].float().cpu()))
        say("matrix", i, "rel err", e)
        assert e <= TOL_BF16
    say("batch invariance: matrix 13 alone")
    alone = mns.muon_ns_batched([xs[13]], steps=5)[0]
    torch.cuda.synchronize()
    assert torch.equal(alone, outs[13])


def test_small_mix_all_matrices(mns):
    say("bf16 heterogeneous 176-matrix batch (shuffled)")
    xs = W.ns_small_mix(device="cuda")
    outs = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    worst = 0
    for x, o in zip(xs, outs):
        e = rel(o.float(), oracle_ns(x.float().cpu()))
        worst = max(worst, e)
        assert e <= TOL_BF16, (tuple(x.shape), e)
    say("worst", worst)


def test_small_mix_tall_variant(mns):
    say("bf16 heterogeneous batch, every other matrix stored tall")
    xs = W.ns_small_mix(device="cuda", tall_every_other=True)
    outs = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for k in range(0, len(xs), 7):
        e = rel(outs[k].float(), oracle_ns(xs[k].float().cpu()))
        assert e <= TOL_BF16, (tuple(xs[k].shape), e)


# ------------------------------------------------------------------ edge cases
def test_edge_cases(mns):
    say("edge: empty list")
    assert mns.muon_ns_batched([], steps=5) == []
    say("edge: empty matrix inside a batch, zero matrix, steps=0")
    xs = [torch.zeros((0, 5), device="cuda", dtype=torch.bfloat16),
          torch.zeros((40, 60), device="cuda", dtype=torch.bfloat16),
          W.gaussian((50, 90), 3, dtype=torch.bfloat16, device="cuda")]
    outs = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    assert outs[0].shape == (0, 5)
    assert torch.count_nonzero(outs[1]) == 0
    assert rel(outs[2].float(), oracle_ns(xs[2].float().cpu())) <= TOL_BF16
    x = W.gaussian((70, 130), 4, device="cuda")
    o0 = mns.muon_ns_batched([x], steps=0)[0]
    torch.cuda.synchronize()
    assert rel(o0, oracle_ns(x.cpu(), steps=0)) <= TOL_F32
    say("edge: NaN propagates")
    y = W.gaussian((64, 128), 5, device="cuda")
    y[3, 7] = float("nan")
    oy = mns.muon_ns_batched([y], steps=5)[0]
    torch.cuda.synchronize()
    assert torch.isnan(oy).any()
    say("edge: in-place and strided input")
    big = W.gaussian((100, 300), 6, device="cuda")
    view = big[:, 50:250]
    ref = oracle_ns(view.cpu())
    o = mns.muon_ns_batched([view], outs=[view], steps=5)[0]
    torch.cuda.synchronize()
    assert rel(o, ref) <= TOL_F32


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 7])
def test_step_counts_on_the_256_tile_path(mns, steps):
    """bf16 matrices with m = 600 (3×3 blocks of 256 after padding) and
    m = 2300 (9×9): the Gram iterates are stored as their upper blocks and
    read back through transposed panels; which products run, and which one
    writes the last Q in full for the final product, depend on the step
    count."""
    xs = [W.gaussian((600, 1500), 40 + steps, dtype=torch.bfloat16, device="cuda"),
          W.gaussian((4700, 2300), 50 + steps, dtype=torch.bfloat16, device="cuda")]
    plan = mns.describe_plan([tuple(x.shape) for x in xs], for_step=False)
    assert all(g["tile"] == 256 and not g["state32"] for g in plan["groups"])
    say("steps", steps, "shapes", [tuple(x.shape) for x in xs])
    outs = mns.muon_ns_batched(xs, steps=steps)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        e = rel(o.float(), oracle_ns(x.float().cpu(), steps=steps))
        say("steps", steps, tuple(x.shape), "rel err", e)
        assert e <= TOL_BF16


def test_run_to_run_bitwise_determinism(mns):
    say("determinism")
    xs = W.ns_small_mix(device="cuda", mix=[(4, 256, 1024), (3, 512, 2048)])
    a = mns.muon_ns_batched(xs, steps=5)
    b = mns.muon_ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ muon_step
def _check_step(mns, shapes, seed0, check_idx, nsteps=2, nesterov=False, weight_decay=0.0,
                grad_dtype=torch.float32, fused=False):
    inp = W.muon_inputs(shapes, seed0, device="cuda")
    # carried operand exponents: the first step casts and records them, the
    # later ones have the momentum pass write the fp16 operand
    sx = mns.scale_exp_buffer(len(shapes), "cuda") if fused else None
    host_W = [p.float().cpu().double().numpy() for p in inp.params]
    host_M = [m.cpu().numpy() for m in inp.momenta]
    lr32, wd32 = float(np.float32(0.02)), float(np.float32(weight_decay))
    decay = 1.0 - lr32 * wd32
    for step in range(nsteps):
        grads = inp.grads if step == 0 else W.fresh_grads(shapes, seed0, step, device="cuda")
        grads = [g.to(grad_dtype) for g in grads]
        host_g = [g.float().cpu().numpy() for g in grads]
        say("muon_step", step, "over", len(shapes), "matrices", "nesterov", nesterov,
            "weight_decay", weight_decay, "grads", grad_dtype, "carried exponents", fused)
        mns.muon_step(inp.params, grads, inp.momenta, beta=0.95, lr=0.02, steps=5,
                      nesterov=nesterov, weight_decay=weight_decay, scale_exp=sx)
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            Mn = oracle.momentum_update(host_M[j], host_g[j], np.float32(0.95))
            got = inp.momenta[j].cpu().numpy()
            ulp = np.spacing(np.abs(Mn).astype(np.float32))
            assert np.all(np.abs(got.astype(np.float64) - Mn) <= ulp), ("momentum", j)
            host_M[j] = got
        for j in check_idx:
            U = host_M[j].astype(np.float64)
            if nesterov:
                U = host_g[j].astype(np.float64) + float(np.float32(0.95)) * U
            O = oracle.muon_orthogonalize(U, tuple(float(np.float32(v)) for v in oracle.QUINTIC), 5, 1e-7)
            r, c = shapes[j]
            lrsc = lr32 * oracle.lr_shape_scale(r, c)
            got = inp.params[j].float().cpu().double().numpy()
            ok, frac, expect = weights_consistent(host_W[j], got, O, lrsc, decay=decay)
            say("weights", shapes[j], "consistent", ok, "fraction != oracle rounding", frac,
                "bound", expect)
            assert ok
            assert frac <= expect
        host_W = [p.float().cpu().double().numpy() for p in inp.params]


def test_muon_step_small_shapes(mns):
    shapes = [(96, 200), (200, 96), (128, 128), (1, 64), (300, 1000)]
    _check_step(mns, shapes, 900, range(len(shapes)))


def test_muon_step_seeded_random_shapes(mns):
    """Thirty seeded random shapes (each side 1–500) through two full steps."""
    import random
    rng = random.Random(11)
    shapes = [(rng.randint(1, 500), rng.randint(1, 500)) for _ in range(30)]
    _check_step(mns, shapes, 1300, range(len(shapes)))


def test_muon_step_qwen_layer(mns):
    shapes = W.qwen_layer_shapes()
    _check_step(mns, shapes, 4001, check_idx=[1, 0], nsteps=2)


@pytest.mark.parametrize("nesterov,weight_decay,grad_dtype", [
    (True, 0.0, torch.float32),
    (False, 0.1, torch.float32),
    (False, 0.0, torch.bfloat16),
    (True, 0.1, torch.bfloat16),
])
def test_muon_step_variants(mns, nesterov, weight_decay, grad_dtype):
    """muon_step_ex: Nesterov input, decoupled weight decay and bf16
    gradients, against the oracle's definitions, over two steps (the second
    step is where the Nesterov input differs from the plain one)."""
    shapes = [(96, 200), (200, 96), (256, 256), (300, 1000), (1, 64), (2304, 512)]
    if nesterov and weight_decay:
        shapes.append((2304, 2304))  # the 256-tile kernels (weights prefetched in the update)
    _check_step(mns, shapes, 950, range(len(shapes)), nsteps=2, nesterov=nesterov,
                weight_decay=weight_decay, grad_dtype=grad_dtype)


@pytest.mark.parametrize("nesterov,weight_decay,grad_dtype", [
    (False, 0.0, torch.float32),
    (True, 0.1, torch.bfloat16),
])
def test_muon_step_carried_exponents(mns, nesterov, weight_decay, grad_dtype):
    """muon_step with scale_exp over three steps (the first casts and records
    the exponents, the later two take the operand the momentum pass wrote):
    wide, tall and ragged shapes on the fp16 256-tile path next to an fp32
    group and a 128-tile group, element by element against the oracle."""
    shapes = [(300, 1200), (1100, 256), (96, 200), (384, 384), (600, 1500), (2304, 512),
              (513, 2100), (1536, 1536), (1, 64)]
    _check_step(mns, shapes, 970, range(len(shapes)), nsteps=3, nesterov=nesterov,
                weight_decay=weight_decay, grad_dtype=grad_dtype, fused=True)


def test_muon_step_qwen_layer_carried_exponents(mns):
    shapes = W.qwen_layer_shapes()
    _check_step(mns, shapes, 4003, check_idx=[1, 0], nsteps=2, fused=True)


def test_muon_step_fp32_params_expose_the_update(mns):
    """fp32 weights starting at zero: W' = −lr·sc·O exactly in fp32, so the
    orthogonalised update itself is compared with the oracle (including a
    tall Qwen shape through the transposed path)."""
    shapes = [(512, 3584), (18944, 3584), (130, 70)]
    inp = W.muon_inputs(shapes, 77, device="cuda", param_dtype=torch.float32)
    for p in inp.params:
        p.zero_()
    host_g = [g.cpu().numpy() for g in inp.grads]
    say("muon_step fp32 params", shapes)
    mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5)
    torch.cuda.synchronize()
    for j, (r, c) in enumerate(shapes):
        lrsc = float(np.float32(0.02)) * oracle.lr_shape_scale(r, c)
        O_gpu = -inp.params[j].double().cpu().numpy() / lrsc
        O = oracle.muon_orthogonalize(host_g[j], tuple(float(np.float32(v)) for v in oracle.QUINTIC), 5, 1e-7)
        e = rel(O_gpu, O)
        say(shapes[j], "rel err of update", e)
        assert e <= TOL_BF16


def test_muon_step_small_near_square_runs_in_fp32(mns):
    """Small, nearly square matrices take fp32 products (their smallest
    singular values make fp16 operands miss the bf16 bound): the update
    recovered from fp32 weights must meet the fp32 bound, over two steps."""
    shapes = [(32, 32), (64, 64), (128, 128), (300, 500), (700, 400)]
    inp = W.muon_inputs(shapes, 61, device="cuda", param_dtype=torch.float32)
    host_M = [m.cpu().numpy() for m in inp.momenta]
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
    for step in range(2):
        grads = inp.grads if step == 0 else W.fresh_grads(shapes, 61, step, device="cuda")
        for p in inp.params:
            p.zero_()
        mns.muon_step(inp.params, grads, inp.momenta, beta=0.95, lr=0.02, steps=5)
        torch.cuda.synchronize()
        for j, (r, c) in enumerate(shapes):
            Mn = oracle.momentum_update(host_M[j], grads[j].cpu().numpy(), np.float32(0.95))
            host_M[j] = Mn
            lrsc = float(np.float32(0.02)) * oracle.lr_shape_scale(r, c)
            O_gpu = -inp.params[j].double().cpu().numpy() / lrsc
            e = rel(O_gpu, oracle.muon_orthogonalize(Mn, c32, 5, 1e-7))
            say("step", step, shapes[j], "rel err of update", e)
            assert e <= TOL_F32


def test_single_hip_runtime_in_process(mns):
    x = W.gaussian((32, 64), 1, device="cuda")
    mns.muon_ns_batched([x])
    torch.cuda.synchronize()
    libs = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                libs.add(line.split()[-1])
    assert len(libs) == 1, libs


@pytest.mark.parametrize("dtype,seed", [(torch.bfloat16, 7), (torch.float32, 8)])
def test_seeded_random_shapes(mns, dtype, seed):
    """Forty shapes drawn from a seeded generator (each side 1–600, a third of
    them tall, some repeated so groups hold several matrices), orthogonalised
    in one call against the oracle: the planner's groups, padding and tile
    choices meet shapes nobody picked by hand."""
    import random
    rng = random.Random(seed)
    shapes = []
    while len(shapes) < 40:
        r, c = rng.randint(1, 600), rng.randint(1, 600)
        shapes.append((r, c))
        if rng.random() < 0.25:
            shapes.append((r, c))
    say(f"{dtype} seeded random shapes", shapes)
    xs = [W.gaussian(s, 700 + i, dtype=dtype) for i, s in enumerate(shapes)]
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=5)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == torch.bfloat16 else TOL_F32
    worst = 0.0
    for x, o in zip(xs, outs):
        e = rel(o.float(), oracle_ns(x.float()))
        worst = max(worst, e)
        assert e <= tol, (tuple(x.shape), e)
    say("worst", worst)


@pytest.mark.parametrize("steps", [1, 5, 12])
def test_bf16_cubic_on_the_256_tile_path(mns, steps):
    """Cubic coefficients (c = 0) on bf16 groups that run on 256-tiles: the
    A² launch has nothing to multiply (B = b·A) and runs as a scaled copy of
    A with no contraction; checked against the oracle's cubic iteration."""
    shapes = [(600, 1500), (2300, 4700), (300, 2000)]
    plan = mns.describe_plan(shapes, for_step=False, coeffs=mns.CUBIC, steps=steps)
    assert all(g["tile"] == 256 and g["op"] == "f16" for g in plan["groups"])
    xs = [W.gaussian(s, 620 + i, dtype=torch.bfloat16) for i, s in enumerate(shapes)]
    say("bf16 cubic steps", steps, shapes)
    outs = mns.muon_ns_batched([x.cuda() for x in xs], steps=steps, coeffs=mns.CUBIC)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        e = rel(o.float(), oracle_ns(x.float(), steps=steps, coeffs=oracle.CUBIC))
        say("cubic", steps, tuple(x.shape), "rel err", e)
        assert e <= TOL_BF16
