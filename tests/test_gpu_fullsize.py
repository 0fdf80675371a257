"""Parity at full size: the Qwen2.5-7B-shaped matrix set in the launch
configuration the benchmark times (one muon_step over all 196 matrices,
sampled outputs checked against the oracle one by one), and the largest Gram
size the library accepts (m = 32768), checked through a block-diagonal input
whose blocks the oracle can compute independently."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from checks import weights_consistent

pytestmark = pytest.mark.gpu

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


def test_qwen_full_set_sampled(mns):
    """One step over the benchmark's 196 matrices (same shapes, seeds and
    dtypes); one matrix of every shape, spread over the layers, is checked:
    momentum exactly (M = 0 before the step, so M' = g), every updated bf16
    weight within the rounding band of an update within ±0.1·rms(O) of the
    oracle's, and the fraction of weights off the oracle's rounding below
    what an update error at the 2e-2 bound would produce."""
    shapes = W.qwen_model_shapes(28)
    say("generating the 196-matrix set")
    inp = W.muon_inputs(shapes, 5001, device="cuda")
    sample = [(0, 0), (13, 1), (27, 2), (5, 3), (20, 4), (27, 5), (9, 6)]  # (layer, shape index)
    idx = [7 * layer + j for layer, j in sample]
    host_W = {i: inp.params[i].float().cpu().double().numpy() for i in idx}
    host_g = {i: inp.grads[i].cpu().numpy() for i in idx}
    say("muon_step over 196 matrices")
    mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5)
    torch.cuda.synchronize()
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
    lr32 = float(np.float32(0.02))
    got_W = {i: inp.params[i].float().cpu().double().numpy() for i in idx}
    got_M = {i: inp.momenta[i].cpu().numpy() for i in idx}
    del inp
    torch.cuda.empty_cache()
    for i in idx:
        r, c = shapes[i]
        assert np.array_equal(got_M[i], host_g[i]), ("momentum", i)
        O = oracle.muon_orthogonalize(host_g[i].astype(np.float64), c32, 5, 1e-7)
        lrsc = lr32 * oracle.lr_shape_scale(r, c)
        ok, frac, expect = weights_consistent(host_W[i], got_W[i], O, lrsc)
        say("matrix", i, shapes[i], "weights consistent", ok, "fraction != oracle rounding", frac,
            "bound", expect)
        assert ok
        assert frac <= expect


def test_qwen_full_set_carried_exponents_sampled(mns):
    """The benchmark's timed configuration: steps over the 196 matrices with
    operand exponents carried from step to step (the first step records them,
    the second has the momentum pass write the fp16 operands).  After the
    second step (fresh gradients) one matrix of every shape is checked: the
    momentum to fp32 rounding of the oracle's, every exponent of a fusable
    matrix known, and every updated bf16 weight as in the one-step test."""
    shapes = W.qwen_model_shapes(28)
    say("generating the 196-matrix set")
    inp = W.muon_inputs(shapes, 5001, device="cuda")
    sx = mns.scale_exp_buffer(len(shapes), "cuda")
    sample = [(3, 0), (17, 1), (26, 2), (8, 3), (22, 4), (1, 5), (14, 6)]  # (layer, shape index)
    idx = [7 * layer + j for layer, j in sample]
    say("first muon_step over 196 matrices (records the exponents)")
    mns.muon_step(inp.params, inp.grads, inp.momenta, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
    torch.cuda.synchronize()
    assert all(-100 <= e <= 100 for e in sx.cpu().tolist()), "an exponent was not recorded"
    g2 = W.fresh_grads(shapes, 5001, 1, device="cuda")
    host_W = {i: inp.params[i].float().cpu().double().numpy() for i in idx}
    host_M = {i: inp.momenta[i].cpu().numpy() for i in idx}
    host_g = {i: g2[i].cpu().numpy() for i in idx}
    say("second muon_step over 196 matrices (fused operands)")
    mns.muon_step(inp.params, g2, inp.momenta, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
    torch.cuda.synchronize()
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
    lr32 = float(np.float32(0.02))
    got_W = {i: inp.params[i].float().cpu().double().numpy() for i in idx}
    got_M = {i: inp.momenta[i].cpu().numpy() for i in idx}
    del inp, g2
    torch.cuda.empty_cache()
    for i in idx:
        r, c = shapes[i]
        Mn = oracle.momentum_update(host_M[i], host_g[i], np.float32(0.95))
        ulp = np.spacing(np.abs(Mn).astype(np.float32))
        assert np.all(np.abs(got_M[i].astype(np.float64) - Mn) <= ulp), ("momentum", i)
        O = oracle.muon_orthogonalize(got_M[i].astype(np.float64), c32, 5, 1e-7)
        lrsc = lr32 * oracle.lr_shape_scale(r, c)
        ok, frac, expect = weights_consistent(host_W[i], got_W[i], O, lrsc)
        say("matrix", i, shapes[i], "weights consistent", ok, "fraction != oracle rounding", frac,
            "bound", expect)
        assert ok
        assert frac <= expect


def test_maximum_gram_size_block_diagonal(mns):
    """m = 32768 (the largest Gram size accepted), n = 131072, bf16: 128
    diagonal blocks of 256×1024 N(0,1) values, zeros elsewhere.  Frobenius
    normalisation is global, and NS maps a block-diagonal matrix block by
    block, so output block i is the plain NS iteration of B_i / (‖X‖_F + ε);
    the oracle computes three sampled blocks that way.  Off-diagonal regions
    must come out exactly zero (every product there sums exact zeros)."""
    nb, br, bc = 128, 256, 1024
    m, n = nb * br, nb * bc
    say("building", m, "x", n, "bf16 block-diagonal input")
    blocks = [W.gaussian((br, bc), 7000 + i, dtype=torch.bfloat16) for i in range(nb)]
    x = torch.zeros((m, n), dtype=torch.bfloat16, device="cuda")
    for i, blk in enumerate(blocks):
        x[i * br:(i + 1) * br, i * bc:(i + 1) * bc] = blk.cuda()
    fro = float(np.sqrt(sum(float((b.double() ** 2).sum()) for b in blocks)))
    say("muon_ns_batched at m = 32768")
    out = mns.muon_ns_batched([x], steps=5)[0]
    torch.cuda.synchronize()
    del x
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
    for i in (0, 57, nb - 1):
        ref = oracle.newton_schulz(blocks[i].double().numpy() / (fro + float(np.float32(1e-7))), c32, 5)
        got = out[i * br:(i + 1) * br, i * bc:(i + 1) * bc].double().cpu().numpy()
        e = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        say("block", i, "rel err", e)
        assert e <= TOL_BF16
    for (r0, c0) in ((0, bc), (m - br, 0), (br * 60, bc * 3), (br * 3, bc * 60)):
        z = out[r0:r0 + br, c0:c0 + bc]
        assert int(torch.count_nonzero(z)) == 0, ("off-diagonal", r0, c0)
    del out
    torch.cuda.empty_cache()
