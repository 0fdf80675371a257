"""The torch.optim front end on the GPU: it must add nothing to the library
call (bitwise equal to muon_step on the same tensors) and follow the oracle's
definition of the step with its options over several steps."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

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


SHAPES = [(256, 512, torch.bfloat16), (512, 256, torch.bfloat16), (300, 100, torch.float32),
          (64, 64, torch.bfloat16)]


def _model(seed):
    ps = []
    for j, (r, c, dt) in enumerate(SHAPES):
        w = W.gaussian((r, c), seed + j, std=0.02, dtype=dt, device="cuda")
        ps.append(torch.nn.Parameter(w))
    return ps


def _grads(ps, seed, step):
    # bf16 parameters get bf16 gradients (what autograd produces), fp32 get fp32
    return [W.gaussian(tuple(p.shape), seed + 1000 * step + j, std=1e-2, device="cuda").to(p.dtype)
            for j, p in enumerate(ps)]


@pytest.mark.parametrize("carry", [True, False])
def test_optimizer_equals_direct_library_call(mns, carry):
    """Bitwise equal to muon_step on the same tensors, with the carried
    operand exponents (the default) against muon_step with one scale_exp
    buffer per call, and without them against the plain call."""
    ps = _model(71)
    ref_w = [p.detach().clone() for p in ps]
    ref_m = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in ps]
    opt = mns.Muon(ps, lr=0.03, momentum=0.9, nesterov=True, weight_decay=0.05,
                   carry_exponents=carry)
    groups = {dt: [j for j, p in enumerate(ps) if p.dtype == dt] for dt in (torch.bfloat16, torch.float32)}
    sx = {dt: mns.scale_exp_buffer(len(idx), "cuda") if carry else None for dt, idx in groups.items()}
    for step in range(3):
        gs = _grads(ps, 500, step)
        for p, g in zip(ps, gs):
            p.grad = g
        opt.step()
        for dt, idx in groups.items():
            mns.muon_step([ref_w[j] for j in idx], [gs[j] for j in idx], [ref_m[j] for j in idx],
                          beta=0.9, lr=0.03, nesterov=True, weight_decay=0.05, scale_exp=sx[dt])
        torch.cuda.synchronize()
        for j, p in enumerate(ps):
            assert torch.equal(p.detach(), ref_w[j]), ("weights", step, j)
            assert torch.equal(opt.state[p]["momentum_buffer"], ref_m[j]), ("momentum", step, j)
        if carry:
            for dt, idx in groups.items():
                got = [int(opt.state[ps[j]]["operand_exp"]) for j in idx]
                assert got == sx[dt].cpu().tolist(), ("exponents", step, dt)
    say("optimizer == muon_step over 3 steps, carried exponents", carry)


def test_optimizer_follows_the_oracle(mns):
    ps = _model(81)
    lr, beta, wd = 0.02, 0.95, 0.1
    opt = mns.Muon(ps, lr=lr, momentum=beta, nesterov=True, weight_decay=wd)
    host_W = [p.detach().double().cpu().numpy() for p in ps]
    host_M = [np.zeros(tuple(p.shape), np.float32) for p in ps]
    c32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
    lr32, b32 = float(np.float32(lr)), float(np.float32(beta))
    decay = 1.0 - lr32 * float(np.float32(wd))
    for step in range(2):
        gs = _grads(ps, 900, step)
        for p, g in zip(ps, gs):
            p.grad = g
        opt.step()
        torch.cuda.synchronize()
        for j, p in enumerate(ps):
            g = gs[j].double().cpu().numpy()
            _, Mn, O = oracle.muon_step(host_W[j], g, host_M[j], b32, lr32, c32, 5, 1e-7,
                                        nesterov=True, weight_decay=wd)
            got_M = opt.state[p]["momentum_buffer"].cpu().numpy()
            assert np.all(np.abs(got_M.astype(np.float64) - Mn) <= np.spacing(np.abs(Mn))), j
            r, c = p.shape
            lrsc = lr32 * oracle.lr_shape_scale(r, c)
            got = p.detach().double().cpu().numpy()
            # the update recovered from the weights: (decay·W0 − W') / (lr·sc)
            O_gpu = (decay * host_W[j] - got) / lrsc
            if p.dtype == torch.float32:
                e = np.linalg.norm(O_gpu - O) / np.linalg.norm(O)
                say("step", step, "fp32 param", tuple(p.shape), "rel err of update", e)
                assert e <= TOL_BF16
            else:
                # bf16 weights: every value must be a correct rounding of an
                # update within ±0.1·rms(O) of the oracle's
                b = 0.1 * float(np.sqrt(np.mean(O * O)))
                lo = oracle.bf16_round(decay * host_W[j] - lrsc * (O + b))
                hi = oracle.bf16_round(decay * host_W[j] - lrsc * (O - b))
                ok = bool(np.all((got >= lo) & (got <= hi)))
                say("step", step, "bf16 param", tuple(p.shape), "consistent", ok)
                assert ok
            host_W[j] = got
            host_M[j] = got_M


def test_selected_optimizer_equals_direct_library_call(mns):
    """selected_fraction runs muon_step_selected (bf16 gradients widened to
    fp32); two steps match the direct call bit for bit."""
    ps = _model(91)
    ref_w = [p.detach().clone() for p in ps]
    ref_m = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in ps]
    opt = mns.Muon(ps, lr=0.02, momentum=0.9, selected_fraction=0.3)
    for step in range(2):
        gs = _grads(ps, 700, step)
        for p, g in zip(ps, gs):
            p.grad = g
        opt.step()
        for dt in (torch.bfloat16, torch.float32):
            idx = [j for j, p in enumerate(ps) if p.dtype == dt]
            mns.muon_step_selected([ref_w[j] for j in idx], [gs[j].float() for j in idx],
                                   [ref_m[j] for j in idx], fraction=0.3, beta=0.9, lr=0.02)
        torch.cuda.synchronize()
        for j, p in enumerate(ps):
            assert torch.equal(p.detach(), ref_w[j]), ("weights", step, j)
            assert torch.equal(opt.state[p]["momentum_buffer"], ref_m[j]), ("buffer", step, j)
    say("selected optimizer == muon_step_selected over 2 steps")
