"""Ten consecutive muon_step calls through the C ABI against the fp64 oracle
evolving its own state from the same gradients: errors must not accumulate.

fp32 weights (so the update −lr·sc·O itself is applied without a bf16
rounding), fresh seeded gradients every step, β = 0.95, lr = 0.02, five
quintic steps; a wide, a tall, a square fp32-path and a small group
(several planner branches in one call, with concurrent lanes).  After every
step the momentum must agree to fp32 rounding (it is the same sum, formed
with one fused multiply-add on the GPU and rounded once from fp64 by the
oracle) and the weights' accumulated change must agree with the oracle's
within the 2e-2 relative tolerance of the orthogonalised update.  The run
is repeated with operand exponents carried from step to step (scale_exp):
the momentum's norm grows over the first steps, so each step's exponent
comes from a different norm than its own.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(300, 1200), (1100, 256), (384, 384), (96, 200), (600, 1500)]
STEPS = 10
Q32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
BETA, LR, EPS = np.float32(0.95), 0.02, 1e-7


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("carried", [False, True])
def test_ten_steps_follow_the_oracle(carried):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import muon_newton_schulz_06_amd as mns
    mns.load()
    inp = W.muon_inputs(SHAPES, 7300, device="cpu", param_dtype=torch.float32)
    W0 = [p.double().numpy() for p in inp.params]
    Wg = [p.cuda() for p in inp.params]
    Mg = [m.cuda() for m in inp.momenta]
    Wo = [w.copy() for w in W0]
    Mo = [m.numpy().copy() for m in inp.momenta]
    lr32 = float(np.float32(LR))
    sx = mns.scale_exp_buffer(len(SHAPES), "cuda") if carried else None
    for step in range(STEPS):
        grads = inp.grads if step == 0 else W.fresh_grads(SHAPES, 7300, step)
        mns.muon_step(Wg, [g.cuda() for g in grads], Mg, beta=float(BETA), lr=LR, steps=5, scale_exp=sx)
        torch.cuda.synchronize()
        worst_m, worst_w = 0.0, 0.0
        for j, (r, c) in enumerate(SHAPES):
            Mo[j] = oracle.momentum_update(Mo[j], grads[j].numpy(), BETA)
            O = oracle.muon_orthogonalize(Mo[j], Q32, 5, EPS)
            Wo[j] = Wo[j] - lr32 * oracle.lr_shape_scale(r, c) * O
            em = rel(Mg[j].double().cpu().numpy(), Mo[j].astype(np.float64))
            ew = rel(Wg[j].double().cpu().numpy() - W0[j], Wo[j] - W0[j])
            worst_m, worst_w = max(worst_m, em), max(worst_w, ew)
            assert em <= 1e-5, ("momentum", step, (r, c), em)
            assert ew <= 2e-2, ("weights", step, (r, c), ew)
        print(f"[case] carried {carried} step {step}: momentum rel err {worst_m:.2e}, "
              f"accumulated update rel err {worst_w:.2e}", flush=True)
        sys.stdout.flush()
