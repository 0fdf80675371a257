"""Parity of the selected-row Muon step (muon_step_selected, through the C
ABI) with the fp64 oracle.

Inputs come from ``workloads.selected_inputs``: rows along the short side
carry distinct scales, and every case first checks that the oracle's k-th
and (k+1)-th scores differ by far more than fp32 summation error, so the
selected set is unique in any precision and must match exactly.

Bars: the buffer is bit-exact (fp32 add, fp32 product by β); weights outside
the selection are unchanged bit for bit; selected bf16 weights lie in the
rounding band of the oracle's update (as for muon_step); with fp32 weights
starting at zero the update itself is exposed and meets the 2e-2 relative
Frobenius bound of the half-precision pipeline.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from checks import weights_consistent

pytestmark = pytest.mark.gpu

Q32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)
BETA = np.float32(0.95)
LR = float(np.float32(0.02))
EPS = float(np.float32(1e-7))


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


def unique_margin(B, k):
    """Relative gap between the k-th and (k+1)-th largest fp64 row scores of
    the oriented buffer (inf when every row is selected)."""
    Bo = B.T if B.shape[0] > B.shape[1] else B
    s = np.sort(np.sum(Bo.astype(np.float64) ** 2, axis=1))[::-1]
    if k >= len(s):
        return np.inf
    return (s[k - 1] - s[k]) / s[k - 1]


def band_ok(W0, got, O, lrsc, band=0.1):
    """Selected weights inside the rounding band of the oracle's update, and
    no more of them off the oracle's rounding than an update error at the
    2e-2 bound would move."""
    ok, frac, expect = weights_consistent(W0, got, O, lrsc, band=band)
    return ok and frac <= expect


def to_gpu(inp):
    """Inputs are drawn on the CPU (so the same values can be checked there)
    and copied to the device."""
    inp.params = [t.cuda() for t in inp.params]
    inp.grads = [t.cuda() for t in inp.grads]
    inp.momenta = [t.cuda() for t in inp.momenta]
    return inp


def step_grads(shapes, seed, t):
    """Gradients of training step t ≥ 1: fresh draws with fresh row scales."""
    g = W.fresh_grads(shapes, seed, 17 * t)
    for j, (r, c) in enumerate(shapes):
        if r and c:
            g[j].mul_(W.row_scales(r, c, seed + j + 7_000_001 + t))
    return g


def run_and_check(mns, shapes, fraction, seed, steps_of_training=2, m_std=1e-2, ns_steps=5):
    inp = to_gpu(W.selected_inputs(shapes, seed, m_std=m_std))
    Wc = [p.float().double().cpu().numpy() for p in inp.params]
    Mc = [m.cpu().numpy().copy() for m in inp.momenta]
    for t in range(steps_of_training):
        if t > 0:
            inp.grads = [g.cuda() for g in step_grads(shapes, seed, t)]
        gc = [g.cpu().numpy() for g in inp.grads]
        say(f"selected step t={t} shapes={shapes} fraction={fraction} seed={seed}")
        mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=fraction, beta=float(BETA),
                               lr=LR, steps=ns_steps)
        torch.cuda.synchronize()
        for j, (r, c) in enumerate(shapes):
            if r == 0 or c == 0:
                continue
            B = (Mc[j].astype(np.float64) + gc[j]).astype(np.float32)
            k = oracle.selected_count(min(r, c), fraction)
            assert unique_margin(B, k) > 1e-4, "inputs do not fix the selection"
            Wn, Mn, S, OS = oracle.muon_step_selected(Wc[j], gc[j], Mc[j], BETA, LR, Q32, ns_steps, EPS,
                                                      fraction)
            got_M = inp.momenta[j].cpu().numpy()
            got_W = inp.params[j].float().double().cpu().numpy()
            assert np.array_equal(got_M, Mn), f"buffer differs ({r}x{c})"
            tall = r > c
            Wo, Go, Wno = (Wc[j].T, got_W.T, Wn.T) if tall else (Wc[j], got_W, Wn)
            rest = np.setdiff1d(np.arange(min(r, c)), S)
            assert np.array_equal(Go[rest], Wo[rest]), f"unselected weights changed ({r}x{c})"
            lrsc = LR * oracle.lr_shape_scale(r, c)
            assert band_ok(Wo[S], Go[S], OS, lrsc), f"selected weights outside the band ({r}x{c})"
            frac = float(np.mean(Go[S] != Wno[S]))
            say(f"  {r}x{c}: k={len(S)} ok, fraction differing from the oracle's rounding {frac:.4f}")
            Wc[j], Mc[j] = got_W, got_M


@pytest.mark.parametrize("fraction", [0.25, 0.5, 1.0])
def test_small_shapes_two_steps(mns, fraction):
    shapes = [(96, 200), (200, 96), (128, 128), (37, 501), (501, 37), (300, 1030), (1, 50), (50, 1)]
    run_and_check(mns, shapes, fraction, 61)


@pytest.mark.parametrize("ns_steps", [0, 1, 2])
def test_other_step_counts(mns, ns_steps):
    """steps = 0 applies the normalised selected block itself; 1 and 2 steps
    exercise the short recursions (the first-step Q and the A chain)."""
    run_and_check(mns, [(96, 200), (200, 96), (300, 1030)], 0.25, 131, steps_of_training=1,
                  ns_steps=ns_steps)


def test_seeded_random_shapes(mns):
    """Twenty-four seeded random shapes (each side 2–400) at ρ = 0.3 over two
    training steps."""
    import random
    rng = random.Random(23)
    shapes = [(rng.randint(2, 400), rng.randint(2, 400)) for _ in range(24)]
    run_and_check(mns, shapes, 0.3, 151)


def test_single_row_and_empty_matrices(mns):
    # fraction so small that k = 1 everywhere; an empty matrix in the list
    run_and_check(mns, [(64, 256), (0, 7), (256, 64), (5, 0)], 1e-6, 71, steps_of_training=1)


def test_update_through_fp32_weights(mns):
    """fp32 weights at zero: W' = −lrsc·O_S exactly up to one fp32 rounding,
    so the orthogonalised block itself meets the 2e-2 relative bound."""
    shapes = [(512, 3584), (3584, 512), (700, 700)]
    inp = to_gpu(W.selected_inputs(shapes, 81, param_dtype=torch.float32))
    for p in inp.params:
        p.zero_()
    gc = [g.cpu().numpy() for g in inp.grads]
    say(f"fp32 weights shapes={shapes}")
    mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=0.25, beta=float(BETA), lr=LR,
                           steps=5)
    torch.cuda.synchronize()
    for j, (r, c) in enumerate(shapes):
        Z = np.zeros((r, c))
        _, Mn, S, OS = oracle.muon_step_selected(Z, gc[j], np.zeros((r, c), np.float32), BETA, LR, Q32, 5,
                                                 EPS, 0.25)
        lrsc = LR * oracle.lr_shape_scale(r, c)
        got = inp.params[j].double().cpu().numpy()
        Go = got.T if r > c else got
        O_gpu = -Go[S] / lrsc
        err = np.linalg.norm(O_gpu - OS) / np.linalg.norm(OS)
        say(f"  {r}x{c}: k={len(S)} rel err {err:.3e}")
        assert err <= 2e-2
        rest = np.setdiff1d(np.arange(min(r, c)), S)
        assert not np.any(Go[rest])
        assert np.array_equal(inp.momenta[j].cpu().numpy(), Mn)


def test_equal_scores_take_the_lower_index(mns):
    """Duplicated rows (columns) have bit-identical scores; the lower index
    wins, as in the oracle."""
    shapes = [(16, 64), (64, 16)]
    inp = to_gpu(W.selected_inputs(shapes, 91))
    g0 = inp.grads[0]
    g0[9] = g0[3]
    g0[12] = g0[3]
    g1 = inp.grads[1]
    g1[:, 10] = g1[:, 2]
    gc = [g.cpu().numpy() for g in inp.grads]
    Wc = [p.float().double().cpu().numpy() for p in inp.params]
    say("ties")
    # k chosen so that the threshold falls inside the tied group for each matrix
    for j, (r, c) in enumerate(shapes):
        Bo = gc[j].T if r > c else gc[j]
        sc = np.sum(Bo.astype(np.float64) ** 2, axis=1)
        tied = 3 if j == 0 else 2
        rank = int(np.sum(sc > sc[tied]))
        fraction = (rank + 0.5) / min(r, c)     # k = rank + 1: the threshold is the tied score
        inp1 = [t[j:j + 1] for t in (inp.params, inp.grads, inp.momenta)]
        mns.muon_step_selected(*inp1, fraction=fraction, beta=float(BETA), lr=LR, steps=5)
        torch.cuda.synchronize()
        _, Mn, S, _ = oracle.muon_step_selected(Wc[j], gc[j], np.zeros((r, c), np.float32), BETA, LR, Q32,
                                                5, EPS, fraction)
        assert tied in S.tolist() and (9 if j == 0 else 10) not in S.tolist()
        assert np.array_equal(inp.momenta[j].cpu().numpy(), Mn)


def test_qwen_layer_shapes_sampled(mns):
    """One step at ρ = 0.25 over one Qwen2.5-7B-shaped layer; q, k, gate and
    down are checked against the oracle (v, o, up share their shapes)."""
    shapes = W.qwen_layer_shapes()
    inp = to_gpu(W.selected_inputs(shapes, 4001))
    check = {0: "q", 1: "k", 4: "gate", 6: "down"}
    Wc = {j: inp.params[j].float().double().cpu().numpy() for j in check}
    gc = {j: inp.grads[j].cpu().numpy() for j in check}
    say("qwen layer, fraction 0.25")
    mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=0.25, beta=float(BETA), lr=LR,
                           steps=5)
    torch.cuda.synchronize()
    for j, name in check.items():
        r, c = shapes[j]
        k = oracle.selected_count(min(r, c), 0.25)
        assert unique_margin(gc[j], k) > 1e-5
        Wn, Mn, S, OS = oracle.muon_step_selected(Wc[j], gc[j], np.zeros((r, c), np.float32), BETA, LR,
                                                  Q32, 5, EPS, 0.25)
        assert np.array_equal(inp.momenta[j].cpu().numpy(), Mn)
        got = inp.params[j].float().double().cpu().numpy()
        Go, Wo = (got.T, Wc[j].T) if r > c else (got, Wc[j])
        rest = np.setdiff1d(np.arange(min(r, c)), S)
        assert np.array_equal(Go[rest], Wo[rest])
        assert band_ok(Wo[S], Go[S], OS, LR * oracle.lr_shape_scale(r, c))
        say(f"  {name} {r}x{c}: k={k} ok")


def test_full_set_sampled(mns):
    """The benchmark's configuration: one selected step (ρ = 0.25) over all
    196 Qwen2.5-7B-shaped matrices in one call (the same chunked launches and
    Gram groups the benchmark times); seven matrices from the first and the
    last layer are checked against the oracle."""
    shapes = W.qwen_model_shapes(28)
    inp = W.selected_inputs(shapes, 5001, device="cuda")
    sample = {0: "L0 q", 1: "L0 k", 4: "L0 gate", 6: "L0 down", 27 * 7 + 2: "L27 v", 27 * 7 + 3: "L27 o",
              27 * 7 + 5: "L27 up"}
    Wc = {j: inp.params[j].float().double().cpu().numpy() for j in sample}
    gc = {j: inp.grads[j].cpu().numpy() for j in sample}
    say("full set, 196 matrices, fraction 0.25")
    mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=0.25, beta=float(BETA), lr=LR,
                           steps=5)
    torch.cuda.synchronize()
    for j, name in sample.items():
        r, c = shapes[j]
        k = oracle.selected_count(min(r, c), 0.25)
        assert unique_margin(gc[j], k) > 1e-5, f"{name}: inputs do not fix the selection"
        Wn, Mn, S, OS = oracle.muon_step_selected(Wc[j], gc[j], np.zeros((r, c), np.float32), BETA, LR,
                                                  Q32, 5, EPS, 0.25)
        assert np.array_equal(inp.momenta[j].cpu().numpy(), Mn), name
        got = inp.params[j].float().double().cpu().numpy()
        Go, Wo = (got.T, Wc[j].T) if r > c else (got, Wc[j])
        rest = np.setdiff1d(np.arange(min(r, c)), S)
        assert np.array_equal(Go[rest], Wo[rest]), name
        assert band_ok(Wo[S], Go[S], OS, LR * oracle.lr_shape_scale(r, c)), name
        say(f"  {name} {r}x{c}: k={k} ok")


def _scores_in_one_byte(shape, seed):
    """A gradient whose squared row norms along the short side are exactly
    0.6 + 1.2·π(i)/m (π a seeded permutation): every score lies in [0.5, 2),
    so all fp32 keys share their top byte and the top-k takes its shortcut
    branch, while neighbouring scores stay 1.2/m apart."""
    r, c = shape
    g = W.gaussian(shape, seed).double()
    m = min(r, c)
    perm = torch.randperm(m, generator=torch.Generator().manual_seed(seed + 1)).double()
    target = 0.6 + 1.2 * perm / m
    if r > c:
        g = g / g.norm(dim=0, keepdim=True) * target.sqrt()[None, :]
    else:
        g = g / g.norm(dim=1, keepdim=True) * target.sqrt()[:, None]
    return g.float()


def test_scores_sharing_the_top_byte(mns):
    """Scores confined to [0.5, 2) (the benchmark's unscaled gradients also
    fall in one such byte): the top-k's shortcut branch, checked like every
    other selected step — buffer bit-exact, unselected weights unchanged,
    selected weights within the update band."""
    shapes = [(512, 3584), (3584, 512), (2048, 4096), (40, 700)]
    inp = W.selected_inputs(shapes, 171)
    inp.grads = [_scores_in_one_byte(s, 180 + j) for j, s in enumerate(shapes)]
    inp.momenta = [torch.zeros(s, dtype=torch.float32) for s in shapes]
    Wc = [p.float().double().numpy() for p in inp.params]
    gc = [g.numpy() for g in inp.grads]
    for j, (r, c) in enumerate(shapes):
        Bo = gc[j].T if r > c else gc[j]
        sc = np.sum(Bo.astype(np.float32) ** 2, axis=1, dtype=np.float32)
        assert np.all((sc >= 0.5) & (sc < 2.0)), "scores must share the top byte"
        assert unique_margin(gc[j], oracle.selected_count(min(r, c), 0.25)) > 1e-4
    inp = to_gpu(inp)
    say("scores sharing their top byte", shapes)
    mns.muon_step_selected(inp.params, inp.grads, inp.momenta, fraction=0.25, beta=float(BETA), lr=LR,
                           steps=5)
    torch.cuda.synchronize()
    for j, (r, c) in enumerate(shapes):
        Wn, Mn, S, OS = oracle.muon_step_selected(Wc[j], gc[j], np.zeros((r, c), np.float32), BETA, LR,
                                                  Q32, 5, EPS, 0.25)
        assert np.array_equal(inp.momenta[j].cpu().numpy(), Mn), (r, c)
        got = inp.params[j].float().double().cpu().numpy()
        Go, Wo = (got.T, Wc[j].T) if r > c else (got, Wc[j])
        rest = np.setdiff1d(np.arange(min(r, c)), S)
        assert np.array_equal(Go[rest], Wo[rest]), (r, c)
        assert band_ok(Wo[S], Go[S], OS, LR * oracle.lr_shape_scale(r, c)), (r, c)
        say(f"  {r}x{c}: k={len(S)} ok")
