"""Caller tensors that are only 8-byte aligned, through the C ABI.

The final product's staged epilogue (16-byte row stores, weights fetched into
LDS) and the fused momentum pass's vector loads need 16-byte aligned rows;
other tensors take the element-by-element paths, which evaluate the same
expressions in the same order.  So on the fp16 256-tile path, with carried
operand exponents (the momentum pass then sums Σu² in one order on either
path), a step over tensors offset by 8 bytes must give the weights, momenta
and exponents of 16-byte aligned tensors bit for bit; and muon_ns_batched
must write the same bits into an offset output as into an aligned one.
"""
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

# wide and tall fp16 256-tile shapes, a ragged one (edge tiles on both paths)
# and two with rows whose length is not a multiple of 8 elements
SHAPES = [(512, 3584), (3584, 512), (300, 1200), (1100, 256), (256, 772), (900, 260)]


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


def offset_copy(t, off_bytes=8):
    """A contiguous copy of t whose data starts off_bytes past a 16-byte boundary."""
    k = off_bytes // t.element_size()
    buf = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    base = (-buf.data_ptr() % 16) // t.element_size()
    v = buf[base + k: base + k + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == off_bytes
    return v


def aligned_copy(t):
    return offset_copy(t, 0)


def test_offset_tensors_match_aligned_ones_bitwise(mns):
    plan = mns.describe_plan(SHAPES, for_step=True)
    assert all(b["fusable"] for b in plan["buckets"]), plan["buckets"]
    inp = W.muon_inputs(SHAPES, 7100, device="cuda")
    runs = {}
    for name, cp in (("aligned", aligned_copy), ("offset", offset_copy)):
        P = [cp(p) for p in inp.params]
        M = [cp(m) for m in inp.momenta]
        sx = mns.scale_exp_buffer(len(SHAPES), "cuda")
        for step in range(3):
            g = inp.grads if step == 0 else W.fresh_grads(SHAPES, 7100, step, device="cuda")
            G = [cp(x) for x in g]
            say(name, "step", step, "param ptr mod 16:", P[0].data_ptr() % 16)
            mns.muon_step(P, G, M, beta=0.95, lr=0.02, steps=5, scale_exp=sx)
        torch.cuda.synchronize()
        runs[name] = (P, M, sx.clone())
    (Pa, Ma, Sa), (Po, Mo, So) = runs["aligned"], runs["offset"]
    for j, s in enumerate(SHAPES):
        assert torch.equal(Pa[j], Po[j]), ("weights", s)
        assert torch.equal(Ma[j], Mo[j]), ("momentum", s)
    assert torch.equal(Sa, So)
    # the steps did change the weights (the comparison is not vacuous)
    assert not torch.equal(Pa[0], inp.params[0])


def test_offset_outputs_match_aligned_ones_bitwise(mns):
    shapes = [(256, 1024), (512, 2048), (300, 1200), (2048, 512), (128, 512)]
    xs = [W.gaussian(s, 7200 + i, dtype=torch.bfloat16, device="cuda") for i, s in enumerate(shapes)]
    outs_a = [aligned_copy(torch.zeros_like(x)) for x in xs]
    outs_o = [offset_copy(torch.zeros_like(x)) for x in xs]
    say("muon_ns_batched into aligned and offset outputs", shapes)
    mns.muon_ns_batched(xs, outs=outs_a, steps=5)
    mns.muon_ns_batched(xs, outs=outs_o, steps=5)
    torch.cuda.synchronize()
    for s, a, o in zip(shapes, outs_a, outs_o):
        assert torch.equal(a, o), s
        assert a.abs().sum() > 0
