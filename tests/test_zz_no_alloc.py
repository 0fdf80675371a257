"""muon_ns_batched_noalloc (the entry point that allocates nothing) against
muon_ns_batched with a caller workspace, through the C ABI.

Two calls in a row, the second with a smaller input, so the second runs on a
scratch array that still holds the first call's contents: each output must
equal muon_ns_batched's bit for bit (same kernels, same plan), and a sampled
matrix of each call must also meet the 2e-2 bound against the oracle.  No
call may allocate device memory through PyTorch's allocator, and a request
larger than the scratch must be rejected with a workspace error.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

Q32 = tuple(float(np.float32(v)) for v in oracle.QUINTIC)


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


def _rel(got, ref):
    got = got.double().cpu().numpy()
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def _run_pair(mns, xs, seed_note):
    outs_ref = mns.muon_ns_batched(xs, steps=5)
    outs = [torch.empty_like(x) for x in xs]
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    mns.muon_ns_batched_noalloc(xs, outs, steps=5)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert after == before, "the no-allocation call allocated through torch"
    for i, (a, b) in enumerate(zip(outs, outs_ref)):
        assert torch.equal(a, b), (seed_note, i, tuple(a.shape))
    x0 = xs[0].float().cpu().double().numpy()
    e = _rel(outs[0].float(), oracle.muon_orthogonalize(x0, Q32, 5, 1e-7))
    say(seed_note, "sampled rel err vs oracle", e)
    tol = 1e-4 if xs[0].dtype == torch.float32 else 2e-2
    assert e <= tol


def test_noalloc_two_calls_second_smaller(mns):
    first = [W.gaussian(s, 9100 + i, dtype=torch.bfloat16, device="cuda")
             for i, s in enumerate([(1024, 4096), (700, 300), (512, 2048), (2304, 600)])]
    need = mns.ns_workspace_size([tuple(x.shape) for x in first])
    say("first call", [tuple(x.shape) for x in first], "workspace", need)
    assert need <= mns.NOALLOC_SCRATCH_BYTES
    _run_pair(mns, first, "first")
    second = [W.gaussian(s, 9200 + i, dtype=torch.bfloat16, device="cuda")
              for i, s in enumerate([(96, 200), (300, 64)])]
    say("second call", [tuple(x.shape) for x in second])
    _run_pair(mns, second, "second")


def test_noalloc_fp32_and_rejects_oversized(mns):
    x = [W.gaussian((256, 1024), 1001, device="cuda")]
    say("fp32 256x1024")
    _run_pair(mns, x, "fp32")
    big = [torch.zeros((2048, 8192), dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(mns.MuonError) as ei:
        mns.muon_ns_batched_noalloc(big, [torch.empty_like(big[0])], steps=5)
    assert ei.value.status_name == "WORKSPACE"
