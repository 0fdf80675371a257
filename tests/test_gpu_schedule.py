"""The cost-table profiler and the one-GPU check of an assignment run on the
GPU (small shapes; the full Qwen2.5-7B table is measured by the module's CLI)."""
import pytest
import torch

from muon_newton_schulz_06_amd import schedule as S

pytestmark = pytest.mark.gpu


def test_profile_and_validate_small_shapes():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    shapes = [(256, 1024), (512, 512), (256, 1024), (512, 512), (256, 1024)]
    t = S.profile_shapes(shapes, batch_sizes=(1, 2), reps=1)
    for s in set(shapes):
        assert 0 < t.cost(s, 1) and 0 < t.cost(s, 2)
    owners = S.assign_greedy(shapes, 2, t)
    meas = S.validate_on_one_gpu(shapes, owners, 2, reps=1)
    assert len(meas) == 2 and all(m > 0 for m in meas)


def test_autotune_small_workload_installs_a_table():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import muon_newton_schulz_06_amd as mns
    from muon_newton_schulz_06_amd import autotune
    shapes = [(512, 2048)] * 4 + [(100, 100)] * 2
    try:
        entries = autotune.tune(shapes, reps=1)
        keys = {(e["m"], e["op"]) for e in entries}
        assert keys == {(512, "f16"), (100, "f32")}
        p = mns.describe_plan(shapes)
        for e in entries:
            g = next(g for g in p["groups"] if g["m"] == e["m"] and g["op"] == e["op"])
            assert g["tile"] == e["tile"]
    finally:
        mns.set_tile_table([])
