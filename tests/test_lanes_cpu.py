"""The planner's concurrent lanes on the host (muon_describe_plan's "lanes"):
every matrix of the call is in exactly one lane, lanes are formed only for
calls whose Gram-space products under-fill the GPU, and MUON_LANES fixes the
count."""
import os

import pytest

import muon_newton_schulz_06_amd as mns
import workloads as W


@pytest.fixture(autouse=True)
def _env():
    old = os.environ.pop("MUON_LANES", None)
    mns.set_tile_table([])
    yield
    os.environ.pop("MUON_LANES", None)
    if old is not None:
        os.environ["MUON_LANES"] = old


def covered_once(plan):
    seen = {}
    for lane in plan["lanes"]:
        for b, b0, b1 in lane:
            assert 0 <= b0 < b1 <= len(plan["buckets"][b]["mats"])
            for k in range(b0, b1):
                assert (b, k) not in seen, ("matrix in two lanes", b, k)
                seen[(b, k)] = True
    total = sum(len(bk["mats"]) for bk in plan["buckets"])
    return len(seen) == total


CASES = {
    "single 256x1024": ([(256, 1024)], False, 1),
    "uniform 32x(1024x4096)": ([(1024, 4096)] * 32, False, 2),
    "small mix": (None, False, 3),
    "one Qwen layer": (W.qwen_layer_shapes(), True, 2),
    "two Qwen layers": (W.qwen_model_shapes(2), True, 2),
    "four Qwen layers": (W.qwen_model_shapes(4), True, 1),
    "Qwen set": (W.qwen_model_shapes(28), True, 1),
    "uniform 8x(1024x4096)": ([(1024, 4096)] * 8, False, 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_lane_partition_and_count(name):
    shapes, for_step, lanes = CASES[name]
    if shapes is None:
        shapes = [tuple(x.shape) for x in W.ns_small_mix()]
    p = mns.describe_plan(shapes, for_step=for_step)
    assert len(p["lanes"]) == lanes
    assert covered_once(p)


@pytest.mark.parametrize("forced", [1, 2, 3, 4])
def test_lanes_env_override(forced):
    os.environ["MUON_LANES"] = str(forced)
    shapes = [(1024, 4096)] * 6 + [(300, 500), (500, 300), (64, 64)]
    p = mns.describe_plan(shapes, for_step=False)
    assert len(p["lanes"]) == forced
    assert covered_once(p)


def test_lanes_balance_work():
    """Two lanes of a uniform batch hold half the matrices each; a dominant
    group is cut across lanes."""
    p = mns.describe_plan([(1024, 4096)] * 32, for_step=False)
    sizes = sorted(sum(b1 - b0 for _, b0, b1 in lane) for lane in p["lanes"])
    assert sizes == [16, 16]
    shapes = [(512, 2048)] * 32 + [(256, 1024)] * 4
    os.environ["MUON_LANES"] = "2"
    p = mns.describe_plan(shapes, for_step=False)
    big = [b for b, bk in enumerate(p["buckets"]) if bk["m"] == 512][0]
    assert all(any(b == big for b, _, _ in lane) for lane in p["lanes"])


def test_more_lanes_than_matrices():
    os.environ["MUON_LANES"] = "4"
    p = mns.describe_plan([(300, 700), (200, 900)], for_step=False)
    assert len(p["lanes"]) == 2
    assert covered_once(p)
