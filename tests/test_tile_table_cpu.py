"""The planner's tile table (C ABI `muon_set_tile_table`) on the host: entries
change the plan of exactly the groups they name, invalid tables are
refused whole, and the state-carrying groups ignore the table."""
import json

import pytest

import muon_newton_schulz_06_amd as mns
from muon_newton_schulz_06_amd import autotune


@pytest.fixture(autouse=True)
def _clear():
    mns.set_tile_table([])
    yield
    mns.set_tile_table([])


def _tiles(shapes, for_step=True):
    p = mns.describe_plan(shapes, for_step=for_step)
    return {(g["m"], g["op"], g["count"]): g["tile"] for g in p["groups"]}


def test_table_overrides_only_matching_groups():
    shapes = [(512, 3584)] * 4 + [(3584, 3584)] * 2 + [(64, 64)] * 3
    base = _tiles(shapes)
    assert base[(512, "f16", 4)] == 256 and base[(3584, "f16", 2)] == 256
    mns.set_tile_table([{"m": 512, "op": "f16", "count_class": 2, "tile": 128},
                        {"m": 64, "op": "f32", "count_class": 1, "tile": 128}])
    t = _tiles(shapes)
    assert t[(512, "f16", 4)] == 128 and t[(64, "f32", 3)] == 128
    assert t[(3584, "f16", 2)] == 256          # no entry
    # another batch-size class does not match
    assert _tiles([(512, 3584)] * 8)[(512, "f16", 8)] == 256
    # workspace follows the tile (padding to the tile edge)
    p = mns.describe_plan(shapes)
    for b in p["buckets"]:
        assert b["Mp"] % p["groups"][b["group"]]["tile"] == 0


def test_invalid_tables_are_refused_and_leave_the_table_unchanged():
    mns.set_tile_table([{"m": 512, "op": "f16", "count_class": 2, "tile": 128}])
    bad = [
        [{"m": 512, "op": "f16", "count_class": 2, "tile": 64}],   # 64 is fp32 only
        [{"m": 512, "op": "f32", "count_class": 2, "tile": 256}],  # 256 is fp16 only
        [{"m": 0, "op": "f16", "count_class": 2, "tile": 128}],
        [{"m": 512, "op": "f16", "count_class": 40, "tile": 128}],
        [{"m": 512, "op": 7, "count_class": 2, "tile": 128}],
    ]
    for b in bad:
        with pytest.raises(mns.MuonError):
            mns.set_tile_table(b)
    assert _tiles([(512, 3584)] * 4)[(512, "f16", 4)] == 128


def test_state_carrying_groups_ignore_the_table():
    mns.set_tile_table([{"m": 1500, "op": "f16", "count_class": 0, "tile": 256}])
    p = mns.describe_plan([(1500, 1600)])
    g = p["groups"][0]
    assert g["state32"] and g["tile"] == 128


def test_count_class_and_table_files(tmp_path):
    assert [autotune.count_class(c) for c in (1, 2, 3, 4, 7, 8, 140)] == [0, 1, 1, 2, 2, 3, 7]
    entries = [{"m": 3584, "op": "f16", "count_class": 7, "tile": 256}]
    path = tmp_path / "t.json"
    autotune.save(entries, str(path), {"device": "x"})
    assert autotune.load_table(str(path)) == entries
    assert json.loads(path.read_text())["meta"]["device"] == "x"
    autotune.apply(str(path))
    assert _tiles([(3584, 18944)] * 140)[(3584, "f16", 140)] == 256
