"""The planner's tile table (C ABI `muon_set_tile_table`) on the host: entries
change the plan of exactly the groups they name, invalid tables are
refused whole, and the state-carrying groups ignore the table."""
import json

import pytest
import torch

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
        [{"m": 512, "op": "f16", "count_class": 2, "tile": 32}],   # 32 is fp32 only
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


def _groups(shapes, for_step=True):
    return {g["m"]: g for g in mns.describe_plan(shapes, for_step=for_step)["groups"]}


def test_entries_keyed_by_n_take_precedence_over_any_n():
    mns.set_tile_table([{"m": 512, "n": 3584, "op": "f16", "count_class": 2, "tile": 128, "band": 2},
                        {"m": 512, "n": 0, "op": "f16", "count_class": 2, "tile": 256, "xcd_window": 16}])
    g = _groups([(512, 3584)] * 4)[512]
    assert g["n_max"] == 3584 and g["tile"] == 128 and g["band"] == 2 and g["xcd_window"] == 32
    g = _groups([(512, 2048)] * 4)[512]
    assert g["n_max"] == 2048 and g["tile"] == 256 and g["xcd_window"] == 16 and g["band"] == 4
    # a group's n is its largest matrix's
    g = _groups([(512, 2048)] * 2 + [(3584, 512)] * 2)[512]
    assert g["n_max"] == 3584 and g["tile"] == 128


def test_tile_order_only_entries_keep_the_built_in_tile():
    mns.set_tile_table([{"m": 3584, "op": "f16", "count_class": 1, "xcd_window": 64, "band": 8}])
    g = _groups([(3584, 3584)] * 2)[3584]
    assert g["tile"] == 256 and g["xcd_window"] == 64 and g["band"] == 8
    # state-carrying groups keep 128-tiles but take the tile order
    mns.set_tile_table([{"m": 1500, "op": "f16", "count_class": 0, "tile": 256, "band": 1}])
    g = _groups([(1500, 1600)])[1500]
    assert g["state32"] and g["tile"] == 128 and g["band"] == 1


def test_invalid_tile_order_entries_are_refused():
    import ctypes
    mns.set_tile_table([{"m": 512, "op": "f16", "count_class": 2, "tile": 128}])
    for bad in ({"xcd_window": 12}, {"xcd_window": 128}, {"band": 3}, {"band": 16}, {"n": -1}):
        with pytest.raises(mns.MuonError):
            mns.set_tile_table([dict({"m": 512, "op": "f16", "count_class": 2}, **bad)])
    arr = (mns.MuonTileEntry * 1)()
    arr[0].m, arr[0].op, arr[0].count_class, arr[0].reserved = 512, 0, 2, 1
    assert mns.load().muon_set_tile_table(arr, 1) == 1
    assert _tiles([(512, 3584)] * 4)[(512, "f16", 4)] == 128


def test_fp32_small_groups_take_split_contraction_tiles():
    """fp32 groups with m ≤ 256 use 32-tiles (contraction split over four
    waves) whatever their matrix count — the split changes the fp32 summation
    order, so a chunk of a call must pick what the whole call picks — and pad
    to the cast's 64-element tiles; larger fp32 groups keep 64 or 128."""
    for reps in (1, 3, 64):
        shapes = [(256, 1024), (100, 130), (1024, 200), (512, 700)] * reps
        p = mns.describe_plan(shapes, for_step=False, dtype=torch.float32)
        g = {gr["m"]: gr for gr in p["groups"]}
        assert g[256]["tile"] == 32 and g[100]["tile"] == 32 and g[200]["tile"] == 32
        assert g[512]["tile"] in (64, 128)
        for b in p["buckets"]:
            t = p["groups"][b["group"]]["tile"]
            assert b["Mp"] % max(t, 64) == 0 and b["Np"] % max(t, 64) == 0
            assert 0 <= b["Mp"] - b["m"] < max(t, 64) and 0 <= b["Np"] - b["n"] < max(t, 64)
    # a table may pick 32 for an fp32 group, and 64 for a small one
    mns.set_tile_table([{"m": 512, "op": "f32", "count_class": 0, "tile": 32},
                        {"m": 256, "op": "f32", "count_class": 0, "tile": 64}])
    try:
        p = mns.describe_plan([(512, 700), (256, 1024)], for_step=False, dtype=torch.float32)
        t = {gr["m"]: gr["tile"] for gr in p["groups"]}
        assert t == {512: 32, 256: 64}
    finally:
        mns.set_tile_table([])
