"""Owner assignment from a per-shape cost table (CPU; synthetic tables)."""
import itertools
import json

import pytest

from muon_newton_schulz_06_amd import schedule as S


def _table(curves):
    t = S.CostTable()
    for shape, pts in curves.items():
        for k, v in pts.items():
            t.add(shape, k, v)
    return t


def test_cost_interpolates_and_extrapolates():
    t = _table({(4, 8): {1: 2.0, 4: 5.0}})
    assert t.cost((4, 8), 0) == 0.0
    assert t.cost((4, 8), 1) == 2.0
    assert t.cost((4, 8), 2) == pytest.approx(3.0)   # between 1 and 4
    assert t.cost((4, 8), 4) == 5.0
    assert t.cost((4, 8), 7) == pytest.approx(8.0)   # slope of the last segment
    one = _table({(2, 2): {2: 3.0}})
    assert one.cost((2, 2), 1) == pytest.approx(1.5) and one.cost((2, 2), 4) == pytest.approx(6.0)
    with pytest.raises(KeyError):
        t.cost((9, 9), 1)


def test_json_round_trip():
    t = _table({(3584, 3584): {1: 10.0, 2: 18.5}, (512, 3584): {1: 0.7}})
    t.meta["device"] = "x"
    u = S.CostTable.from_json(t.to_json())
    assert u.costs == t.costs and u.meta == t.meta
    json.loads(t.to_json())


def _brute_force(shapes, R, t):
    best = None
    for owners in itertools.product(range(R), repeat=len(shapes)):
        m = S.makespan(shapes, list(owners), R, t)
        best = m if best is None else min(best, m)
    return best


def test_greedy_is_within_the_lpt_bound_on_additive_costs():
    """With costs linear in k (no batching gain) the load model is plain
    makespan scheduling, where longest-processing-time-first is within
    4/3 − 1/(3R) of the optimum (Graham's bound); checked by brute force."""
    shapes = [(1, i) for i in (7, 5, 4, 4, 3, 3, 2, 2)]
    t = _table({s: {1: float(s[1])} for s in set(shapes)})
    for R in (2, 3):
        g = S.assign_greedy(shapes, R, t)
        opt = _brute_force(shapes, R, t)
        assert S.makespan(shapes, g, R, t) <= (4 / 3 - 1 / (3 * R)) * opt + 1e-9
        assert S.makespan(shapes, g, R, t) >= S.lower_bound(shapes, R, t) - 1e-9


def test_greedy_keeps_batching_gains_and_beats_round_robin():
    """Concave costs (a shape's second matrix is cheaper than its first):
    the greedy model keeps same-shape matrices together where that pays, and
    round robin puts all heavy matrices on one rank for a periodic order."""
    big, small = (3584, 3584), (512, 3584)
    t = _table({big: {1: 10.0, 2: 16.0, 4: 28.0}, small: {1: 1.0, 2: 1.5, 4: 2.5}})
    shapes = [big, small] * 4
    R = 2
    rr = S.assign_round_robin(shapes, R)
    g = S.assign_greedy(shapes, R, t)
    assert S.makespan(shapes, rr, R, t) == pytest.approx(28.0)   # all big ones on rank 0
    assert S.makespan(shapes, g, R, t) == pytest.approx(16.0 + 1.5)
    assert S.makespan(shapes, g, R, t) == pytest.approx(_brute_force(shapes, R, t))


def test_every_matrix_gets_exactly_one_owner_and_is_deterministic():
    shapes = S.QWEN_LAYER * 3
    t = _table({s: {1: float(s[0] * s[1]) / 1e6, 4: 3.0 * s[0] * s[1] / 1e6}
                for s in set(S.QWEN_LAYER)})
    a = S.assign_greedy(shapes, 8, t)
    b = S.assign_greedy(shapes, 8, t)
    assert a == b and len(a) == len(shapes) and all(0 <= o < 8 for o in a)
    ld = S.loads(shapes, a, 8, t)
    assert sum(1 for x in ld if x > 0) == 8
    with pytest.raises(ValueError):
        S.loads(shapes, [8] * len(shapes), 8, t)
    with pytest.raises(ValueError):
        S.assign_greedy(shapes, 0, t)
