"""Pins for the selected-row Muon step of the oracle (CPU only).

The Dion3 review states the rule in words only (rows / columns of the
momentum are selected; error feedback carries what an approximation leaves
out into later steps), so these pins tie the oracle to brute force, closed
forms and exact identities rather than to printed values.
"""
import itertools
import math

import numpy as np
import pytest

import oracle

Q = oracle.QUINTIC


def _inputs(rows, cols, seed, spread=True):
    """bf16-valued weights, fp32 gradient and buffer; with `spread` the
    oriented rows get distinct scales so every selection is unambiguous."""
    rng = np.random.default_rng(seed)
    W = oracle.bf16_round(rng.standard_normal((rows, cols)) * 0.02)
    g = (rng.standard_normal((rows, cols)) * 1e-2).astype(np.float32)
    M = (rng.standard_normal((rows, cols)) * 1e-2).astype(np.float32)
    if spread:
        m = min(rows, cols)
        s = (0.5 + rng.permutation(m) / m).astype(np.float32)
        if rows > cols:
            g = (g * s[None, :]).astype(np.float32)
            M = (M * s[None, :]).astype(np.float32)
        else:
            g = (g * s[:, None]).astype(np.float32)
            M = (M * s[:, None]).astype(np.float32)
    return W, g, M


@pytest.mark.parametrize("m,k", [(1, 1), (4, 2), (6, 3), (7, 1), (7, 6), (5, 5)])
def test_selection_is_the_best_k_subset_by_brute_force(m, k):
    """Among all k-subsets, the selection has the largest total score, and
    among those the lexicographically smallest index tuple (ties to the lower
    index).  Integer scores with many ties exercise the tie rule."""
    rng = np.random.default_rng(100 * m + k)
    for trial in range(20):
        s = rng.integers(0, 4, size=m).astype(np.float64)
        best = max(itertools.combinations(range(m), k), key=lambda c: (sum(s[i] for i in c), [-i for i in c]))
        got = oracle.select_rows(s, k)
        assert tuple(got) == tuple(sorted(best)), (s, got, best)


@pytest.mark.parametrize("m,rho,k", [(10, 0.3, 3), (3584, 0.25, 896), (512, 0.25, 128), (7, 1e-9, 1),
                                     (7, 1.0, 7), (1, 0.5, 1), (0, 0.5, 0), (9, 0.5, 5)])
def test_selected_count_is_the_ceiling(m, rho, k):
    assert oracle.selected_count(m, rho) == k


@pytest.mark.parametrize("rows,cols", [(12, 40), (40, 12), (16, 16)])
def test_full_selection_is_the_plain_step(rows, cols):
    """ρ = 1 selects every row: from a zero buffer the update equals the
    plain Muon step's and the stored buffer is β times the plain one."""
    W, g, _ = _inputs(rows, cols, 5)
    Z = np.zeros_like(g)
    Wp, Mp, Op = oracle.muon_step(W, g, Z, np.float32(0.95), 0.02, Q, 5, 1e-7)
    Ws, Ms, S, OS = oracle.muon_step_selected(W, g, Z, np.float32(0.95), 0.02, Q, 5, 1e-7, 1.0)
    assert len(S) == min(rows, cols)
    Oo = Op.T if rows > cols else Op
    assert np.linalg.norm(OS - Oo) <= 1e-13 * np.linalg.norm(Oo)
    assert np.array_equal(Ws, Wp)
    assert np.array_equal(Ms, (np.float64(np.float32(0.95)) * Mp.astype(np.float64)).astype(np.float32))


def test_full_selection_follows_the_plain_recursion_over_steps():
    """With ρ = 1 the orthogonalised buffer obeys B_t = β·B_{t−1} + g_t, the
    plain momentum recursion; three steps track the plain step's weights."""
    rows, cols = 10, 30
    W, _, _ = _inputs(rows, cols, 6)
    rng = np.random.default_rng(61)
    gs = [(rng.standard_normal((rows, cols)) * 1e-2).astype(np.float32) for _ in range(3)]
    beta = np.float32(0.9)
    Wp, Mp = W.copy(), np.zeros((rows, cols), np.float32)
    Ws, Ms = W.copy(), np.zeros((rows, cols), np.float32)
    for g in gs:
        Wp, Mp, Op = oracle.muon_step(Wp, g, Mp, beta, 0.02, Q, 5, 1e-7)
        Ws, Ms, _, OS = oracle.muon_step_selected(Ws, g, Ms, beta, 0.02, Q, 5, 1e-7, 1.0)
        assert np.linalg.norm(OS - Op) <= 1e-6 * np.linalg.norm(Op)
        ref = float(beta) * Mp.astype(np.float64)
        assert np.linalg.norm(Ms - ref) <= 1e-6 * np.linalg.norm(ref)   # two fp32 roundings vs one


@pytest.mark.parametrize("rows,cols", [(9, 30), (30, 9)])
def test_one_row_closed_form(rows, cols):
    """k = 1: the block is the single highest-norm row b, whose only singular
    value after normalisation is 1, so O = φ^s(1)·b/‖b‖."""
    W, g, M = _inputs(rows, cols, 7)
    Wn, Mn, S, OS = oracle.muon_step_selected(W, g, M, np.float32(0.95), 0.02, Q, 5, 0.0, 1e-6)
    B = (M.astype(np.float64) + g).astype(np.float32).astype(np.float64)
    Bo = B.T if rows > cols else B
    norms = np.linalg.norm(Bo, axis=1)
    assert list(S) == [int(np.argmax(norms))]
    b = Bo[S[0]]
    want = oracle.scalar_map(1.0, Q, 5) * b / np.linalg.norm(b)
    assert np.linalg.norm(OS[0] - want) <= 1e-13 * np.linalg.norm(want)
    assert abs(oracle.scalar_map(1.0, Q, 5) - 0.69643641) < 1e-6


@pytest.mark.parametrize("rows,cols", [(12, 33), (33, 12)])
def test_unselected_rows_keep_weights_and_carry_the_buffer(rows, cols):
    """Weights outside the selection are unchanged bit for bit; the buffer
    keeps B there (error feedback) and β·B on the selection."""
    W, g, M = _inputs(rows, cols, 8)
    beta = np.float32(0.95)
    Wn, Mn, S, _ = oracle.muon_step_selected(W, g, M, beta, 0.02, Q, 5, 1e-7, 0.25)
    tall = rows > cols
    m = min(rows, cols)
    rest = np.setdiff1d(np.arange(m), S)
    Wo, Wno, Mno = (W.T, Wn.T, Mn.T) if tall else (W, Wn, Mn)
    B = (M.astype(np.float64) + g).astype(np.float32)
    Bo = B.T if tall else B
    assert np.array_equal(Wno[rest], Wo[rest])
    assert not np.array_equal(Wno[S], Wo[S])
    assert np.array_equal(Mno[rest], Bo[rest])
    assert np.array_equal(Mno[S], (float(beta) * Bo[S].astype(np.float64)).astype(np.float32))


def test_error_feedback_accumulates_an_unselected_row_without_decay():
    """A row that never wins the selection accumulates Σ g_t exactly (fp32
    additions in order), while selected rows decay by β."""
    rows, cols = 6, 20
    rng = np.random.default_rng(9)
    W = oracle.bf16_round(rng.standard_normal((rows, cols)) * 0.02)
    M = np.zeros((rows, cols), np.float32)
    acc = np.zeros(cols, np.float32)
    for t in range(4):
        g = (rng.standard_normal((rows, cols)) * 1e-2).astype(np.float32)
        g[0] *= np.float32(1e-3)        # row 0 is always the smallest
        W, M, S, _ = oracle.muon_step_selected(W, g, M, np.float32(0.9), 0.02, Q, 5, 1e-7, 0.5)
        assert 0 not in S
        acc = (acc + g[0]).astype(np.float32)
        assert np.array_equal(M[0], acc)


def test_selection_is_permutation_equivariant():
    """Permuting the rows of (W, g, M) permutes the selected rows and the
    result the same way (row-selected NS is row-permutation equivariant)."""
    rows, cols = 16, 48
    W, g, M = _inputs(rows, cols, 10)
    perm = np.random.default_rng(11).permutation(rows)
    Wa, Ma, Sa, _ = oracle.muon_step_selected(W, g, M, np.float32(0.95), 0.02, Q, 5, 1e-7, 0.375)
    Wb, Mb, Sb, _ = oracle.muon_step_selected(W[perm], g[perm], M[perm], np.float32(0.95), 0.02, Q, 5,
                                              1e-7, 0.375)
    assert sorted(perm[Sb].tolist()) == Sa.tolist()
    assert np.array_equal(Mb, Ma[perm])
    assert np.max(np.abs(Wb - Wa[perm])) <= 2.0 ** -14   # within one bf16 rounding step of 0.02-scale values


def test_tall_matrix_selects_columns_like_its_transpose_selects_rows():
    """A tall matrix is handled as its transpose: the same indices are
    selected (as columns), the buffer is the transpose and the block's
    orthogonalisation is identical."""
    W, g, M = _inputs(14, 40, 12)
    a = oracle.muon_step_selected(W, g, M, np.float32(0.95), 0.02, Q, 5, 1e-7, 0.5)
    b = oracle.muon_step_selected(W.T, g.T, M.T, np.float32(0.95), 0.02, Q, 5, 1e-7, 0.5)
    assert a[2].tolist() == b[2].tolist()
    assert np.array_equal(a[1], b[1].T)
    assert np.linalg.norm(a[3] - b[3]) <= 1e-13 * np.linalg.norm(a[3])


def test_scale_invariance_of_the_update():
    """Scaling gradient and buffer by a power of two (exact in fp32) leaves
    the selection and the orthogonalised block unchanged."""
    W, g, M = _inputs(10, 25, 13)
    a = oracle.muon_step_selected(W, g, M, np.float32(0.95), 0.02, Q, 5, 0.0, 0.5)
    b = oracle.muon_step_selected(W, g * np.float32(8), M * np.float32(8), np.float32(0.95), 0.02, Q, 5,
                                  0.0, 0.5)
    assert a[2].tolist() == b[2].tolist()
    assert np.linalg.norm(a[3] - b[3]) <= 1e-13 * np.linalg.norm(a[3])
    assert np.array_equal(a[0], b[0])
    assert math.isclose(float(np.linalg.norm(b[1])), 8 * float(np.linalg.norm(a[1])), rel_tol=1e-6)
