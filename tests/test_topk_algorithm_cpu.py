"""CPU model of the selected step's top-k algorithm (sel_topk_kernel), checked
against sorting.

The kernel finds the k-th largest fp32 score by an MSB-first 8-bit radix
select over the bit patterns (non-negative floats order like their bits),
then takes every key above it and the lowest-indexed keys equal to it.  When
every key shares its top byte, the first histogram pass is skipped (that
byte is taken as the prefix directly).  This file restates that algorithm in
Python — per-thread index ranges of a 1024-thread workgroup, the histogram
digit rule, the tie scan in thread order — and runs it with the shortcut on
and off over random, tied, zero and common-top-byte score sets, so both
branches are checked against the definition (the k largest, ties to the
lower index) independently of the GPU.  It is a model of the kernel, not the
oracle; the oracle's selection is pinned in test_oracle_selected.py.
"""
import numpy as np
import pytest

THREADS = 1024


def model_topk(scores, k, shortcut=True):
    """Indices (ascending) the kernel's algorithm selects."""
    keys = np.asarray(scores, np.float32).view(np.uint32).astype(np.uint64)
    m = len(keys)
    per = (m + THREADS - 1) // THREADS
    prefix, mask, krem = 0, 0, k
    pass0 = 0
    kor = int(np.bitwise_or.reduce(keys)) if m else 0
    kand = int(np.bitwise_and.reduce(keys)) if m else 0xFFFFFFFF
    if shortcut and ((kor ^ kand) >> 24) == 0:
        prefix = kand & 0xFF000000
        mask = 0xFF000000
        pass0 = 1
    for p in range(pass0, 4):
        shift = 24 - 8 * p
        sel = (keys & mask) == prefix
        hist = np.bincount(((keys[sel] >> shift) & 255).astype(np.int64), minlength=256)
        above, d = 0, 255
        while d > 0:
            if above + hist[d] >= krem:
                break
            above += hist[d]
            d -= 1
        prefix |= d << shift
        krem -= above
        mask |= 255 << shift
    T = prefix
    out, eq_seen = [], 0
    for t in range(THREADS):           # thread order = index order
        for q in range(per):
            j = t * per + q
            if j >= m:
                break
            kv = int(keys[j])
            take = kv > T
            if kv == T:
                take = eq_seen < krem
                eq_seen += 1
            if take:
                out.append(j)
    return out


def by_sorting(scores, k):
    s = np.asarray(scores, np.float32)
    order = sorted(range(len(s)), key=lambda i: (-float(s[i]), i))
    return sorted(order[:k])


def common_top_byte(scores):
    keys = np.asarray(scores, np.float32).view(np.uint32)
    return len(set((keys >> 24).tolist())) == 1


@pytest.mark.parametrize("shortcut", [True, False])
def test_random_tied_and_zero_scores(shortcut):
    rng = np.random.default_rng(0)
    for trial in range(240):
        m = int(rng.integers(1, 3000))
        k = int(rng.integers(1, m + 1))
        kind = trial % 4
        if kind == 0:
            s = rng.random(m).astype(np.float32)
        elif kind == 1:
            s = rng.integers(0, 5, m).astype(np.float32)       # heavy ties
        elif kind == 2:
            s = np.zeros(m, np.float32)                         # all equal
        else:
            s = (rng.random(m) * 1e30).astype(np.float32)
            s[rng.integers(0, m, m // 3)] = 0
        assert model_topk(s, k, shortcut) == by_sorting(s, k), (trial, m, k)


@pytest.mark.parametrize("shortcut", [True, False])
def test_scores_sharing_their_top_byte(shortcut):
    """Scores inside one aligned pair of binades ([0.5, 2): biased exponents
    126 and 127 share their upper seven bits) take the shortcut branch."""
    rng = np.random.default_rng(1)
    for m in (1, 7, 512, 1000, 3584, 18944, 32768):
        s = (0.5 + 1.5 * rng.random(m)).astype(np.float32)
        assert common_top_byte(s)
        for k in sorted({1, max(1, m // 4), max(1, m // 2), m}):
            assert model_topk(s, k, shortcut) == by_sorting(s, k), (m, k)
        # ties inside the common byte
        t = np.round(s * 8) / 8
        t = np.clip(t, 0.5, 1.875).astype(np.float32)
        assert common_top_byte(t)
        for k in sorted({1, max(1, m // 3), m}):
            assert model_topk(t, k, shortcut) == by_sorting(t, k), (m, k)


def test_shortcut_and_full_pass_agree():
    rng = np.random.default_rng(2)
    for trial in range(100):
        m = int(rng.integers(1, 5000))
        k = int(rng.integers(1, m + 1))
        s = (rng.random(m) * 4.0 ** rng.integers(-3, 3)).astype(np.float32)
        assert model_topk(s, k, True) == model_topk(s, k, False)
