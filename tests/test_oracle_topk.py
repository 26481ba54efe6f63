"""Pins of the oracle's top-k selection: brute force over tiny inputs, closed forms (k >= n,
all-equal scores), the signed-zero order, invariance of the selected set under permutations of
the other positions, and the causal window count."""

import itertools

import numpy as np
import pytest

from oracle import topk as tk


def brute_force(v, k):
    """Every k-subset; the best is the one whose sorted (score desc, +0 before -0, position asc)
    sequence is lexicographically largest."""
    n = len(v)
    def rank(i):
        return (v[i], 0 if np.signbit(v[i]) else 1, -i)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = sorted((rank(i) for i in sub), reverse=True)
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(best[1])


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    n = 8
    v = rng.integers(-3, 4, n).astype(np.float32)        # many ties
    if seed % 2:
        v[rng.integers(0, n)] = -0.0
    for k in (1, 3, 5, 8, 10):
        got = tk.select_topk(v, n, k)
        want = brute_force(v, k)
        assert list(got[:len(want)]) == want, (v, k)
        assert np.all(got[len(want):] == -1)


def test_closed_forms():
    v = np.linspace(-1, 1, 50).astype(np.float32)
    assert list(tk.select_topk(v, 50, 64)) == list(range(50)) + [-1] * 14      # k >= n
    assert list(tk.select_topk(v, 50, 5)) == [45, 46, 47, 48, 49]                # increasing scores
    eq = np.full(30, 2.5, dtype=np.float32)
    assert list(tk.select_topk(eq, 30, 7)) == list(range(7))                     # ties by position
    z = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert list(tk.select_topk(z, 4, 2)) == [1, 3]                               # +0 above -0
    assert list(tk.select_topk(v, 0, 3)) == [-1, -1, -1]


def test_selected_set_invariant_under_permuting_the_rest():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(500).astype(np.float32)
    sel = set(tk.select_topk(v, 500, 40).tolist())
    w = v.copy()
    rest = np.array(sorted(set(range(500)) - sel))
    w[rest] = w[rng.permutation(rest)]
    assert set(tk.select_topk(w, 500, 40).tolist()) == sel
    thr = min(v[list(sel)])
    assert np.all(v[rest] <= thr)


def test_causal_window():
    assert tk.visible_count(100, 3, 0) == 98
    assert tk.visible_count(100, 3, 2) == 100
    assert tk.visible_count(1, 3, 0) == 0
    s = np.arange(24, dtype=np.float32).reshape(1, 2, 12)
    out = tk.topk_indices(s, [10], 2, 4)
    assert list(out[0, 0]) == [5, 6, 7, 8]      # token 0 sees positions 0..8
    assert list(out[0, 1]) == [6, 7, 8, 9]      # token 1 sees positions 0..9
