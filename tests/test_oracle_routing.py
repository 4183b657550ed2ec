"""Pins of the oracle's router, top-k, gate weights and schedule.

Brute-force top-k (rank counting, O(E^2)) on tiny inputs with many exact ties and signed zeros;
closed forms of the weights (k = 1, k = E, sum to one) against SciPy's softmax; schedule invariants
and Python's stable sort; the fixed float32 order of the router sum on a case where order changes
the result.
"""
import numpy as np
import pytest
import scipy.special

from moe_inputs import f32_to_bf16
from oracle import moe as M
from oracle.formats import bf16_to_f64


def _brute_topk(l, k):
    T, E = l.shape
    out = np.zeros((T, k), np.int64)
    for t in range(T):
        ranks = []
        for e in range(E):
            le = l[t, e] + 0.0
            better = sum(1 for f in range(E)
                         if (l[t, f] + 0.0 > le) or (l[t, f] + 0.0 == le and f < e))
            ranks.append(better)
        ranks = np.array(ranks)
        for j in range(k):
            (sel,) = np.nonzero(ranks == j)
            assert len(sel) == 1
            out[t, j] = sel[0]
    return out


@pytest.mark.parametrize("E,k", [(1, 1), (4, 2), (8, 2), (8, 8), (13, 5), (64, 10)])
def test_topk_vs_brute_force_with_ties(rng, E, k):
    l = rng.integers(-3, 4, size=(40, E)).astype(np.float64)  # many exact ties
    l[l == 0] = rng.choice([0.0, -0.0], size=int((l == 0).sum()))
    assert np.array_equal(M.topk(l, k), _brute_topk(l, k))


def test_topk_signed_zero_and_lowest_index_tie():
    l = np.array([[-0.0, 0.0, -1.0, 0.0], [0.5, 0.5, 0.5, 0.5]])
    assert M.topk(l, 2).tolist() == [[0, 1], [0, 1]]
    assert M.topk(l, 4).tolist() == [[0, 1, 3, 2], [0, 1, 2, 3]]


def test_topk_random_vs_brute_force(rng):
    l = rng.standard_normal((30, 16)).astype(np.float32)
    assert np.array_equal(M.topk(l, 3), _brute_topk(l.astype(np.float64), 3))


def test_weights_closed_forms(rng):
    l = rng.standard_normal((50, 12)) * 3
    idx1 = M.topk(l, 1)
    assert np.all(M.topk_weights(l, idx1) == 1.0)
    idxE = M.topk(l, 12)
    wE = M.topk_weights(l, idxE)
    full = scipy.special.softmax(l, axis=1)
    assert np.allclose(wE, np.take_along_axis(full, idxE.astype(np.int64), axis=1),
                       rtol=1e-13, atol=0)
    idx4 = M.topk(l, 4)
    w4 = M.topk_weights(l, idx4)
    assert np.allclose(w4.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    p = np.take_along_axis(full, idx4.astype(np.int64), axis=1)
    assert np.allclose(w4, p / p.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.all(np.diff(w4, axis=1) <= 0)  # slots in descending-weight (rank) order


def test_router_fixed_order_is_left_to_right():
    # x = [2**24, 1, -2**24], W = [1, 1, 1]: left to right in float32 gives 2**24 + 1 -> 2**24
    # (tie to even), then 0; the exact sum is 1
    x = f32_to_bf16(np.array([[2.0 ** 24, 1.0, -2.0 ** 24]], np.float32))
    w = f32_to_bf16(np.ones((1, 3), np.float32))
    assert M.router_logits_fixed_order(x, w)[0, 0] == 0.0
    assert M.router_logits_f64(x, w)[0, 0] == 1.0
    # right to left would give (-2**24 + 1) + 2**24 = 1 (-2**24 + 1 is exact in float32), so the 0
    # above pins the left-to-right order; putting the 1 first gives 0 again, since 1 + 2**24
    # rounds to 2**24 before -2**24 is added:
    x2 = f32_to_bf16(np.array([[1.0, 2.0 ** 24, -2.0 ** 24]], np.float32))
    assert M.router_logits_fixed_order(x2, w)[0, 0] == 0.0
    x3 = f32_to_bf16(np.array([[-2.0 ** 24, 1.0, 2.0 ** 24]], np.float32))
    assert M.router_logits_fixed_order(x3, w)[0, 0] == 1.0  # (-2**24 + 1) is exact, then + 2**24


def test_router_fixed_order_vs_f64_bound(rng):
    T, h, E = 16, 512, 24
    x = f32_to_bf16(rng.standard_normal((T, h)).astype(np.float32))
    w = f32_to_bf16((rng.standard_normal((E, h)) / np.sqrt(h)).astype(np.float32))
    b = rng.standard_normal(E).astype(np.float32)
    l32 = M.router_logits_fixed_order(x, w, b).astype(np.float64)
    l64 = M.router_logits_f64(x, w, b)
    # recursive summation bound: h * u * sum |x_i w_i| (+ the bias rounding), u = 2**-24
    mag = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(w)).T + np.abs(b)[None, :]
    assert np.all(np.abs(l32 - l64) <= (h + 1) * 2.0 ** -24 * mag)
    assert not np.array_equal(l32, l64)  # float32 rounding is really there


def test_schedule_invariants_and_stable_sort(rng):
    for E, R in [(1, 7), (6, 300), (50, 128), (7, 0)]:
        a = rng.integers(0, E, size=R).astype(np.int32)
        if E == 50:
            a[:] = np.where(a < 10, 3, a)  # some empty experts, one heavy one
        counts, offsets, perm, inv = M.schedule(a, E)
        assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(np.sort(perm), np.arange(R))
        assert np.array_equal(inv[perm], np.arange(R))
        assert perm.tolist() == sorted(range(R), key=lambda q: (a[q], q))
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(a[seg] == e) and np.all(np.diff(seg) > 0)


def test_schedule_each_token_expert_pair_once(rng):
    T, E, k = 40, 16, 4
    l = rng.standard_normal((T, E))
    idx = M.topk(l, k)
    counts, offsets, perm, inv = M.schedule(idx.reshape(-1), E)
    pairs = {(int(p) // k, int(idx.reshape(-1)[p])) for p in perm}
    assert len(pairs) == T * k
    with pytest.raises(ValueError):
        M.schedule(np.array([0, 5]), 5)


def test_schedule_drops_out_of_range_ids(rng):
    """Reading: an expert id outside [0, E) gets no row and inv = -1; the kept assignments are
    scheduled exactly as if the dropped ones were not there (brute force with Python sorted)."""
    E, R = 7, 500
    a = rng.integers(-3, E + 3, size=R).astype(np.int32)
    a[:5] = [E, -1, 0x7FFFFFFF, 3, 3]
    counts, offsets, perm, inv = M.schedule(a, E, drop=True)
    valid = [q for q in range(R) if 0 <= a[q] < E]
    assert counts.sum() == len(valid) == offsets[-1] == perm.size
    assert perm.tolist() == sorted(valid, key=lambda q: (a[q], q))
    assert all(inv[q] == -1 for q in range(R) if not 0 <= a[q] < E)
    assert np.array_equal(inv[perm], np.arange(perm.size))
    with pytest.raises(ValueError):
        M.schedule(a, E)
