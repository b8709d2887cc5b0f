"""Pins for the oracle's top-k routing and permutation (CPU only)."""
import numpy as np
import pytest
import scipy.special

from oracle.routing import permute, topk_route


def _tie_logits(rng, T, E):
    # values on a 0.5 grid -> many exact ties
    return (rng.integers(-4, 5, (T, E)) * 0.5).astype(np.float32)


def test_ids_bruteforce_sorted_with_ties():
    rng = np.random.default_rng(0)
    for T, E, k in ((40, 6, 3), (30, 8, 8), (25, 5, 1), (20, 17, 4)):
        lg = _tie_logits(rng, T, E)
        ids, _ = topk_route(lg, k)
        for t in range(T):
            want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
            assert list(ids[t]) == want


def test_route_invariants_random():
    rng = np.random.default_rng(1)
    T, E, k = 200, 64, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::7, 3] = lg[::7, 9]          # some exact ties
    ids, w = topk_route(lg, k)
    for t in range(T):
        s = set(ids[t].tolist())
        assert len(s) == k and all(0 <= e < E for e in s)
        sel = lg[t, ids[t]]
        rest = np.delete(lg[t], ids[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)            # slot order: logit descending
        for j in range(k - 1):
            if sel[j] == sel[j + 1]:
                assert ids[t, j] < ids[t, j + 1]    # ties: lower id first
    assert np.allclose(w.sum(1), 1.0, atol=1e-12, rtol=0)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_weights_full_softmax_when_k_equals_e():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    ids, w = topk_route(lg, 12)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w, axis=1)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


def test_weights_are_renormalised_full_softmax():
    """Top-k of the full softmax, renormalised over the chosen k, is the same
    thing as a softmax over the chosen logits."""
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((60, 32)) * 3).astype(np.float32)
    ids, w = topk_route(lg, 5)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12, atol=0)


def test_minus_inf_never_chosen_while_finite_remain():
    lg = np.zeros((3, 6), np.float32)
    lg[:, 4:] = -np.inf
    lg[0, 0] = 5
    ids, w = topk_route(lg, 4)
    assert not np.isin(ids, [4, 5]).any()
    ids, w = topk_route(lg, 6)
    assert np.all(w[:, 4:] == 0.0)
    assert set(ids[0, 4:].tolist()) == {4, 5}


def test_permutation_is_stable_argsort_and_scan():
    rng = np.random.default_rng(4)
    T, E, k = 97, 13, 3
    ids, _ = topk_route(rng.standard_normal((T, E)).astype(np.float32), k)
    counts, offsets, sa = permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(sa, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(sa), np.arange(T * k))
    for e in range(E):
        seg = sa[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg // k) > 0)


def test_permutation_shards_partition_the_full_one():
    rng = np.random.default_rng(5)
    T, E, k = 64, 24, 4
    ids, _ = topk_route(rng.standard_normal((T, E)).astype(np.float32), k)
    _, off_full, sa_full = permute(ids, E)
    parts = []
    for r in range(4):
        c, o, s = permute(ids, E, local_offset=6 * r, local_count=6)
        assert np.array_equal(o, off_full[6 * r:6 * r + 7] - off_full[6 * r])
        parts.append(s)
    assert np.array_equal(np.concatenate(parts), sa_full)


def test_empty_and_dead_experts():
    ids = np.array([[0, 2], [2, 0]], np.int32)
    c, o, s = permute(ids, 4)
    assert list(c) == [2, 0, 2, 0] and list(o) == [0, 2, 2, 4, 4]
    assert list(s) == [0, 3, 1, 2]
    c, o, s = permute(np.zeros((0, 2), np.int32), 3)
    assert list(o) == [0, 0, 0, 0] and s.size == 0


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        topk_route(np.zeros((2, 3), np.float32), 4)
