"""Pins for the oracle's route table (CPU only): numpy library routines,
a hand-worked example, brute-force ranks and invariants."""
import numpy as np
import pytest

from oracle.route import route_table
from helpers import read_pairs


def _lib_table(ids, mask, E):
    """The same table from numpy primitives: bincount, cumsum, stable argsort."""
    ids = ids.reshape(-1)
    act = np.ones(ids.size, bool) if mask is None else mask.reshape(-1) != 0
    act &= (ids >= 0) & (ids < E)
    key = np.where(act, ids, E)
    counts = np.bincount(key, minlength=E + 1)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.argsort(key, kind="stable")
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    return counts, offsets, order, inv


def _check_invariants(rt, ids, mask, E):
    T, k = ids.shape
    R = T * k
    assert rt.counts.sum() == R
    assert rt.offsets[0] == 0 and rt.offsets[-1] == R
    assert np.all(np.diff(rt.offsets) >= 0)
    assert np.array_equal(np.sort(rt.sorted_routes), np.arange(R))
    assert np.array_equal(rt.sorted_routes[rt.route_rows], np.arange(R))
    act = np.ones(R, bool) if mask is None else mask.reshape(-1) != 0
    flat = ids.reshape(-1)
    for b in range(E + 1):
        seg = rt.sorted_routes[rt.offsets[b]:rt.offsets[b + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending route order
        if b < E:
            assert np.all(flat[seg] == b) and np.all(act[seg])
    # permutation round trip: gather(scatter(v)) == v bit for bit
    v = np.random.default_rng(0).standard_normal(R)
    scattered = np.empty_like(v)
    scattered[rt.route_rows] = v
    assert np.array_equal(scattered[rt.route_rows], v)
    assert np.array_equal(scattered, v[rt.sorted_routes])


def test_worked_example():
    g = {row[0]: [int(v) for v in row[1:]] for row in read_pairs("route_table_worked.txt")}
    T, k, E = g["T"][0], g["k"][0], g["E"][0]
    ids = np.array(g["topk_ids"], np.int32).reshape(T, k)
    mask = np.array(g["route_mask"], np.uint8).reshape(T, k)
    rt = route_table(ids, mask, E)
    assert rt.counts.tolist() == g["counts"]
    assert rt.offsets.tolist() == g["offsets"]
    assert rt.sorted_routes.tolist() == g["sorted_routes"]
    assert rt.route_rows.tolist() == g["route_rows"]


@pytest.mark.parametrize("seed,T,k,E,p", [(0, 50, 6, 16, 0.1), (1, 401, 6, 256, 0.05),
                                          (2, 7, 1, 1, 0.0), (3, 33, 8, 9, 0.5), (4, 1, 6, 256, 0.0)])
def test_matches_numpy(seed, T, k, E, p):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    mask = (rng.random((T, k)) >= p).astype(np.uint8)
    rt = route_table(ids, mask, E)
    c, o, s, r = _lib_table(ids, mask, E)
    assert np.array_equal(rt.counts, c) and np.array_equal(rt.offsets, o)
    assert np.array_equal(rt.sorted_routes, s) and np.array_equal(rt.route_rows, r)
    _check_invariants(rt, ids, mask, E)


def test_brute_force_ranks():
    rng = np.random.default_rng(5)
    for _ in range(20):
        T, k, E = rng.integers(1, 6), rng.integers(1, 4), rng.integers(1, 5)
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
        mask = (rng.random((T, k)) >= 0.3).astype(np.uint8)
        rt = route_table(ids, mask, E)
        key = [int(i) if m else E for i, m in zip(ids.reshape(-1), mask.reshape(-1))]
        for r, kr in enumerate(key):
            pos = sum(1 for kk in key if kk < kr) + sum(1 for rr in range(r) if key[rr] == kr)
            assert rt.route_rows[r] == pos


def test_edge_cases():
    # all masked: everything lands in bin E, in route order
    ids = np.zeros((5, 3), np.int32)
    rt = route_table(ids, np.zeros((5, 3), np.uint8), 4)
    assert rt.counts.tolist() == [0, 0, 0, 0, 15]
    assert rt.sorted_routes.tolist() == list(range(15))
    # no mask given = all active; one expert takes every route
    rt = route_table(np.full((4, 2), 3, np.int32), None, 4)
    assert rt.counts.tolist() == [0, 0, 0, 8, 0]
    assert rt.offsets.tolist() == [0, 0, 0, 0, 8, 8]
    # an active id outside [0, E) is treated as masked; masked ids are ignored
    ids = np.array([[0, 7, -1], [2, 2, 99]], np.int32)
    mask = np.array([[1, 1, 1], [1, 0, 0]], np.uint8)
    rt = route_table(ids, mask, 3)
    assert rt.counts.tolist() == [1, 0, 1, 4]
    assert rt.sorted_routes.tolist() == [0, 3, 1, 2, 4, 5]
    _check_invariants(rt, np.where(mask.astype(bool) & (ids >= 0) & (ids < 3), ids, 0),
                      (mask.astype(bool) & (ids >= 0) & (ids < 3)).astype(np.uint8), 3)
