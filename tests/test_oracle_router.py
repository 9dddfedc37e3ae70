"""Pins of the router oracle (oracle/router.py) against definitions it does not
share code with: a library sort with the stated tie rule, the full softmax
(scipy) when every expert is selected, closed forms, and invariances."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle.router import route_topk, select_topk_row


def _library_topk(z, k):
    # descending value, ties to the lower index: one key sort
    return sorted(range(len(z)), key=lambda e: (-z[e], e))[:k]


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_library_sort_with_ties(seed):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        z = rng.integers(-3, 4, E).astype(np.float32).tolist()  # many ties
        assert select_topk_row(z, k) == _library_topk(z, k)


def test_all_selected_gates_are_the_softmax():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((20, 16)).astype(np.float32)
    ids, w = route_topk(logits, None, 16)
    for t in range(20):
        ref = softmax(logits[t].astype(np.float64))[ids[t]].astype(np.float32)
        ulp = np.spacing(ref)
        assert np.all(np.abs(w[t] - ref) <= ulp), (w[t], ref)
        assert np.all(np.diff(logits[t][ids[t]]) <= 0)


def test_equal_logits_closed_form():
    ids, w = route_topk(np.full((3, 10), 0.25, np.float32), None, 4)
    assert (ids == np.arange(4)).all()
    assert (w == np.float32(1.0 / 4)).all()


def test_top1_gate_is_one():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((30, 8)).astype(np.float32)
    ids, w = route_topk(logits, None, 1)
    assert (w == 1.0).all()
    assert (ids[:, 0] == np.argmax(logits, axis=1)).all()


def test_bias_is_added_in_fp32_before_selection():
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2))  # 1 + 2^-23
    # expert 0: 1 + 0.6 ulp rounds to 1 + 1 ulp in fp32 and ties expert 1,
    # so the lower index wins; in fp64 expert 1 would be larger
    logits = np.array([[one, up]], np.float32)
    bias = np.array([0.6 * 2.0 ** -23, 0.0], np.float32)
    ids, w = route_topk(logits, bias, 2)
    assert ids.tolist() == [[0, 1]]
    assert w[0, 0] == w[0, 1] == np.float32(0.5)


def test_gates_sum_to_one_and_descend():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 64)).astype(np.float32)
    bias = (rng.standard_normal(64) * 0.5).astype(np.float32)
    ids, w = route_topk(logits, bias, 6)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 6 * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(40):
        assert len(set(ids[t].tolist())) == 6


def test_shift_invariance_on_exact_values():
    rng = np.random.default_rng(4)
    logits = rng.integers(-20, 20, (10, 32)).astype(np.float32)
    a = route_topk(logits, None, 6)
    b = route_topk(logits + np.float32(64), None, 6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_generator_routing_agrees():
    # the workloads' generator selects with the same rule, in its own code
    from routed_expert_prefill_amd import synth

    wl = synth.WORKLOADS["tiny_T32_d512_f256_E16"]
    z = synth.make_logits(wl, seed=0)
    r = synth.make_routing(wl, seed=0)
    ids, w = route_topk(z, None, wl.k)
    assert np.array_equal(ids, r.topk_ids)
    assert np.all(np.abs(w - r.topk_w) <= np.spacing(r.topk_w))
