"""GPU route build vs the oracle: bit-exact counts, offsets, sorted_routes and
route_rows, on the workloads' routings and on edge cases."""
import numpy as np
import pytest

from oracle.route import route_table
from routed_expert_prefill_amd import synth
from gpu_util import np_dev, routing_with_counts

pytestmark = pytest.mark.gpu


def _gpu_table(ids, mask, E):
    import torch

    import routed_expert_prefill_amd as rep

    rt = rep.route_build(np_dev(ids), None if mask is None else np_dev(mask), E)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in rt]


def _check(ids, mask, E):
    got = _gpu_table(ids, mask, E)
    ref = route_table(ids, mask, E)
    for g, r, name in zip(got, ref, ("counts", "offsets", "sorted_routes", "route_rows")):
        assert np.array_equal(g, r), name


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_routings(name):
    wl = synth.WORKLOADS[name]
    r = synth.make_routing(wl, seed=0)
    _check(r.topk_ids, r.route_mask, wl.E)


@pytest.mark.parametrize("T,k,E,p,seed", [
    (1, 1, 1, 0.0, 0), (1, 6, 256, 0.0, 1), (7, 3, 5, 0.3, 2), (21, 3, 256, 0.5, 3),
    (700, 6, 256, 0.05, 4), (20000, 6, 256, 0.05, 5), (4097, 16, 256, 0.2, 6), (333, 2, 2, 0.1, 7),
    # 1024-route steps of the one-workgroup path and the chunked path
    (1024, 1, 256, 0.1, 8), (1025, 1, 256, 0.1, 9), (4096, 4, 256, 0.05, 10),
    (4097, 4, 256, 0.05, 11), (2731, 6, 100, 0.3, 12),
    # around the one-workgroup limit (5,120 routes); chunk counts around the
    # scatter's eight-chunk load groups, few bins, an empty trailing bin
    (1024, 5, 256, 0.1, 13), (1025, 5, 256, 0.1, 14), (1024, 6, 256, 0.1, 18),
    (1536, 6, 7, 0.2, 15),
    (8193, 1, 256, 0.0, 16), (2048, 4, 256, 1.0, 17),
])
def test_random(T, k, E, p, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    mask = (rng.random((T, k)) >= p).astype(np.uint8)
    _check(ids, mask, E)


def test_edge_cases():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 16, (40, 6)).astype(np.int32)
    _check(ids, None, 16)  # no mask
    _check(ids, np.zeros((40, 6), np.uint8), 16)  # all masked
    _check(np.full((50, 4), 7, np.int32), np.ones((50, 4), np.uint8), 16)  # one expert takes all
    ids2, mask2 = routing_with_counts([0, 5, 0, 0, 64, 1, 0, 130], 6, 1, masked_extra=9, invalid_extra=4)
    _check(ids2, mask2, 8)  # empty experts, out-of-range ids count as masked
    neg = ids.copy()
    neg[::3, 1] = -5
    _check(neg, np.ones_like(neg, dtype=np.uint8), 16)


def test_repeatable_and_workspace_contents_ignored():
    import torch

    import routed_expert_prefill_amd as rep

    rng = np.random.default_rng(11)
    ids = np_dev(rng.integers(0, 256, (5000, 6)).astype(np.int32))
    mask = np_dev((rng.random((5000, 6)) > 0.05).astype(np.uint8))
    lib = rep.load_library()
    ws = torch.full((lib.moe_route_build_workspace(5000, 6, 256),), 0xAB, dtype=torch.uint8,
                    device=ids.device)
    a = [t.clone() for t in rep.route_build(ids, mask, 256, workspace=ws)]
    for _ in range(5):
        b = rep.route_build(ids, mask, 256, workspace=ws)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
