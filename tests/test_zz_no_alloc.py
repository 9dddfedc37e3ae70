"""moe_route_build_noalloc (the route build on the library's own device
scratch, for callers that cannot allocate) against moe_route_build on the
same inputs, bit for bit, over consecutive calls that reuse the scratch with
a smaller input each time, and against the integer oracle.  Runs after the
other GPU tests (and alone): its name sorts last."""
import numpy as np
import pytest

from oracle.route import route_table
from routed_expert_prefill_amd import synth
from gpu_util import np_dev

pytestmark = pytest.mark.gpu


def _tables(ids, mask, E):
    import torch

    import routed_expert_prefill_amd as rep

    di = np_dev(ids)
    dm = None if mask is None else np_dev(mask)
    a = rep.route_build_noalloc(di, dm, E)
    b = rep.route_build(di, dm, E)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in b]


def test_noalloc_matches_workspace_route_build_on_consecutive_calls():
    from routed_expert_prefill_amd import _lib

    rng = np.random.default_rng(5)
    cases = []
    # the largest call the scratch holds: 2^20 routes, every chunk slot used
    Tm, km = _lib.MOE_ROUTE_NOALLOC_MAX_ROUTES // 16, 16
    cases.append((rng.integers(0, 256, (Tm, km)).astype(np.int32),
                  (rng.random((Tm, km)) >= 0.05).astype(np.uint8), 256))
    # the 8192-token Zipf-routed chunk, then smaller calls reusing the scratch
    wl = synth.WORKLOADS["prefill_T8192_zipf_bf16"]
    r = synth.make_routing(wl, seed=0)
    cases.append((r.topk_ids, r.route_mask, wl.E))
    ids = rng.integers(-3, 100, (3000, 6)).astype(np.int32)  # ids outside [0,E) too
    cases.append((ids, (rng.random((3000, 6)) >= 0.2).astype(np.uint8), 97))
    cases.append((rng.integers(0, 16, (100, 4)).astype(np.int32), None, 16))  # one-workgroup path
    for ids, mask, E in cases:
        got, ref = _tables(ids, mask, E)
        for g, w, name in zip(got, ref, ("counts", "offsets", "sorted_routes", "route_rows")):
            assert np.array_equal(g, w), (ids.shape, name)
        if ids.size <= 50000:
            oracle = route_table(ids, mask, E)
            for g, w, name in zip(got, oracle, ("counts", "offsets", "sorted_routes", "route_rows")):
                assert np.array_equal(g, w), (ids.shape, name, "oracle")


def test_noalloc_rejects_beyond_the_scratch_without_touching_outputs():
    import torch

    import routed_expert_prefill_amd as rep
    from routed_expert_prefill_amd import _lib

    T = _lib.MOE_ROUTE_NOALLOC_MAX_ROUTES // 4 + 1
    ids = torch.zeros((T, 4), dtype=torch.int32, device="cuda:0")
    with pytest.raises(RuntimeError, match="MOE_ETOOLARGE"):
        rep.route_build_noalloc(ids, None, 8)
