"""Expert-owner sharding, one owner at a time on one GPU.

With the experts split into G contiguous ranges, owner g runs the unchanged
path on route_mask AND (expert in range g).  Non-owned routes fall into the
masked bin, so every route is computed by exactly one owner and the G
partial outputs sum to the single-GPU output up to fp32 summation order; a
token with no owned route gets exactly +0.0 from that owner ("perf(ds4):
batch heterogeneous MoE prefill by expert", Summary: grouped graphs per
owner, non-owned routes are exact-zero contributions)."""
import numpy as np
import pytest

from oracle import moe as omoe
from routed_expert_prefill_amd import synth
from gpu_util import bf16_dev, np_dev, rel_frob

pytestmark = pytest.mark.gpu


def _run(r, W, E, mask):
    import torch

    import routed_expert_prefill_amd as rep

    T, k = r.topk_ids.shape
    d = r.x.shape[1]
    f = W["wg"].shape[1]
    run = rep.MoEPrefill(T, k, E, d, f)
    out = run(bf16_dev(r.x), np_dev(r.topk_ids), np_dev(r.topk_w), np_dev(mask),
              bf16_dev(W["wg"]), bf16_dev(W["wu"]), bf16_dev(W["wd"]))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_owner_partials_sum_to_full_output():
    wl = synth.Workload(name="owner_test", T=96, d=256, f=256, E=64, k=6, x_std=1.0, w_std=0.02,
                        mask_p=0.1, routing="softmax", dtype="bf16")
    r = synth.make_routing(wl, seed=3)
    ws = [synth.expert_weights(wl, e, 3) for e in range(wl.E)]
    W = {n: np.stack([w[n] for w in ws]) for n in ("wg", "wu", "wd")}
    full = _run(r, W, wl.E, r.route_mask)
    G = 8
    parts = []
    for g in range(G):
        m = synth.owner_mask(r.topk_ids, r.route_mask, wl.E, G, g)
        out_g = _run(r, W, wl.E, m)
        none = m.sum(axis=1) == 0
        assert np.all(out_g[none].view(np.uint32) == 0)  # exact +0.0
        ref_g = omoe.moe_ref_per_token(r.x, r.topk_ids, r.topk_w, m, omoe.dict_source(W), wl.E)
        assert np.abs(out_g - ref_g).max() <= 2e-2
        assert rel_frob(out_g, ref_g) <= 1e-3
        parts.append(out_g.astype(np.float32))
    total = np.zeros_like(parts[0])
    for p_ in parts:
        total += p_
    assert rel_frob(total, full) <= 1e-6
    assert np.abs(total - full).max() <= 1e-6 * np.abs(full).max()
