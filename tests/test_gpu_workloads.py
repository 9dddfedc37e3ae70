"""The five synthetic workloads at full size, in the launch configuration the
benchmark times (MoEPrefill: route build, grouped FFN, combine).

Route tables are compared bit for bit in full.  Outputs are compared with the
fp64 per-token oracle on a sample of tokens (the oracle evaluates one token
at a time, regenerating the experts it needs from the seeded generator); the
tiny workload is compared in full.  fp8 activation codes and scales are
compared bit for bit on a sample of rows.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import moe as omoe
from oracle import numerics as nx
from oracle.route import route_table
from routed_expert_prefill_amd import synth
from gpu_util import rel_frob

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "fp8": (5e-2, 5e-3)}
N_SAMPLE = 6


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _sample_tokens(r, T, n):
    rng = np.random.default_rng(123)
    toks = list(rng.choice(T, size=min(n, T), replace=False))
    dead = np.flatnonzero(r.route_mask.sum(axis=1) == 0)
    if dead.size:
        toks.append(int(dead[0]))  # a token with every route masked, if there is one
    return sorted(set(int(t) for t in toks))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload(name):
    import torch

    import routed_expert_prefill_amd as rep

    wl = synth.WORKLOADS[name]
    fp8 = wl.dtype == "fp8"
    print(f"[workload {name}] generating inputs", flush=True)
    r, ten = synth.device_inputs(wl, seed=0, threads=_threads())
    run = rep.MoEPrefill(wl.T, wl.k, wl.E, wl.d, wl.f, fp8=fp8)
    out = run(ten["x"], ten["topk_ids"], ten["topk_w"], ten["route_mask"], ten["w_gate"],
              ten["w_up"], ten["w_down"], ten.get("s_gate"), ten.get("s_up"), ten.get("s_down"))
    torch.cuda.synchronize()
    print(f"[workload {name}] GPU path done", flush=True)

    rt = route_table(r.topk_ids, r.route_mask, wl.E)
    for got, ref, what in zip(run.rt, rt, ("counts", "offsets", "sorted_routes", "route_rows")):
        assert np.array_equal(got.cpu().numpy(), ref), what

    if fp8:
        q, s = rep.quant_rows_fp8(ten["x"])
        rows = np.random.default_rng(7).choice(wl.T, 64, replace=False)
        xs = nx.bf16_bits_to_f64(r.x[rows]).astype(np.float32)
        qr, sr = nx.quant_rows_fp8(xs)
        assert np.array_equal(q.cpu().numpy()[rows], qr)
        assert np.array_equal(s.cpu().numpy()[rows], sr)

    toks = _sample_tokens(r, wl.T, N_SAMPLE if wl.T > 64 else wl.T)
    if wl.T <= 64:
        toks = list(range(wl.T))
    needed = sorted({int(r.topk_ids[t, j]) for t in toks for j in range(wl.k) if r.route_mask[t, j]})
    with ThreadPoolExecutor(_threads()) as ex:
        cache = dict(zip(needed, ex.map(lambda e: synth.expert_weights(wl, e, 0), needed)))
    ref = omoe.moe_ref_per_token(r.x, r.topk_ids, r.topk_w, r.route_mask, cache.__getitem__, wl.E,
                                 fp8=fp8, tokens=toks)
    got = out.cpu().numpy()[toks].astype(np.float64)
    err = np.abs(got - ref).max()
    rel = rel_frob(got, ref)
    print(f"[workload {name}] tokens={len(toks)} max_abs={err:.3e} rel_frob={rel:.3e}", flush=True)
    assert err <= TOL[wl.dtype][0] and rel <= TOL[wl.dtype][1], (err, rel)
    for i, t in enumerate(toks):
        if r.route_mask[t].sum() == 0:
            assert np.all(out[t].cpu().numpy().view(np.uint32) == 0)
    del ten, run, out
    torch.cuda.empty_cache()
