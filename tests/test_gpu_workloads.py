"""The five synthetic workloads at full size, in the launch configuration the
benchmark times (MoEPrefill: route build, grouped FFN, combine).

Route tables are compared bit for bit in full.  Every token's output and
every active route's row of y are compared with the fp64 oracle: the
expert-major variant ``moe_ref_blocked``, which is pinned to the literal
per-token loop at 1e-12 on the CPU, evaluated on all experts (weights
regenerated from the seeded generator, never read back from the GPU).  y is
filled with NaN before the run: every row below offsets[E] must then be
written and every row at or past it left alone.  A sample of tokens is also
checked against the literal per-token loop itself.  fp8 activation codes and
scales are compared bit for bit on a sample of rows.
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
N_SAMPLE = 4


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _host_experts(wl):
    """Every expert's weights, regenerated on the host from the seeded generator."""
    with ThreadPoolExecutor(_threads()) as ex:
        return dict(zip(range(wl.E), ex.map(lambda e: synth.expert_weights(wl, e, 0), range(wl.E))))


def _check(got, ref, tol, what):
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    rel = rel_frob(got, ref)
    print(f"  {what}: max_abs={err:.3e} rel_frob={rel:.3e}", flush=True)
    assert err <= tol[0] and rel <= tol[1], (what, err, rel)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload(name):
    import torch

    import routed_expert_prefill_amd as rep
    from threadpoolctl import threadpool_limits

    wl = synth.WORKLOADS[name]
    fp8 = wl.dtype == "fp8"
    tol = TOL[wl.dtype]
    print(f"[workload {name}] generating inputs", flush=True)
    r, ten = synth.device_inputs(wl, seed=0, threads=_threads())
    assert np.all((r.topk_ids >= 0) & (r.topk_ids < wl.E))
    run = rep.MoEPrefill(wl.T, wl.k, wl.E, wl.d, wl.f, fp8=fp8)
    run.y.fill_(float("nan"))
    out = run(ten["x"], ten["topk_ids"], ten["topk_w"], ten["route_mask"], ten["w_gate"],
              ten["w_up"], ten["w_down"], ten.get("s_gate"), ten.get("s_up"), ten.get("s_down"))
    torch.cuda.synchronize()
    print(f"[workload {name}] GPU path done", flush=True)

    rt = route_table(r.topk_ids, r.route_mask, wl.E)
    for got, ref, what in zip(run.rt, rt, ("counts", "offsets", "sorted_routes", "route_rows")):
        assert np.array_equal(got.cpu().numpy(), ref), what
    n_act = int(rt.offsets[wl.E])

    # y: rows of active routes all written, rows of masked routes untouched
    y = run.y.cpu().numpy()
    assert not np.any(np.isnan(y[:n_act])), "an active row of y was not written"
    assert np.all(np.isnan(y[n_act:])), "a masked row of y was written"
    got_out = out.cpu().numpy().astype(np.float64)
    del ten, run, out
    torch.cuda.empty_cache()

    if fp8:
        xq = torch.from_numpy(r.x.view(np.int16)).view(torch.bfloat16).cuda()
        q, s = rep.quant_rows_fp8(xq)
        rows = np.random.default_rng(7).choice(wl.T, 64, replace=False)
        xs = nx.bf16_bits_to_f64(r.x[rows]).astype(np.float32)
        qr, sr = nx.quant_rows_fp8(xs)
        assert np.array_equal(q.cpu().numpy()[rows], qr)
        assert np.array_equal(s.cpu().numpy()[rows], sr)
        del xq, q, s

    print(f"[workload {name}] oracle over all {wl.T} tokens", flush=True)
    W = _host_experts(wl)
    with threadpool_limits(limits=_threads()):
        ref_out, ref_y, _ = omoe.moe_ref_blocked(r.x, r.topk_ids, r.topk_w, r.route_mask,
                                                 W.__getitem__, wl.E, fp8=fp8)
    print(f"[workload {name}] T={wl.T} active rows={n_act}", flush=True)
    _check(y[:n_act].astype(np.float64), ref_y[:n_act], tol, "y (every active route)")
    _check(got_out, ref_out, tol, "out (every token)")
    dead = np.flatnonzero(r.route_mask.sum(axis=1) == 0)
    for t in dead:
        assert np.all(got_out[t] == 0) and not np.any(np.signbit(got_out[t])), t  # +0.0

    # a few tokens against the literal per-token loop as well
    toks = sorted(set(np.random.default_rng(123).choice(wl.T, min(N_SAMPLE, wl.T),
                                                         replace=False).tolist()))
    ref_tok = omoe.moe_ref_per_token(r.x, r.topk_ids, r.topk_w, r.route_mask, W.__getitem__,
                                     wl.E, fp8=fp8, tokens=toks)
    _check(got_out[toks], ref_tok, tol, f"out (tokens {toks}, per-token loop)")
