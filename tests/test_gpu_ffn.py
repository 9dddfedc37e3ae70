"""GPU grouped FFN + combine vs the fp64 per-token oracle.

Tolerances: bf16 max-abs <= 2e-2 and relative Frobenius <= 1e-3; fp8
5e-2 / 5e-3.  Both sides round h to bf16 (and quantise x and h per row in
fp8) at the same point, so what is left is fp32 accumulation order and rare
bf16 rounding-boundary flips of h.

The per-expert row counts below put experts in every tile capacity and at
its edges: remainders of 1-32 rows (32-row tiles), 33-64, 65-128, 129-192
and 193-256, full 256-row tiles plus a remainder, and empty experts.
"""
import numpy as np
import pytest

from oracle import moe as omoe
from oracle.route import route_table
from gpu_util import bf16_dev, np_dev, rel_frob, routing_with_counts

pytestmark = pytest.mark.gpu

BF16_TOL = (2e-2, 1e-3)
FP8_TOL = (5e-2, 5e-3)


def _weights(E, d, f, fp8, seed, w_std=0.02):
    import torch

    rng = np.random.default_rng(seed)
    W = {}
    shapes = {"wg": (E, f, d), "wu": (E, f, d), "wd": (E, d, f)}
    for n, shp in shapes.items():
        z = rng.standard_normal(shp).astype(np.float32)
        if fp8:
            z = np.clip(z * 112.0, -448, 448).astype(np.float32)
            W[n] = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            W[n] = torch.from_numpy(z * np.float32(w_std)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if fp8:
        for n, src in (("sg", "wg"), ("su", "wu"), ("sd", "wd")):
            e, r, c = shapes[src]
            W[n] = (rng.uniform(0.5, 2.0, (e, r // 128, c // 128)) * (w_std / 448.0)).astype(np.float32)
    return W


def _x(T, d, seed, std=1.0):
    import torch

    rng = np.random.default_rng(seed + 1000)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32) * np.float32(std))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dev_weights(W, fp8):
    if fp8:
        return {n: np_dev(a) for n, a in W.items()}
    return {n: bf16_dev(a) for n, a in W.items()}


def _run(ids, w, mask, x, W, E, fp8, y_fill=None):
    import torch

    import routed_expert_prefill_amd as rep

    T, k = ids.shape
    d = x.shape[1]
    f = W["wg"].shape[1]
    Wd = _dev_weights(W, fp8)
    run = rep.MoEPrefill(T, k, E, d, f, fp8=fp8)
    if y_fill is not None:
        run.y.fill_(y_fill)
    out = run(bf16_dev(x), np_dev(ids), np_dev(w), np_dev(mask), Wd["wg"], Wd["wu"], Wd["wd"],
              Wd.get("sg"), Wd.get("su"), Wd.get("sd"))
    torch.cuda.synchronize()
    return run, out.cpu().numpy().astype(np.float64)


def _check(got, ref, tol):
    err = np.abs(got - ref).max()
    rel = rel_frob(got, ref)
    assert err <= tol[0] and rel <= tol[1], (err, rel)
    return err, rel


CLASS_COUNTS = [0, 1, 7, 16, 17, 31, 32, 33, 64, 128, 129, 160, 161, 192, 193, 250, 300, 0, 2]


@pytest.mark.parametrize("fp8", [False, True])
def test_tile_classes(fp8):
    E = len(CLASS_COUNTS)
    d, f = (256, 256) if fp8 else (384, 256)
    ids, mask = routing_with_counts(CLASS_COUNTS, 6, seed=1, masked_extra=13)
    T, k = ids.shape
    rng = np.random.default_rng(2)
    w = rng.random((T, k)).astype(np.float32)
    x = _x(T, d, 3)
    W = _weights(E, d, f, fp8, 4)
    run, out = _run(ids, w, mask, x, W, E, fp8, y_fill=float("nan"))
    # routes reach y in sorted order; masked rows (>= offsets[E]) are never written
    rt = route_table(ids, mask, E)
    assert np.array_equal(run.rt.offsets.cpu().numpy(), rt.offsets)
    y = run.y.cpu().numpy()
    n_act = int(rt.offsets[E])
    assert np.all(np.isnan(y[n_act:]))
    assert not np.any(np.isnan(y[:n_act]))
    src = omoe.dict_source(W)
    # per-route FFN outputs on a sample of routes from every expert
    sample = [int(rt.sorted_routes[i]) for i in range(0, n_act, 7)]
    yr = omoe.route_outputs_ref(x, ids, src, sample, fp8=fp8)
    _check(y[rt.route_rows[sample]], yr, FP8_TOL if fp8 else BF16_TOL)
    ref = omoe.moe_ref_per_token(x, ids, w, mask, src, E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)


# Several experts with more than 256 rows (their 256-row tiles are handed out
# from the compute queue) beside many small ones (the stream queue), so both
# queues hold many items and workgroups switch between them.
QUEUE_COUNTS = [700, 1, 520, 33, 257, 0, 300, 5, 64, 129, 17, 200, 2, 40, 90, 3, 513, 31, 8, 256]


@pytest.mark.parametrize("fp8", [False, True])
def test_compute_and_stream_queues(fp8):
    E = len(QUEUE_COUNTS)
    d, f = 256, 256
    ids, mask = routing_with_counts(QUEUE_COUNTS, 6, seed=11, masked_extra=29)
    T, k = ids.shape
    rng = np.random.default_rng(12)
    w = rng.random((T, k)).astype(np.float32)
    x = _x(T, d, 13)
    W = _weights(E, d, f, fp8, 14)
    run, out = _run(ids, w, mask, x, W, E, fp8, y_fill=float("nan"))
    rt = route_table(ids, mask, E)
    n_act = int(rt.offsets[E])
    y = run.y.cpu().numpy()
    assert not np.any(np.isnan(y[:n_act]))  # every item of both queues ran
    assert np.all(np.isnan(y[n_act:]))
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)


@pytest.mark.parametrize("fp8", [False, True])
def test_tiny_workload_random_routing(fp8):
    rng = np.random.default_rng(5)
    T, k, E, d, f = 45, 6, 16, 512, 256
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    mask = (rng.random((T, k)) >= 0.1).astype(np.uint8)
    mask[3] = 0  # a token with no active route
    w = rng.random((T, k)).astype(np.float32)
    x = _x(T, d, 6)
    W = _weights(E, d, f, fp8, 7)
    _, out = _run(ids, w, mask, x, W, E, fp8)
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)
    assert np.all(out[3] == 0) and not np.any(np.signbit(out[3]))


@pytest.mark.parametrize("T,d,f,seed", [(1, 256, 384, 20), (3, 384, 256, 21), (4, 512, 2048, 22),
                                         (5, 256, 256, 23)])
def test_decode_sized_chunks(T, d, f, seed):
    """At most 32 routed rows: items narrowed to 128 or 64 weight rows (4, 512,
    2048 takes 128 for gate/up and 64 for down on a 256-CU device)."""
    rng = np.random.default_rng(seed)
    k, E = 6, 64
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T >= 3:
        ids[1] = ids[0]  # an expert with more than one row
    mask = (rng.random((T, k)) >= 0.2).astype(np.uint8)
    w = rng.random((T, k)).astype(np.float32)
    x = _x(T, d, seed + 1)
    W = _weights(E, d, f, False, seed + 2)
    run, out = _run(ids, w, mask, x, W, E, False, y_fill=float("nan"))
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E)
    _check(out, ref, BF16_TOL)
    n_act = int(run.rt.offsets[E].item())
    y = run.y.cpu().numpy()
    assert np.all(np.isnan(y[n_act:])) and not np.any(np.isnan(y[:n_act]))


SKINNY_COUNTS = [1, 5, 9, 17, 20, 24, 28, 31, 32, 3, 12, 7, 0, 30, 26, 15]
MIXED_COUNTS = [40, 70, 130, 300, 10, 20, 5, 64, 200, 33, 1, 2, 0, 513]
COUNT_SETS = {
    "skinny": SKINNY_COUNTS,
    "mixed": MIXED_COUNTS,
    # 40 and 8 experts of at most 32 rows: at d = 2048 (eight blocks of 256
    # outputs per tile) four-block items would leave fewer items than half
    # the workgroups of a 256-CU device, so the kernel halves the blocks per
    # item (to two for 40 experts, to one for 8)
    "skinny40": [(7 * e) % 29 + 3 for e in range(40)],
    "skinny8": [5, 32, 17, 1, 30, 9, 22, 14],
}


@pytest.mark.parametrize("fp8,counts,d", [
    (False, "skinny", 1024), (False, "mixed", 1024), (False, "skinny", 1536), (False, "mixed", 1536),
    (False, "skinny40", 2048), (False, "skinny8", 2048),
    (True, "mixed", 384), (True, "mixed", 768), (True, "skinny", 1024)])
def test_feature_blocks_per_item(fp8, counts, d):
    """Down-projection items of one, two and four feature blocks: only 32-row
    tiles ("skinny") or many taller tiles ("mixed").  bf16 blocks are 256
    outputs: d = 1024 is tiled by items of 512 and 1024 outputs, d = 1536
    only by 512.  fp8 blocks are 128 outputs, each with its own row of weight
    block scales: d = 384 takes one block per item, 768 two, 1024 four.
    Every active row of y is written, every masked row is not."""
    cnt = COUNT_SETS[counts]
    E, f = len(cnt), 256
    ids, mask = routing_with_counts(cnt, 6, seed=30, masked_extra=9)
    T, k = ids.shape
    w = np.random.default_rng(31).random((T, k)).astype(np.float32)
    x = _x(T, d, 32)
    W = _weights(E, d, f, fp8, 33)
    run, out = _run(ids, w, mask, x, W, E, fp8, y_fill=float("nan"))
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)
    n_act = int(run.rt.offsets[E].item())
    y = run.y.cpu().numpy()
    assert np.all(np.isnan(y[n_act:])) and not np.any(np.isnan(y[:n_act]))


def _random_case(seed):
    """A seeded random shape: E, k, d, f, token count, mask rate and a skewed
    (Zipf-like) expert choice, so that tiles of every class, skinny and mixed
    queues and one-tile experts all occur across the seeds."""
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([8, 40, 100, 256]))
    k = int(rng.choice([k for k in (1, 2, 6, 8) if k <= E]))
    d = int(rng.choice([256, 512, 1024]))
    f = int(rng.choice([128, 256, 384]))
    T = int(rng.integers(1, 900 // k + 1))
    p = (np.arange(1, E + 1, dtype=np.float64)) ** -float(rng.choice([0.0, 1.2, 2.0]))
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    mask = (rng.random((T, k)) >= float(rng.choice([0.0, 0.1, 0.5]))).astype(np.uint8)
    w = rng.random((T, k)).astype(np.float32)
    return E, k, d, f, ids, mask, w


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Random shapes against the per-token oracle, bf16 for even seeds and fp8
    for odd ones; every active row of y written, no masked row."""
    fp8 = seed % 2 == 1
    E, k, d, f, ids, mask, w = _random_case(seed)
    T = ids.shape[0]
    x = _x(T, d, 40 + seed)
    W = _weights(E, d, f, fp8, 50 + seed)
    run, out = _run(ids, w, mask, x, W, E, fp8, y_fill=float("nan"))
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)
    n_act = int(run.rt.offsets[E].item())
    y = run.y.cpu().numpy()
    assert np.all(np.isnan(y[n_act:])) and not np.any(np.isnan(y[:n_act]))


def test_single_expert_single_route_is_dense_mlp():
    """E = 1, k = 1, gate 1, no mask: a dense SwiGLU MLP, checked also against
    torch's own matmul on the GPU (an independent library product)."""
    import torch

    T, d, f = 300, 512, 384
    ids = np.zeros((T, 1), np.int32)
    mask = np.ones((T, 1), np.uint8)
    w = np.ones((T, 1), np.float32)
    x = _x(T, d, 8)
    W = _weights(1, d, f, False, 9)
    _, out = _run(ids, w, mask, x, W, 1, False)
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), 1)
    _check(out, ref, BF16_TOL)
    X = bf16_dev(x).float()
    Wg, Wu, Wd = (bf16_dev(W[n][0]).float() for n in ("wg", "wu", "wd"))
    h = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)).to(torch.bfloat16).float()
    lib_ref = (h @ Wd.T).cpu().numpy()
    _check(out, lib_ref, BF16_TOL)


def test_deterministic_and_zero_input():
    import torch

    import routed_expert_prefill_amd as rep

    ids, mask = routing_with_counts([40, 3, 0, 150, 20], 4, seed=10, masked_extra=5)
    T, k = ids.shape
    E, d, f = 5, 256, 256
    w = np.random.default_rng(1).random((T, k)).astype(np.float32)
    x = _x(T, d, 11)
    W = {n: bf16_dev(a) for n, a in _weights(E, d, f, False, 12).items()}
    run = rep.MoEPrefill(T, k, E, d, f)
    args = (np_dev(ids), np_dev(w), np_dev(mask), W["wg"], W["wu"], W["wd"])
    first = run(bf16_dev(x), *args).clone()
    for _ in range(4):
        run.ffn_ws.fill_(0xFF)  # stale workspace contents must not matter
        again = run(bf16_dev(x), *args)
        assert torch.equal(first.view(torch.int32), again.view(torch.int32))
    zero = run(bf16_dev(np.zeros_like(x)), *args)
    torch.cuda.synchronize()
    assert torch.all(zero.view(torch.int32) == 0)


@pytest.mark.parametrize("fp8", [False, True])
def test_active_routes_with_out_of_range_ids_add_exact_zeros(fp8):
    """An active route whose id lies outside [0, E) counts as masked on both
    sides: the route build sends it to the trailing bin, the FFN never writes
    its row of y (NaN-filled here), the combine reads no row at or past
    offsets[E], and the oracle skips it.  Tokens whose only active routes are
    such ids get exactly +0.0."""
    E, d, f = 12, 256, 256
    counts = [30, 0, 7, 64, 1, 0, 40, 3, 12, 0, 33, 5]
    ids, mask = routing_with_counts(counts, 6, seed=60, masked_extra=11, invalid_extra=17)
    T, k = ids.shape
    ids = ids.copy()
    bad = np.flatnonzero(ids.reshape(-1) >= E)
    ids.reshape(-1)[bad[::2]] = -7  # negative ids too
    # a token whose routes are all active and all out of range
    ids = np.concatenate([ids, np.array([[E + 1, -1, 2 ** 20, -(2 ** 30), E, E + 5]], np.int32)])
    mask = np.concatenate([mask, np.ones((1, 6), np.uint8)])
    T += 1
    w = np.random.default_rng(61).random((T, k)).astype(np.float32)
    x = _x(T, d, 62)
    W = _weights(E, d, f, fp8, 63)
    run, out = _run(ids, w, mask, x, W, E, fp8, y_fill=float("nan"))
    assert np.all(np.isfinite(out))
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)
    valid = (mask != 0) & (ids >= 0) & (ids < E)
    none = np.flatnonzero(valid.sum(axis=1) == 0)
    assert T - 1 in none
    for t in none:
        assert np.all(out[t] == 0) and not np.any(np.signbit(out[t])), t
    n_act = int(run.rt.offsets[E].item())
    assert n_act == int(valid.sum())
    y = run.y.cpu().numpy()
    assert np.all(np.isnan(y[n_act:])) and not np.any(np.isnan(y[:n_act]))


@pytest.mark.parametrize("fp8", [False, True])
def test_stage_calls_run_again_on_one_plan(fp8):
    """moe_ffn_gate_up and moe_ffn_down may run again without a new
    moe_ffn_plan (each persistent GEMM resets its queue heads when its last
    workgroup leaves); the second pass writes the same bits."""
    import torch

    import routed_expert_prefill_amd as rep

    E, d, f = len(QUEUE_COUNTS), 256, 256
    ids, mask = routing_with_counts(QUEUE_COUNTS, 6, seed=70, masked_extra=7)
    T, k = ids.shape
    x = _x(T, d, 71)
    Wn = _weights(E, d, f, fp8, 72)
    Wd = _dev_weights(Wn, fp8)
    rt = rep.route_build(np_dev(ids), np_dev(mask), E)
    desc = rep.ffn_desc(T, k, E, d, f, fp8)
    ws = rep._ffn_ws(desc, torch.device("cuda:0"), None)
    y = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda:0")
    xd = bf16_dev(x)
    rep.ffn_plan(desc, xd, rt.offsets, ws)
    rep.ffn_gate_up(desc, xd, rt.sorted_routes, Wd["wg"], Wd["wu"], Wd.get("sg"), Wd.get("su"), ws)
    rep.ffn_down(desc, rt.offsets, Wd["wd"], Wd.get("sd"), y, ws)
    torch.cuda.synchronize()
    first = y.clone()
    n_act = int(rt.offsets[E].item())
    for _ in range(2):
        y.fill_(float("nan"))
        rep.ffn_gate_up(desc, xd, rt.sorted_routes, Wd["wg"], Wd["wu"], Wd.get("sg"), Wd.get("su"),
                        ws)
        rep.ffn_down(desc, rt.offsets, Wd["wd"], Wd.get("sd"), y, ws)
        torch.cuda.synchronize()
        assert torch.equal(first[:n_act].view(torch.int32), y[:n_act].view(torch.int32))
        assert torch.all(torch.isnan(y[n_act:]))
    w = np.random.default_rng(73).random((T, k)).astype(np.float32)
    out = rep.combine(y, rt.route_rows, np_dev(w), np_dev(mask)).cpu().numpy().astype(np.float64)
    ref = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(Wn), E, fp8=fp8)
    _check(out, ref, FP8_TOL if fp8 else BF16_TOL)


# Experts of 257 to 2000 rows at the workloads' width (d = 4096, f = 2048):
# 35 256-row tiles of multi-tile experts (560 compute-queue items per
# projection), including the 208- and 220-row last tiles of the 2000- and
# 1500-row experts, beside remainder tiles of 13 to 188 rows on the stream
# queue; compared in full with the expert-major oracle.
TALL_COUNTS = [1100, 1037, 900, 0, 1300, 257, 2000, 700, 1500, 600]


def test_compute_bound_tiles():
    from threadpoolctl import threadpool_limits

    E, d, f = len(TALL_COUNTS), 4096, 2048
    ids, mask = routing_with_counts(TALL_COUNTS, 6, seed=80, masked_extra=40)
    T, k = ids.shape
    w = np.random.default_rng(81).random((T, k)).astype(np.float32)
    x = _x(T, d, 82)
    W = _weights(E, d, f, False, 83)
    run, out = _run(ids, w, mask, x, W, E, False, y_fill=float("nan"))
    n_act = int(run.rt.offsets[E].item())
    y = run.y.cpu().numpy()
    assert np.all(np.isnan(y[n_act:])) and not np.any(np.isnan(y[:n_act]))
    with threadpool_limits(limits=16):
        ref_out, ref_y, _ = omoe.moe_ref_blocked(x, ids, w, mask, omoe.dict_source(W), E)
    _check(y[:n_act].astype(np.float64), ref_y[:n_act], BF16_TOL)
    _check(out, ref_out, BF16_TOL)
    toks = [0, T // 2, T - 1]
    ref_tok = omoe.moe_ref_per_token(x, ids, w, mask, omoe.dict_source(W), E, tokens=toks)
    _check(out[toks], ref_tok, BF16_TOL)
