"""Pins for the oracle's FFN and combine (CPU only).

* per-token loop vs brute-force dense "all experts x gate mask" evaluation;
* expert-major blocked evaluation vs the per-token loop;
* one expert, one route, gate 1, no mask -> a dense SwiGLU MLP evaluated with
  torch CPU ops (torch's silu, matmul and bfloat16 conversion);
* block-scale dequantisation vs a Kronecker-product expansion;
* combine vs a dense one-hot gate matrix product;
* invariants: zero input, masked routes (NaN-poisoned), power-of-two gate
  scaling, token permutation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe, numerics as nx
from helpers import rel_frob, small_problem


def _src(weights):
    return moe.dict_source(weights)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed,T,E,k", [(0, 9, 5, 3), (1, 4, 3, 3), (2, 6, 8, 2)])
def test_per_token_matches_dense(seed, T, E, k, fp8):
    d, f = (256, 128) if fp8 else (48, 40)
    ids, w, mask, x, W = small_problem(seed, T, E, k, d, f, fp8=fp8, mask_p=0.25)
    a = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E, fp8=fp8)
    b = moe.moe_ref_dense(x, ids, w, mask, _src(W), E, fp8=fp8)
    assert rel_frob(a, b) <= 1e-12
    assert np.abs(a).max() > 0


@pytest.mark.parametrize("fp8", [False, True])
def test_blocked_matches_per_token(fp8):
    T, E, k = 24, 6, 4
    d, f = (256, 128) if fp8 else (64, 96)
    ids, w, mask, x, W = small_problem(7, T, E, k, d, f, fp8=fp8, mask_p=0.2)
    a = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E, fp8=fp8)
    out, y, rt = moe.moe_ref_blocked(x, ids, w, mask, _src(W), E, fp8=fp8)
    assert rel_frob(out, a) <= 1e-12
    # y rows hold the per-route FFN outputs
    rs = [r for r in range(T * k) if mask.reshape(-1)[r]][:10]
    yr = moe.route_outputs_ref(x, ids, _src(W), rs, fp8=fp8)
    assert rel_frob(y[rt.route_rows[rs]], yr) <= 1e-12


def test_single_expert_is_dense_swiglu_mlp_bf16():
    T, d, f = 16, 64, 32
    ids, w, mask, x, W = small_problem(11, T, 1, 1, d, f, mask_p=0.0)
    w[:] = 1.0
    ours = moe.moe_ref_per_token(x, ids, w, None, _src(W), 1)

    def tb(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)

    X, Wg, Wu, Wd = tb(x), tb(W["wg"][0]), tb(W["wu"][0]), tb(W["wd"][0])
    h = torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)
    h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    ref = (h @ Wd.T).numpy()
    assert rel_frob(ours, ref) <= 1e-12


def test_single_expert_is_dense_swiglu_mlp_fp8():
    T, d, f = 8, 256, 128
    ids, w, mask, x, W = small_problem(12, T, 1, 1, d, f, fp8=True, mask_p=0.0)
    w[:] = 1.0
    ours = moe.moe_ref_per_token(x, ids, w, None, _src(W), 1, fp8=True)

    def deq(codes, scale):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
        return v * torch.from_numpy(np.kron(scale.astype(np.float64), np.ones((128, 128))))

    def tq(rows32):  # per-row quantisation with torch's conversion
        t = rows32.to(torch.float32)
        s = t.abs().amax(dim=1, keepdim=True) / 448.0
        q = (t / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return q * s.to(torch.float64)

    X = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    Xq = tq(X)
    Wg, Wu, Wd = deq(W["wg"][0], W["sg"][0]), deq(W["wu"][0], W["su"][0]), deq(W["wd"][0], W["sd"][0])
    h = torch.nn.functional.silu(Xq @ Wg.T) * (Xq @ Wu.T)
    h = h.to(torch.float32).to(torch.bfloat16)
    ref = (tq(h) @ Wd.T).numpy()
    assert rel_frob(ours, ref) <= 1e-12


def test_block_dequant_matches_kron():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    scale = rng.uniform(0.5, 2, (2, 3)).astype(np.float32)
    ours = moe._block_dequant(codes, scale)
    ref = nx.e4m3_decode(codes) * np.kron(scale.astype(np.float64), np.ones((128, 128)))
    assert np.array_equal(ours, ref)


def test_combine_matches_onehot_matmul():
    rng = np.random.default_rng(6)
    T, k, d = 13, 6, 40
    y = rng.standard_normal((T * k, d)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    mask = (rng.random((T, k)) > 0.3).astype(np.uint8)
    rr = rng.permutation(T * k).astype(np.int32)
    ours = moe.combine_ref(y, rr, w, mask, T, k)
    G = np.zeros((T, T * k))
    for t in range(T):
        for j in range(k):
            if mask[t, j]:
                G[t, rr[t * k + j]] = w[t, j]
    ref = G @ y.astype(np.float64)
    assert rel_frob(ours, ref) <= 1e-14


def test_combine_never_reads_masked_lanes():
    rng = np.random.default_rng(8)
    T, k, d = 6, 4, 16
    y = rng.standard_normal((T * k, d)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    mask = (rng.random((T, k)) > 0.5).astype(np.uint8)
    mask[0] = 0  # one token with no active route
    rr = np.arange(T * k, dtype=np.int32)
    base = moe.combine_ref(y, rr, w, mask, T, k)
    yp, wp, rrp = y.copy(), w.copy(), rr.copy()
    for t in range(T):
        for j in range(k):
            if not mask[t, j]:
                yp[rr[t * k + j]] = np.nan
                wp[t, j] = np.inf
    poisoned = moe.combine_ref(yp, rrp, wp, mask, T, k)
    assert np.array_equal(base.view(np.uint64), poisoned.view(np.uint64))
    assert np.all(base[0].view(np.uint64) == 0)  # +0.0 bits


def test_zero_input_gives_positive_zero():
    T, E, k, d, f = 5, 4, 2, 32, 16
    ids, w, mask, x, W = small_problem(9, T, E, k, d, f)
    x[:] = 0
    out = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    assert np.all(out.view(np.uint64) == 0)


def test_masked_routes_are_exact_zero_even_with_nan_weights():
    T, E, k, d, f = 6, 5, 3, 32, 24
    ids, w, mask, x, W = small_problem(10, T, E, k, d, f, mask_p=0.4)
    base = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    # drop experts only masked routes use, poison their weights, corrupt masked gates
    used = {int(ids[t, j]) for t in range(T) for j in range(k) if mask[t, j]}
    W2 = {n: a.copy() for n, a in W.items()}
    for e in range(E):
        if e not in used:
            for n in ("wg", "wu", "wd"):
                W2[n][e] = 0x7FC0  # bf16 NaN
    w2 = w.copy()
    w2[mask == 0] = np.nan
    got = moe.moe_ref_per_token(x, ids, w2, mask, _src(W2), E)
    assert np.array_equal(base.view(np.uint64), got.view(np.uint64))


def test_power_of_two_gate_scaling_is_exact():
    T, E, k, d, f = 7, 4, 3, 32, 16
    ids, w, mask, x, W = small_problem(13, T, E, k, d, f)
    a = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    b = moe.moe_ref_per_token(x, ids, (w * 4).astype(np.float32), mask, _src(W), E)
    assert np.array_equal(4 * a, b)


def test_token_permutation_equivariance():
    T, E, k, d, f = 10, 5, 3, 32, 16
    ids, w, mask, x, W = small_problem(14, T, E, k, d, f)
    perm = np.random.default_rng(0).permutation(T)
    a = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    b = moe.moe_ref_per_token(x[perm], ids[perm], w[perm], mask[perm], _src(W), E)
    assert np.array_equal(a[perm], b)


def test_rounding_point_of_h_is_observable():
    """Dropping the bf16 rounding of h changes the result by far more than the
    fp32-accumulation noise, so the GPU tolerance can tell them apart."""
    T, E, k, d, f = 8, 3, 2, 512, 256
    ids, w, mask, x, W = small_problem(15, T, E, k, d, f, mask_p=0.0, w_std=0.02)
    a = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    orig = nx.bf16_round
    try:
        moe.nx.bf16_round = lambda v: np.asarray(v, dtype=np.float64)
        b = moe.moe_ref_per_token(x, ids, w, mask, _src(W), E)
    finally:
        moe.nx.bf16_round = orig
    assert rel_frob(b, a) > 1e-3
    assert not math.isnan(rel_frob(b, a))


def test_shared_output_combine_is_routed_plus_shared():
    """Shared-output combine: the dense one-hot product plus the shared rows;
    with no shared rows it is the plain combine."""
    rng = np.random.default_rng(31)
    T, k, d = 9, 4, 12
    R = T * k
    y = rng.standard_normal((R, d))
    rr = rng.permutation(R).astype(np.int32)
    w = rng.random((T, k))
    mask = (rng.random((T, k)) > 0.3).astype(np.uint8)
    shared = rng.standard_normal((T, d))
    G = np.zeros((T, R))
    for t in range(T):
        for j in range(k):
            if mask[t, j]:
                G[t, rr[t * k + j]] += w[t, j]
    ours = moe.combine_shared_ref(y, rr, w, mask, shared, T, k)
    assert np.allclose(ours, G @ y + shared, rtol=1e-13, atol=1e-13)
    plain = moe.combine_shared_ref(y, rr, w, mask, None, T, k)
    assert np.array_equal(plain, moe.combine_ref(y, rr, w, mask, T, k))
