"""GPU combine vs the fp64 oracle combine (1e-6 relative, the differential
tolerance the fused-combine qualification used), exact zeros for masked
routes, +0.0 for tokens with no active route, power-of-two exactness."""
import numpy as np
import pytest

from oracle.moe import combine_ref
from gpu_util import np_dev

pytestmark = pytest.mark.gpu


def _run(y, rr, w, mask):
    import torch

    import routed_expert_prefill_amd as rep

    out = rep.combine(np_dev(y), np_dev(rr), np_dev(w), None if mask is None else np_dev(mask))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _case(seed, T, k, d, p):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((T * k, d)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    mask = (rng.random((T, k)) >= p).astype(np.uint8)
    rr = rng.permutation(T * k).astype(np.int32)
    return y, rr, w, mask


@pytest.mark.parametrize("seed,T,k,d,p", [(0, 401, 6, 4096, 0.05), (1, 3, 1, 4, 0.0),
                                          (2, 33, 16, 1028, 0.5), (3, 1, 6, 8, 1.0)])
def test_matches_oracle(seed, T, k, d, p):
    y, rr, w, mask = _case(seed, T, k, d, p)
    got = _run(y, rr, w, mask)
    ref = combine_ref(y, rr, w, mask, T, k)
    scale = np.abs(y).max() * np.abs(w).sum(axis=1).max()
    assert np.abs(got - ref).max() <= 1e-6 * scale


def test_masked_routes_never_read():
    T, k, d = 64, 6, 256
    y, rr, w, mask = _case(5, T, k, d, 0.3)
    mask[0] = 0
    base = _run(y, rr, w, mask)
    yp, wp = y.copy(), w.copy()
    rrp = rr.copy().reshape(T, k)
    for t in range(T):
        for j in range(k):
            if not mask[t, j]:
                yp[rr[t * k + j]] = np.nan
                wp[t, j] = np.inf
                rrp[t, j] = 2 ** 30  # far out of range: must not be dereferenced
    got = _run(yp, rrp.reshape(-1), wp, mask)
    assert np.array_equal(base.view(np.uint32), got.view(np.uint32))
    assert np.all(base[0].view(np.uint32) == 0)  # +0.0 bits


def test_signed_zero_and_scaling():
    T, k, d = 16, 4, 64
    y, rr, w, mask = _case(6, T, k, d, 0.2)
    y[rr[0:k]] = -0.0  # token 0 sums only negative zeros -> +0.0
    a = _run(y, rr, w, mask)
    assert np.all(a[0].view(np.uint32) == 0)
    b = _run(y, rr, (w * 8).astype(np.float32), mask)
    assert np.array_equal((a * 8).view(np.uint32), b.view(np.uint32))


def test_no_mask_means_all_active():
    y, rr, w, _ = _case(7, 10, 3, 32, 0.0)
    ones = np.ones((10, 3), np.uint8)
    assert np.array_equal(_run(y, rr, w, None), _run(y, rr, w, ones))


def _run_shared(y, rr, w, mask, shared, want_fp32=True, want_bf16=True):
    import torch

    import routed_expert_prefill_amd as rep

    out, ob = rep.combine_shared(np_dev(y), np_dev(rr), np_dev(w),
                                 None if mask is None else np_dev(mask),
                                 None if shared is None else np_dev(shared),
                                 want_fp32=want_fp32, want_bf16=want_bf16)
    torch.cuda.synchronize()
    o = None if out is None else out.cpu().numpy()
    b = None if ob is None else ob.view(torch.int16).cpu().numpy().view(np.uint16)
    return o, b


@pytest.mark.parametrize("seed,T,k,d,p", [(10, 401, 6, 4096, 0.05), (11, 7, 16, 36, 0.5),
                                          (12, 2, 6, 8, 1.0)])
def test_shared_output_form(seed, T, k, d, p):
    from oracle.moe import combine_shared_ref
    from oracle.numerics import bf16_bits_to_f64

    y, rr, w, mask = _case(seed, T, k, d, p)
    rng = np.random.default_rng(seed + 100)
    shared = rng.standard_normal((T, d)).astype(np.float32)
    out, ob = _run_shared(y, rr, w, mask, shared)
    ref = combine_shared_ref(y, rr, w, mask, shared, T, k)
    scale = np.abs(y).max() * np.abs(w).sum(axis=1).max() + np.abs(shared).max()
    assert np.abs(out - ref).max() <= 1e-6 * scale
    # bf16 copy: round to nearest of the sum, within the fp32 error of the sum
    bf = bf16_bits_to_f64(ob)
    half_ulp = np.ldexp(1.0, np.frexp(ref)[1] - 9)  # bf16 keeps 8 significant bits
    assert np.all(np.abs(bf - ref) <= half_ulp * (1 + 1e-6) + 1e-6 * scale)
    # without shared rows and with only the fp32 output it is the plain combine, bit for bit
    plain, none = _run_shared(y, rr, w, mask, None, want_bf16=False)
    assert none is None
    assert np.array_equal(plain.view(np.uint32), _run(y, rr, w, mask).view(np.uint32))
    # bf16 only
    none2, ob2 = _run_shared(y, rr, w, mask, shared, want_fp32=False)
    assert none2 is None and np.array_equal(ob2, ob)


def test_row_limit_skips_trailing_rows():
    """With a row limit n, a route whose row is n or more is never read, like
    a masked one: the output equals the combine with those routes masked,
    bit for bit, even with NaN in the skipped rows and gates."""
    import torch

    import routed_expert_prefill_amd as rep

    T, k, d = 97, 6, 512
    y, rr, w, mask = _case(20, T, k, d, 0.1)
    n = (T * k * 3) // 4
    yp, wp = y.copy(), w.copy().reshape(-1)
    beyond = rr >= n
    yp[n:] = np.nan
    wp[beyond] = np.nan
    lim = torch.tensor([n], dtype=torch.int32, device="cuda:0")
    for m in (mask, None):
        got = rep.combine(np_dev(yp), np_dev(rr), np_dev(wp.reshape(T, k)),
                          None if m is None else np_dev(m), row_limit=lim)
        eff = (np.ones((T, k), np.uint8) if m is None else m).copy().reshape(-1)
        eff[beyond] = 0
        want = _run(y, rr, w, eff.reshape(T, k))
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    # the shared-output form honours the same bound
    sh = np.random.default_rng(21).standard_normal((T, d)).astype(np.float32)
    o1, _ = rep.combine_shared(np_dev(yp), np_dev(rr), np_dev(wp.reshape(T, k)), np_dev(mask),
                               np_dev(sh), row_limit=lim)
    eff = mask.copy().reshape(-1)
    eff[beyond] = 0
    o2, _ = rep.combine_shared(np_dev(y), np_dev(rr), np_dev(w), np_dev(eff.reshape(T, k)),
                               np_dev(sh))
    torch.cuda.synchronize()
    assert np.array_equal(o1.cpu().numpy().view(np.uint32), o2.cpu().numpy().view(np.uint32))
