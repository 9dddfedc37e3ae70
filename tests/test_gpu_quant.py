"""GPU per-row E4M3 quantisation vs the oracle: codes and scales bit-exact."""
import numpy as np
import pytest

from oracle import numerics as nx
from routed_expert_prefill_amd.synth import f32_to_bf16_bits
from gpu_util import bf16_dev

pytestmark = pytest.mark.gpu


def _gpu(xbits):
    import torch

    import routed_expert_prefill_amd as rep

    q, s = rep.quant_rows_fp8(bf16_dev(xbits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,cols,scale", [(64, 4096, 1.0), (37, 2048, 3e-3), (5, 128, 50.0),
                                             (300, 16384, 1.0), (8, 256, 2.0 ** -60),
                                             (3, 384, 1.0), (2, 4224, 1.0), (1031, 640, 7.0),
                                             (4, 512, 2.0 ** -128), (4, 512, 2.0 ** 110)])
def test_matches_oracle(rows, cols, scale):
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
    x[0, :5] = [0.0, -0.0, 1e-30, -1e-30, 0.0]
    bits = f32_to_bf16_bits(x)
    q, s = _gpu(bits)
    qr, sr = nx.quant_rows_fp8(nx.bf16_bits_to_f64(bits).astype(np.float32))
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


def test_values_on_and_near_rounding_boundaries():
    """Quotients on and within a few ulp of E4M3 rounding boundaries (ties to
    even, normal and subnormal ranges), for scales that are and are not
    powers of two."""
    rng = np.random.default_rng(12)
    mids = np.array([432.0, 208.0, 17.0, 1.0625, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 3.5 * 2.0 ** -9,
                     2.0 ** -6 * 1.0625, 7.5 * 2.0 ** -9], np.float64)
    rows = []
    for amax in (448.0, 300.0, 1.0, 7.3e-3, 5.1e4):
        sc = np.float32(np.float32(amax) / np.float32(448.0))
        r = (mids[rng.integers(0, len(mids), 255)] * np.float64(sc) *
             rng.choice([-1.0, 1.0], 255)).astype(np.float32)
        row = np.concatenate([[np.float32(amax)], r]).astype(np.float32)
        rows.append(row)
    x = np.stack(rows)
    bits = f32_to_bf16_bits(x)
    # nudge some values by one bf16 ulp either way
    bits[:, 1::3] += 1
    bits[:, 2::3] -= 1
    q, s = _gpu(bits)
    qr, sr = nx.quant_rows_fp8(nx.bf16_bits_to_f64(bits).astype(np.float32))
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


def test_zero_rows_and_wide_dynamic_range():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    x[1] = 0.0
    x[2] = -0.0
    x[3, 7] = 3e4  # one large value pushes the rest into the subnormal codes
    x[4] *= 1e-6
    bits = f32_to_bf16_bits(x)
    q, s = _gpu(bits)
    qr, sr = nx.quant_rows_fp8(nx.bf16_bits_to_f64(bits).astype(np.float32))
    assert np.array_equal(q, qr) and np.array_equal(s, sr)
    assert s[1] == 1.0 and not q[1].any() and not q[2].any()


def test_every_bf16_value_with_unit_scale():
    """Rows whose largest magnitude is 448 have scale 1, so every quotient is
    the bf16 value itself: all finite bf16 patterns of magnitude at most 448,
    both signs, against the oracle's encoder (every E4M3 code, every tie,
    the subnormal codes)."""
    mags = np.arange(0, 0x43e0 + 1, dtype=np.uint16)  # +0 .. 448 as bf16 bit patterns
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    cols = 4096
    per_row = cols - 1
    nrows = -(-len(vals) // per_row)
    bits = np.zeros((nrows, cols), np.uint16)
    bits[:, 0] = 0x43e0  # 448
    flat = np.resize(vals, nrows * per_row)  # the last row repeats values from the start
    bits[:, 1:] = flat.reshape(nrows, per_row)
    q, s = _gpu(bits)
    qr, sr = nx.quant_rows_fp8(nx.bf16_bits_to_f64(bits).astype(np.float32))
    assert np.all(s == 1.0) and np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)
