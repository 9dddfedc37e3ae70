"""Pins for the oracle's number formats (CPU only).

bf16 rounding and E4M3 decode/encode are checked against torch's CPU
conversions (independent implementations of the same standards) and against
the landmark values of the format definitions in tests/golden.
"""
import math

import numpy as np
import pytest
import torch

from oracle import numerics as nx
from helpers import read_pairs


def _f32_bits(u32):
    return np.asarray(u32, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- bf16

def test_bf16_landmarks():
    for bits, val in read_pairs("bf16_landmarks.txt"):
        got = nx.bf16_bits_to_f64(np.array([int(bits, 16)], dtype=np.uint16))[0]
        assert got == float(val), (bits, got, val)
        # a landmark is already on the grid
        if math.isfinite(float(val)):
            assert nx.bf16_round(np.array([float(val)]))[0] == float(val)


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = nx.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def _torch_bf16(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_round_matches_torch_random():
    rng = np.random.default_rng(1)
    # random bit patterns cover every binade, subnormals, inf and nan
    u = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = _f32_bits(u)
    with np.errstate(invalid="ignore"):
        ours = nx.bf16_round(x.astype(np.float64))
    ref = _torch_bf16(x)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all(), np.flatnonzero(~same)[:5]


def test_bf16_round_ties_even():
    # fp32 patterns exactly halfway between two bf16 values: low half 0x8000
    hi = np.arange(0x0000, 0x7F7F, 97, dtype=np.uint32)
    x = _f32_bits((hi << 16) | 0x8000)
    ours = nx.bf16_round(x.astype(np.float64))
    ref = _torch_bf16(x)
    assert np.array_equal(ours, ref)
    # tie goes to the even neighbour: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    assert nx.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert nx.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_bf16_round_overflow_and_specials():
    big = (2 - 2.0 ** -8) * 2.0 ** 127  # halfway past the largest finite -> inf
    assert nx.bf16_round(np.array([big]))[0] == np.inf
    assert nx.bf16_round(np.array([-big]))[0] == -np.inf
    assert nx.bf16_round(np.array([3.3895313892515355e38]))[0] == 3.3895313892515355e38
    assert np.isnan(nx.bf16_round(np.array([np.nan]))[0])
    z = nx.bf16_round(np.array([-0.0]))[0]
    assert z == 0 and math.copysign(1, z) == -1


# ---------------------------------------------------------------- e4m3

def test_e4m3_landmarks():
    for code, val in read_pairs("e4m3_landmarks.txt"):
        c = int(code, 16)
        got = nx.e4m3_decode(np.array([c], dtype=np.uint8))[0]
        v = float(val)
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), (code, got, v)
            assert nx.e4m3_encode(np.array([v]))[0] == c


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = nx.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = nx.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(nx.e4m3_encode(vals[fin]), codes[fin])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(447.99), 300_000))
    x = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    ours = nx.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_and_saturation():
    vals = nx.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact halfway points
    ours = nx.e4m3_encode(mids)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.all(ours % 2 == 0)  # ties to the even mantissa
    sat = np.array([448.0, 448.0001, 460.0, 1e30, np.inf], dtype=np.float64)
    assert np.all(nx.e4m3_encode(sat) == 0x7E)
    assert np.all(nx.e4m3_encode(-sat) == 0xFE)
    assert nx.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    assert nx.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert nx.e4m3_encode(np.array([-1e-9]))[0] == 0x80
    assert nx.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00  # tie between 0 and 2^-9 -> even (0)
    assert nx.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02


def _torch_quant_row(row32):
    t = torch.from_numpy(np.asarray(row32, dtype=np.float32))
    amax = t.abs().max()
    if float(amax) == 0.0:
        return np.zeros(t.shape, np.uint8), np.float32(1.0)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    q = (t / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, np.float32(s.item())


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.5, 2.0 ** -20])
def test_quant_row_matches_torch(scale):
    rng = np.random.default_rng(3)
    for _ in range(50):
        row = (rng.standard_normal(512) * scale).astype(np.float32)
        q, s = nx.quant_row_fp8(row)
        qt, st = _torch_quant_row(row)
        assert s == st
        assert np.array_equal(q, qt)
        # the row maximum lands on the largest code
        i = np.argmax(np.abs(row))
        assert (q[i] & 0x7F) == 0x7E
        # every code is within half a step of the scaled value (3 mantissa bits)
        deq = nx.e4m3_decode(q) * np.float64(s)
        big = np.abs(row) > 2.0 ** -6 * float(s)
        assert np.all(np.abs(deq[big] - row[big]) <= np.abs(row[big]) * 2.0 ** -4 * 1.0001)


def test_quant_row_zero():
    q, s = nx.quant_row_fp8(np.zeros(256, np.float32))
    assert s == 1.0 and not q.any()


def test_silu_matches_torch():
    z = np.linspace(-60, 60, 10001)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(nx.silu(z), ref, rtol=1e-15, atol=0)
    assert nx.silu(np.array([-800.0]))[0] == 0.0
