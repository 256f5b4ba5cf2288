"""Pins for oracle.mxfp8: closed-form codec vs torch's float8_e4m3fn, a
hand-worked golden file, exact round trips, exhaustive bf16 sweep."""
import math

import numpy as np
import pytest
import torch

from oracle import mxfp8
from tests.conftest import golden_path
from workloads import bf16_bits_to_f32


def torch_e4m3_cast(v):
    """torch CPU float -> float8_e4m3fn (round to nearest even, keeps -0,
    non-saturating); callers clamp to +-448 first."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = mxfp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits).astype(np.float64)
    return v[np.isfinite(v)]


def test_encode_matches_torch_on_every_bf16_value():
    v = all_finite_bf16()
    c = np.clip(v, -448.0, 448.0)
    assert np.array_equal(mxfp8.e4m3_encode(v), torch_e4m3_cast(c))


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 500)]).astype(np.float32)
    c = np.clip(v.astype(np.float64), -448.0, 448.0)
    assert np.array_equal(mxfp8.e4m3_encode(v.astype(np.float64)), torch_e4m3_cast(c))


def test_block_exponent_against_log2():
    v = all_finite_bf16()
    v = np.abs(v[v != 0])
    X = mxfp8.block_exponent(v)
    ref = np.array([min(127, max(-127, math.floor(math.log2(x)) - 8)) for x in v])
    assert np.array_equal(X, ref)
    assert mxfp8.block_exponent(0.0) == -127


def _golden_blocks():
    blocks, cur = [], None
    for line in open(golden_path("mxfp8_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "block":
            cur = dict(name=vals[0], v=np.zeros(32), codes=np.zeros(32, np.uint8), scale=None)
            blocks.append(cur)
        elif key == "v":
            cur["v"][int(vals[0])] = float(vals[1])
        elif key == "scale":
            cur["scale"] = int(vals[0])
        elif key == "code":
            cur["codes"][int(vals[0])] = int(vals[1], 16)
    return blocks


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b["name"])
def test_quantize_hand_worked_blocks(blk):
    codes, scales = mxfp8.quantize(blk["v"][None, :], axis=1)
    assert scales.tolist() == [[blk["scale"]]]
    assert codes[0].tolist() == blk["codes"].tolist()


def test_round_trip_exact_on_representable_blocks():
    rng = np.random.default_rng(1)
    pos = mxfp8.e4m3_decode(np.arange(0x7F))
    for X in (-127, -100, -20, -8, 0, 5, 60, 110):
        for _ in range(20):
            # grid values times 2^X, with the block max in [256, 448] so the
            # chosen X is the one the rule picks back
            vals = rng.choice(pos, size=32) * rng.choice([-1.0, 1.0], size=32)
            vals[rng.integers(32)] = rng.choice(pos[(pos >= 256)]) * rng.choice([-1.0, 1.0])
            v = np.ldexp(vals, X)
            c, s = mxfp8.quantize(v[None, :], axis=1)
            if X > -127:
                assert s[0, 0] == X + 127
                assert np.array_equal(mxfp8.dequantize(c, s, axis=1)[0], v)


def test_saturation_and_zero_block():
    v = np.zeros((1, 32))
    v[0, 0] = 470.0          # floor(log2 470) = 8 -> X = 0, 470 saturates
    v[0, 1] = -500.0
    c, s = mxfp8.quantize(v, axis=1)
    assert s[0, 0] == 127 and c[0, 0] == 0x7E and c[0, 1] == 0xFE
    c, s = mxfp8.quantize(np.zeros((2, 64)), axis=1)
    assert np.all(s == 0) and np.all(c == 0)
    c, s = mxfp8.quantize(-np.zeros((1, 32)), axis=1)
    assert np.all(c == 0x80)


def test_axis0_equals_axis1_of_transpose():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 96))
    c0, s0 = mxfp8.quantize(v, axis=0)
    c1, s1 = mxfp8.quantize(v.T, axis=1)
    assert np.array_equal(c0, c1.T) and np.array_equal(s0, s1.T)


def test_relative_error_bound():
    """In E4M3's normal range a value keeps 3 mantissa bits:
    |DQ(Q(v)) - v| <= 2^-4 |v| for 2^-6 <= |v| / 2^X <= 448; above 448 (the
    block max can reach 512 * 2^X under the floor rule) it saturates."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((256, 32)) * np.exp(rng.uniform(-5, 5, size=(256, 1)))
    c, s = mxfp8.quantize(v, axis=1)
    dq = mxfp8.dequantize(c, s, axis=1)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    sat = np.abs(v) > np.ldexp(448.0, X)
    normal = (np.abs(v) >= np.ldexp(1.0, X - 6)) & ~sat
    assert np.all(np.abs(dq - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4)
    assert np.all(np.abs(dq)[sat] == np.ldexp(448.0, X)[sat])
