"""Pins for the oracle's number formats: e4m3 decode and rounding, bf16 rounding.

Each check ties the oracle to something other than itself: the format's
closed-form anchors, torch's own float8_e4m3fn / bfloat16 casts (library
routines), exhaustive enumeration, or exact rational arithmetic."""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.bf16_ref import bf16_bits_of_fraction


def test_e4m3_anchors(orc):
    assert orc.e4m3_value(0x7E) == 448.0          # largest finite
    assert orc.e4m3_value(0xFE) == -448.0
    assert orc.e4m3_value(0x38) == 1.0            # exponent field 7 = bias
    assert orc.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert orc.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert orc.e4m3_value(0x00) == 0.0
    v = orc.e4m3_value(0x80)
    assert v == 0.0 and np.signbit(v)
    assert np.isnan(orc.e4m3_value(0x7F)) and np.isnan(orc.e4m3_value(0xFF))
    assert orc.e4m3_value(0x77) == 240.0          # 1.875 * 2^7: finite in the FN variant


def test_e4m3_decode_matches_torch_all_codes(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = orc.e4m3_table()
    nan = np.isnan(ref)
    assert (nan == np.isnan(ours)).all()
    assert nan.sum() == 2
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(v.astype(np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _all_rounding_probes() -> np.ndarray:
    grid = np.array([float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float())
                     for c in range(0x7F)], dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2           # exact in fp32 (few significant bits)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    probes = [grid.astype(np.float32), mids32,
              np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(0)),
              np.array([464.0, 470.0, 479.99, 480.0, 500.0, 1e6, 3e38], dtype=np.float32),
              np.array([2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -11, 1e-30, 1e-45], dtype=np.float32)]
    rng = np.random.default_rng(7)
    probes.append((rng.standard_normal(20000) * 100).astype(np.float32))
    probes.append(np.exp2(rng.uniform(-14, 9, 20000)).astype(np.float32))
    p = np.concatenate(probes)
    return np.concatenate([p, -p])


def test_e4m3_rounding_matches_torch(orc):
    v = _all_rounding_probes()
    ours = np.array([orc.e4m3_from_float(float(x)) for x in v], dtype=np.uint8)
    ref = _torch_e4m3(v)
    # +-0 codes are both acceptable only when the value rounds to zero
    zero = (ref & 0x7F) == 0
    assert np.array_equal(ours[~zero], ref[~zero])
    assert ((ours[zero] & 0x7F) == 0).all()


def test_e4m3_rounding_edge_cases(orc):
    assert orc.e4m3_from_float(448.0) == 0x7E
    assert orc.e4m3_from_float(464.0) == 0x7E      # midpoint 448/480: even code 0x7E
    assert orc.e4m3_from_float(470.0) == 0x7E      # saturates (not the NaN slot)
    assert orc.e4m3_from_float(1e30) == 0x7E
    assert orc.e4m3_from_float(-1e30) == 0xFE
    assert orc.e4m3_from_float(-0.0) == 0x80
    assert orc.e4m3_from_float(2.0 ** -10) == 0x00  # half the smallest subnormal: tie -> even 0
    assert orc.e4m3_from_float(3 * 2.0 ** -10) == 0x02  # 1.5 subnormal steps: tie -> even 2
    assert orc.e4m3_from_float(1.0 + 1.0 / 16) == 0x38  # midpoint 1 / 1.125 -> even (1.0)
    assert orc.e4m3_from_float(1.0 + 3.0 / 16) == 0x3A  # midpoint 1.125 / 1.25 -> even (1.25)
    assert orc.e4m3_from_float(float("nan")) & 0x7F == 0x7F


def _bf16_val(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def test_bf16_exhaustive_exact_midpoints_and_neighbours(orc):
    """Every finite positive bf16 value maps to itself; the exact midpoint to
    its upper neighbour goes to the even pattern; a hair above or below the
    midpoint goes to the nearer one."""
    for bits in range(0x0000, 0x7F80):
        v = _bf16_val(bits)
        assert orc.bf16_from_double(v) == bits
        assert orc.bf16_from_double(-v) == (bits | 0x8000)
        if bits + 1 < 0x7F80:
            nxt = _bf16_val(bits + 1)
            mid = (v + nxt) / 2                     # exact in fp64
            even = bits if bits % 2 == 0 else bits + 1
            assert orc.bf16_from_double(mid) == even
            eps = (nxt - v) * 2.0 ** -30
            assert orc.bf16_from_double(mid + eps) == bits + 1
            assert orc.bf16_from_double(mid - eps) == bits


def test_bf16_overflow_and_specials(orc):
    top = _bf16_val(0x7F7F)
    half_ulp = 2.0 ** (127 - 8)
    assert orc.bf16_from_double(top + half_ulp * 0.999) == 0x7F7F
    assert orc.bf16_from_double(top + half_ulp) == 0x7F80   # tie to even -> inf
    assert orc.bf16_from_double(1e300) == 0x7F80
    assert orc.bf16_from_double(-1e300) == 0xFF80
    assert orc.bf16_from_double(float("inf")) == 0x7F80
    assert orc.bf16_from_double(float("nan")) & 0x7F80 == 0x7F80
    assert orc.bf16_from_double(2.0 ** -134) == 0x0000      # half the smallest subnormal -> even 0
    assert orc.bf16_from_double(2.0 ** -134 * 1.5) == 0x0001
    assert orc.bf16_from_double(-0.0) == 0x8000


def test_bf16_matches_torch_on_fp32_inputs(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(50000) * 10,
                        np.exp2(rng.uniform(-140, 127, 20000)) * rng.choice([-1, 1], 20000)])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    ours = np.array([orc.bf16_from_double(float(x)) for x in v32], dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_single_rounding_from_fp64(orc):
    """Rounding straight from fp64 differs from rounding through fp32 on
    values just above a bf16 midpoint; the oracle rounds once."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        x = float(rng.standard_normal() * 2.0 ** rng.integers(-20, 20))
        assert orc.bf16_from_double(x) == bf16_bits_of_fraction(Fraction(x))
    # 1 + 2^-8 + 2^-40: above the midpoint 1 + 2^-8, but fp32 would round it to the midpoint
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert orc.bf16_from_double(x) == 0x3F81
    assert bf16_bits_of_fraction(Fraction(x)) == 0x3F81
