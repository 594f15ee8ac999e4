"""Pins of the oracle's number formats (bfloat16, OCP E4M3, E8M0 / MX blocks).

Each check ties the oracle to something other than itself: torch's own
float32->bfloat16 and float8_e4m3fn conversions (library routines), exact
rational arithmetic, and hand-derived values of the OCP MX v1.0 rules."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc


def _f32_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    return pats.view(np.float32)


def test_bf16_from_f32_matches_torch_rne():
    """For float32 inputs a single RNE to bf16 is what torch does."""
    v = _f32_patterns()
    ours = orc.bf16_from_f64(v.astype(np.float64))
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def _bf16_exact(q: Fraction) -> Fraction:
    """Round a rational to the nearest bf16 value, ties to even (normal range)."""
    if q == 0:
        return q
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128  # 8 significant bits
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Fraction(lo, 128) * (Fraction(2) ** e)


def test_bf16_from_double_rounds_once():
    """Doubles just above a bf16 midpoint must round up (a detour through
    float32 would round twice and land on the even neighbour)."""
    cases = [1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8 + 2.0 ** -40), 3 + 2.0 ** -7 + 2.0 ** -45,
             1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 123.456789, -0.0001234567]
    rng = np.random.default_rng(7)
    cases += list(rng.standard_normal(2000) * 10.0 ** rng.integers(-20, 20, 2000))
    got = orc.f64_from_bf16(orc.bf16_from_f64(np.array(cases)))
    for c, g in zip(cases, got):
        assert Fraction(g) == _bf16_exact(Fraction(c)), c
    assert orc.bf16_from_f64(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81


def test_bf16_specials():
    v = np.array([np.inf, -np.inf, 0.0, -0.0, 3.5e38, -3.5e38, 1e-45, 2.0 ** -133, 2.0 ** -134 * 1.5])
    b = orc.bf16_from_f64(v)
    assert b[0] == 0x7F80 and b[1] == 0xFF80 and b[2] == 0x0000 and b[3] == 0x8000
    assert b[4] == 0x7F80 and b[5] == 0xFF80  # overflow to infinity
    assert b[7] == 0x0001  # smallest subnormal
    assert b[8] == 0x0001  # 0.75 of the subnormal quantum rounds up to one quantum
    assert b[6] == 0x0000  # far below half a quantum
    assert orc.f64_from_bf16(b[7:8])[0] == 2.0 ** -133


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.f64_from_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
                        orc.f64_from_e4m3(np.arange(256, dtype=np.uint8))])
    v = v[np.isfinite(v)].astype(np.float32)
    v = v[np.abs(v) <= 448]
    ours = orc.e4m3_from_f64(v.astype(np.float64))
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch encodes -0.0 and tiny negatives to 0x80; same for us
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    v = np.array([448.0, 463.99, 464.0, 480.0, 500.0, 1e9, -1e9, -464.0])
    c = orc.e4m3_from_f64(v)
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_mx_block_exponent_rule():
    """OCP MX: shared exponent = floor(log2(amax)) - 8 for E4M3."""
    blocks, want_scale, want_codes = [], [], []
    for n in (-10, 0, 3):
        b = np.zeros(32, np.float32)
        b[5] = 448.0 * 2.0 ** n  # amax 448*2^n -> floor(log2) = 8+n -> scale n
        b[7] = -2.0 ** n
        blocks.append(b)
        want_scale.append(127 + n)
        c = np.zeros(32, np.uint8)
        c[5] = 0x7E
        c[7] = 0x80 | 0x38  # -1.0 = exponent field 7, mantissa 0
        want_codes.append(c)
    b = np.zeros(32, np.float32)
    b[0] = 1.0  # amax = 2^0 -> scale -8 -> element 256 = 0x78
    blocks.append(b)
    want_scale.append(127 - 8)
    c = np.zeros(32, np.uint8)
    c[0] = 0x78
    want_codes.append(c)
    blocks.append(np.zeros(32, np.float32))  # all zero -> code 0
    want_scale.append(0)
    want_codes.append(np.zeros(32, np.uint8))
    b = np.zeros(32, np.float32)
    b[3] = 1.99  # scale -8, 1.99*256 = 509.4 saturates to 448
    blocks.append(b)
    want_scale.append(127 - 8)
    c = np.zeros(32, np.uint8)
    c[3] = 0x7E
    want_codes.append(c)
    codes, scales = orc.mx_quantize(np.stack(blocks))
    assert list(scales[:, 0]) == want_scale
    assert np.array_equal(codes, np.stack(want_codes))


def test_mx_round_trip_and_error_bound():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-20, 20, (64, 1))).astype(np.float32)
    codes, scales = orc.mx_quantize(v)
    d = orc.mx_dequantize(codes, scales)
    s = np.repeat(orc.f64_from_e8m0(scales), 32, axis=-1)
    scaled = np.abs(v.astype(np.float64)) / s
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448)
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * np.abs(v.astype(np.float64))[normal])
    # values already on the grid survive a second pass unchanged
    codes2, scales2 = orc.mx_quantize(d.astype(np.float32))
    assert np.array_equal(orc.mx_dequantize(codes2, scales2), d)


def test_mx_quantize_rejects_ragged():
    with pytest.raises(ValueError):
        orc.mx_quantize(np.zeros((2, 33), np.float32))
