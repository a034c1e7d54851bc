"""Pins for the oracle's rounding grids and quantisers (CPU).

bf16 and e4m3fn rounding are pinned to PyTorch's own casts; E2M1 to an exhaustive nearest-grid
search over every finite bf16 input; INT8 to exact rational arithmetic; E8M0 to math.frexp."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant


def _all_finite_bf16():
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


# ---------------------------------------------------------------------------------------- bf16

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * np.exp2(rng.integers(-140, 20, 200000)),
        rng.random(50000),                                 # softmax-like values in [0, 1)
    ])
    # exact midpoints between neighbouring bf16 values (ties)
    b = _all_finite_bf16()
    b = np.sort(b[np.abs(b) < 1e30])
    mids = (b[1:] + b[:-1]) / 2
    x = np.concatenate([x, mids[::7]]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(quant.bf16_rne(x), ref)


# ---------------------------------------------------------------------------------------- e4m3fn

def _e4m3_all_values():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, quant.e4m3fn_decode(codes)


def test_e4m3_decode_matches_torch():
    codes, vals = _e4m3_all_values()
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals, ref)


def test_e4m3_rne_matches_torch_cast_within_range():
    codes, vals = _e4m3_all_values()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2                       # every tie
    rng = np.random.default_rng(1)
    samp = rng.uniform(-448, 448, 300000)
    small = rng.standard_normal(100000) * np.exp2(rng.integers(-12, 0, 100000))
    x = np.concatenate([samp, small, mids, -mids, pos, -pos]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(quant.e4m3fn_rne_sat(x), ref)


def test_e4m3_saturates_and_encodes():
    assert quant.e4m3fn_rne_sat(np.array([470.0, 1e6, -1e6]))[0] == 448.0
    assert quant.e4m3fn_rne_sat(np.array([-1e6]))[0] == -448.0
    codes, vals = _e4m3_all_values()
    enc = quant.e4m3fn_encode(vals, codes >= 0x80)
    np.testing.assert_array_equal(enc, codes)


# ---------------------------------------------------------------------------------------- E2M1

def _e2m1_brute(v):
    """Nearest grid magnitude; among equidistant candidates the even code (mantissa bit 0)."""
    grid = quant.E2M1_GRID
    mag = np.minimum(np.abs(v), 1e300)
    d = np.abs(mag[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # prefer even codes, then the larger code among two evens cannot happen (adjacent grid)
    score = np.where(cand, np.where(np.arange(8) % 2 == 0, 2, 1), 0)
    code = np.argmax(score, axis=1)
    over = mag > 6.0                                    # saturation
    return np.where(over, 7, code).astype(np.uint8)


@pytest.mark.parametrize("e", [-127, -20, -3, -2, 0, 1, 5, 30, 125])
def test_e2m1_exhaustive_over_bf16(e):
    x = _all_finite_bf16()
    v = x * 2.0 ** (-e)
    np.testing.assert_array_equal(quant.e2m1_rne_sat(v), _e2m1_brute(v))


def test_mxfp4_scale_exponent_matches_frexp():
    rng = np.random.default_rng(2)
    x = _all_finite_bf16()
    x = x[np.abs(x) > 0]
    rows = rng.choice(x, size=(4000, 64))
    codes, e8 = quant.mxfp4(rows)
    a = np.abs(rows.reshape(4000, 2, 32)).max(axis=2)
    for i in range(0, 4000, 37):
        for j in range(2):
            exp = min(max(math.frexp(a[i, j])[1] - 1 - 2, -127), 127)
            assert int(e8[i, j]) == exp + 127
    # every scaled group max lands in [4, 8) unless the exponent was clamped
    e = e8.astype(np.int64) - 127
    free = (e > -127) & (e < 127)
    scaled = a * np.ldexp(1.0, -e)
    assert np.all((scaled[free] >= 4) & (scaled[free] < 8))


def test_mxfp4_zero_group_and_sign():
    x = np.zeros((1, 64))
    x[0, 33] = -3.0
    codes, e8 = quant.mxfp4(x)
    assert e8[0, 0] == 0                                 # all-zero group -> exponent -127
    assert e8[0, 1] == 127 + (1 - 2)                     # floor(log2 3) = 1 -> e = -1
    assert codes[0, 33] == 8 | 7                         # -3 * 2^1 = -6 -> sign | code of 6
    np.testing.assert_array_equal(quant.mxfp4_decode(codes, e8)[0, 33], -3.0)


# ---------------------------------------------------------------------------------------- INT8

def _f32_rne_fraction(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a positive rational to fp32 (normal range)."""
    e = math.floor(math.log2(x))
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    q = Fraction(2) ** (e - 23)
    n = x / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * q


def test_int8_block_matches_exact_rational_emulation():
    rng = np.random.default_rng(3)
    for trial in range(12):
        x = quant.bf16_rne(rng.standard_normal((16, 8)) * 10 ** rng.uniform(-3, 2))
        codes, s = quant.int8_block(x)
        a = Fraction(float(np.max(np.abs(x))))
        r = _f32_rne_fraction(Fraction(127) / a)
        for i in range(16):
            for j in range(8):
                xv = Fraction(float(x[i, j]))
                y = _f32_rne_fraction(abs(xv) * r) if xv != 0 else Fraction(0)
                fl = math.floor(y)
                rem = y - fl
                if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
                    fl += 1
                c = min(fl, 127) * (1 if xv >= 0 else -1)
                assert int(codes[i, j]) == c
        assert Fraction(float(s)) == _f32_rne_fraction(a / 127)


def test_int8_error_bound_and_absmax_code():
    rng = np.random.default_rng(4)
    for _ in range(50):
        x = quant.bf16_rne(rng.standard_normal((32, 16)) * rng.uniform(0.01, 100))
        codes, s = quant.int8_block(x)
        s = float(s)
        assert np.all(np.abs(x - codes * s) <= s * (0.5 + 2.0 ** -14))
        i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert abs(int(codes[i])) == 127
    c0, s0 = quant.int8_block(np.zeros((4, 4)))
    assert s0 == 0 and not c0.any()


# fp32 overflow bound of a correctly rounded quotient: values at or above (2 - 2^-24) * 2^127 round to
# infinity (IEEE 754 round-to-nearest: the midpoint between the largest finite value and 2^128)
_F32_OVERFLOW = (2 - Fraction(1, 2 ** 24)) * 2 ** 127


def _tiny_bf16_values():
    """Positive bf16 values from the subnormal range up to 1e-30, every one of them."""
    f = _all_finite_bf16()
    return f[(f > 0) & (f < 1e-30)]


def test_int8_block_reciprocal_overflow_is_a_zero_block():
    # Exact rational arithmetic decides for every tiny bf16 maximum whether f32(127/a) overflows;
    # exactly those blocks must come out as zeros with scale 0, all others with the +-127 code.
    hits = 0
    for a in _tiny_bf16_values():
        overflow = Fraction(127) / Fraction(float(a)) >= _F32_OVERFLOW
        x = np.array([[a, -a / 2, 0.0, a / 4]])
        codes, s = quant.int8_block(x)
        if overflow:
            hits += 1
            assert s == 0 and not codes.any(), a
        else:
            assert codes[0, 0] == 127 and codes[0, 2] == 0 and s > 0, a
    assert 0 < hits < _tiny_bf16_values().size


# ---------------------------------------------------------------------------------------- FP8 V

def test_fp8_v_channel_scale_and_zero_channel():
    rng = np.random.default_rng(5)
    v = quant.bf16_rne(rng.standard_normal((100, 8)))
    v[:, 3] = 0.0
    vp = np.concatenate([v, np.zeros((12, 8))])
    codes, s = quant.fp8_v(v, vp)
    assert s[3] == 0 and not codes[:, 3].any()
    for d in (0, 1, 7):
        i = np.argmax(np.abs(v[:, d]))
        assert quant.e4m3fn_decode(codes[i, d]) == np.copysign(448.0, v[i, d])
    deq = quant.e4m3fn_decode(codes) * s.astype(np.float64)
    # e4m3 relative step is 2^-3 in the normal range
    big = np.abs(vp) > np.max(np.abs(v), axis=0) * 2.0 ** -6
    assert np.all(np.abs(deq - vp)[big] <= np.abs(vp)[big] * 2.0 ** -4 * 1.0001)
    assert not codes[100:].any()


def test_fp8_v_reciprocal_overflow_is_a_zero_channel():
    # one channel per tiny bf16 maximum; a channel is zero (codes 0, scale 0) exactly when the exact
    # quotient 448/a rounds to fp32 infinity, otherwise its maximum gets the code for +-448
    tiny = _tiny_bf16_values()
    v = np.zeros((3, tiny.size))
    v[0] = tiny
    v[1] = -tiny / 2
    vp = np.concatenate([v, np.zeros((2, tiny.size))])
    codes, s = quant.fp8_v(v, vp)
    over = np.array([Fraction(448) / Fraction(float(a)) >= _F32_OVERFLOW for a in tiny])
    assert 0 < over.sum() < tiny.size
    assert np.all(s[over] == 0) and not codes[:, over].any()
    ok = ~over
    assert np.all(s[ok] > 0)
    assert np.all(quant.e4m3fn_decode(codes[0, ok]) == 448.0)
    assert np.all(np.isfinite(quant.e4m3fn_decode(codes[:, ok])))


def test_nvfp4_matches_brute_force_nearest_grid_point():
    """Each NVFP4 value is the nearest point of its group's grid {+-E2M1 * step}, step = s_g s_t
    (ties to the even code), with s_g the E4M3 rounding of amax/(6 s_t); found here by exhaustive
    search."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 64)) * np.exp(rng.uniform(-4, 4, (6, 1)))).astype(np.float64)
    x[2, 16:32] = 0.0                       # an all-zero group
    x[3, 5] = 40.0                          # an outlier sets the tensor scale
    got = quant.nvfp4_dequant(x)
    s_t = np.abs(x).max() / (6 * 448)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for r in range(x.shape[0]):
        for g in range(4):
            blk = x[r, 16 * g:16 * g + 16]
            s_g = quant.e4m3fn_rne_sat(np.array([np.abs(blk).max() / (6 * s_t)]))[0]
            for i, v in enumerate(blk):
                if s_g == 0:
                    assert got[r, 16 * g + i] == 0.0
                    continue
                cand = grid * (s_g * s_t)      # the group's grid: E2M1 values times its step
                d = np.abs(np.abs(v) - cand)
                best = np.flatnonzero(d == d.min())
                k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
                exp = np.copysign(cand[k], v) if cand[k] != 0 else (np.copysign(0.0, v))
                assert got[r, 16 * g + i] == exp, (r, g, i, v, got[r, 16 * g + i], exp)


def test_nvfp4_exact_on_representable_values_and_saturates():
    # values already on a group's grid come back unchanged: pick s_t from the tensor max, a group
    # scale on the e4m3 grid, elements on the E2M1 grid
    s_t = 6.0 / (6 * 448)                     # tensor max 6 -> s_t = 1/448
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    row = np.concatenate([grid, -grid[::-1]]) * 448 * s_t   # group scale 448 (largest) -> max 6
    x = np.stack([row, row * 0.5])            # second group: scale 224 (on the e4m3 grid)
    np.testing.assert_array_equal(quant.nvfp4_dequant(x), x)
    # the largest element of every group maps to at most 6 * s_g * s_t
    rng = np.random.default_rng(3)
    y = rng.standard_normal((4, 32))
    v = quant.nvfp4_dequant(y)
    assert np.all(np.abs(v) <= np.abs(y).max() * (1 + 2 ** -3) + 1e-12)
