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


def _f32_rne(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a non-negative rational to fp32, zero and subnormals
    included (quantum 2^-149 below 2^-126)."""
    if x == 0:
        return Fraction(0)
    e = math.floor(math.log2(x))
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 23)
    n = x / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * q


def _e4m3_torch(v: float) -> float:
    """torch's own e4m3fn cast (round to nearest even, saturating the finite range here)."""
    return float(torch.tensor([min(v, 448.0)], dtype=torch.float32).to(torch.float8_e4m3fn).float())


def _nvfp4_reference(x):
    """NVFP4 of x by exact rational arithmetic, each fp32 step rounded to nearest even by hand, the
    E4M3 step by torch's float8 cast, and every code by searching the E2M1 grid for the nearest
    value (ties to the even code).  Returns (codes, group scale values, t)."""
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    amax = max(abs(Fraction(float(v))) for v in x.ravel())
    t = _f32_rne(amax / 2688)
    codes = np.zeros(x.shape, np.uint8)
    sgs = np.zeros(x.shape[:-1] + (x.shape[-1] // 16,))
    if t == 0:
        return codes, sgs, t
    d = _f32_rne(6 * t)
    for idx in np.ndindex(x.shape[:-1]):
        for g in range(x.shape[-1] // 16):
            blk = [Fraction(float(v)) for v in x[idx + (slice(16 * g, 16 * g + 16),)]]
            a_g = max(abs(v) for v in blk)
            sg = Fraction(_e4m3_torch(float(_f32_rne(a_g / d))))
            sgs[idx + (g,)] = float(sg)
            step = _f32_rne(sg * t)
            inv = _f32_rne(1 / step) if step > 0 else Fraction(0)
            if inv >= Fraction(2) ** 128:   # the fp32 reciprocal rounds to infinity
                inv = Fraction(0)
            for i, v in enumerate(blk):     # magnitude 0 where inv is 0; the sign bit stays
                y = _f32_rne(abs(v) * inv)
                dist = [abs(y - gv) for gv in grid]
                best = [k for k, dd in enumerate(dist) if dd == min(dist)]
                k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
                neg = np.signbit(x[idx + (16 * g + i,)])
                codes[idx + (16 * g + i,)] = k | (8 if neg else 0)
    return codes, sgs, t


def test_nvfp4_matches_exact_step_by_step_reference():
    """Tensor scale, group scales and codes equal an exact rational evaluation of the same fp32
    steps (R30), with the E4M3 rounding taken from torch and the E2M1 rounding from a nearest-grid
    search; inputs span several binades, a zero group, an outlier and negative zeros."""
    rng = np.random.default_rng(11)
    x = quant.bf16_rne(rng.standard_normal((5, 64)) * np.exp(rng.uniform(-4, 4, (5, 1))))
    x[2, 16:32] = 0.0                       # an all-zero group
    x[3, 5] = 40.0                          # an outlier sets the tensor scale
    x[4, 7] = -0.0
    codes, sg_code, t = quant.nvfp4(x)
    rc, rsg, rt = _nvfp4_reference(x)
    assert Fraction(float(t)) == rt
    np.testing.assert_array_equal(quant.e4m3fn_decode(sg_code), rsg)
    np.testing.assert_array_equal(codes, rc)
    # decoding: E2M1 value x group scale x tensor scale
    v = quant.nvfp4_decode(codes, sg_code, t)
    grid = quant.E2M1_GRID
    exp = np.where(rc & 8, -1.0, 1.0) * grid[rc & 7] * np.repeat(rsg, 16, axis=-1) * float(rt)
    np.testing.assert_array_equal(v, exp)


def test_nvfp4_codes_exhaustive_over_bf16():
    """Every finite bf16 value inside a tensor whose scales are fixed by two anchor elements gets the
    code of the exact step-by-step reference."""
    vals = _all_finite_bf16()
    vals = vals[np.abs(vals) <= 2.0 ** 6]
    n = (vals.size + 13) // 14 * 14
    body = np.zeros(n)
    body[:vals.size] = vals
    rows = body.reshape(-1, 14)
    anchors = np.tile([2.0 ** 6, -1.5], (rows.shape[0], 1))  # tensor amax 64; every group has 1.5
    x = np.concatenate([rows, anchors], axis=1)               # groups of 16 = one row each
    codes, sg_code, t = quant.nvfp4(x)
    d = Fraction(float(quant.F32(6) * t))
    assert Fraction(float(t)) == _f32_rne(Fraction(64) / 2688)
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    sgv = quant.e4m3fn_decode(sg_code)[:, 0]
    for r in range(rows.shape[0]):           # every row: every value, and a spread of group maxima
        a_g = max(abs(Fraction(float(v))) for v in x[r])
        assert sgv[r] == _e4m3_torch(float(_f32_rne(a_g / d)))
        step = _f32_rne(Fraction(float(sgv[r])) * Fraction(float(t)))
        inv = _f32_rne(1 / step)
        for i in range(16):
            y = _f32_rne(abs(Fraction(float(x[r, i]))) * inv)
            dist = [abs(y - gv) for gv in grid]
            best = [k for k, dd in enumerate(dist) if dd == min(dist)]
            k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert codes[r, i] & 7 == k and (codes[r, i] >> 3) == int(np.signbit(x[r, i])), (r, i)


def test_nvfp4_exact_on_representable_values_and_zero_tensor():
    # values already on a group's grid come back unchanged: amax = 2688 * 2^-9 makes t = 2^-9 and
    # the group scales 448 and 224 exact; elements on the E2M1 grid times the step
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    t = 2.0 ** -9
    row = np.concatenate([grid, -grid[::-1]]) * 448 * t
    x = np.stack([row, row * 0.5])
    np.testing.assert_array_equal(quant.nvfp4_dequant(x), x)
    c, s, t0 = quant.nvfp4(np.zeros((2, 32)))
    assert t0 == 0 and not c.any() and not s.any()
    # the element that sets the tensor scale maps to +-6 x 448 x t, the top of the format
    rng = np.random.default_rng(3)
    y = quant.bf16_rne(rng.standard_normal((4, 32)))
    codes, sg_code, tt = quant.nvfp4(y)
    i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert codes[i] & 7 == 7 and quant.e4m3fn_decode(sg_code[i[0], i[1] // 16]) == 448.0


def test_nvfp4_vanishing_tensors_match_reference():
    """Tensors small enough that the fp32 tensor scale and the group steps are subnormal, or that a
    step's fp32 reciprocal overflows (the group's magnitudes are then 0, R30), against the exact
    reference; bf16 subnormal inputs included."""
    rng = np.random.default_rng(21)
    base = rng.standard_normal((3, 32)) * np.array([[1.0], [0.05], [8.0]])
    base[1, :16] = -np.abs(base[1, :16])     # an all-negative group: the sign bits must survive
    for k in (116, 122, 126, 128, 132):
        x = quant.bf16_rne(base * 2.0 ** -k)
        codes, sg_code, t = quant.nvfp4(x)
        rc, rsg, rt = _nvfp4_reference(x)
        assert Fraction(float(t)) == rt, k
        np.testing.assert_array_equal(quant.e4m3fn_decode(sg_code), rsg, err_msg=str(k))
        np.testing.assert_array_equal(codes, rc, err_msg=str(k))
    # the largest step is amax / 6; once that is below 1 / FLT_MAX (2^-132 here) every reciprocal
    # overflows: all magnitudes 0, the signs kept
    x = quant.bf16_rne(base * 2.0 ** -132)
    codes, _, t = quant.nvfp4(x)
    assert t > 0 and not (codes & 7).any()
    assert ((codes >> 3) == np.signbit(x)).all()
    # at 2^-128 the regimes mix: some groups keep finite reciprocals and nonzero codes
    c128, _, _ = quant.nvfp4(quant.bf16_rne(base * 2.0 ** -128))
    assert (c128 & 7).any() and not (c128[1] & 7).any()


def test_nvfp4_scaled_value_rounds_in_fp32():
    """R30 rounds |x| * inv to fp32 before the E2M1 rounding.  Found by search: with tensor maximum
    1.5 and group maximum 0.65234375, inv = f32(1/step) = 9.33333302, and x = 0.1875 and 0.375 give
    exact products just below the E2M1 ties 1.75 and 3.5 but fp32 products exactly on them, which
    round to the even codes 4 (2.0) and 6 (4.0) instead of 3 and 5."""
    row = np.zeros((1, 32))
    row[0, :4] = [0.65234375, 0.1875, 0.375, -0.1875]
    row[0, 16] = 1.5                         # the tensor maximum, in the second group
    codes, sg_code, t = quant.nvfp4(row)
    assert list(codes[0, 1:4]) == [4, 6, 8 | 4]
    rc, rsg, rt = _nvfp4_reference(row)
    np.testing.assert_array_equal(codes, rc)


def test_mxfp4_ceil_rule_is_the_smallest_unsaturated_exponent():
    # the quality sweep's alternative MX scale rule: amax 2^-e in (3, 6], i.e. e = ceil(log2(amax/6)),
    # checked against exact rational arithmetic on every finite positive bf16 group maximum
    vals = _all_finite_bf16()
    vals = vals[(vals > 2.0 ** -120) & (vals < 2.0 ** 120)]
    x = np.zeros((vals.size, 32))
    x[:, 3] = vals
    x[:, 7] = -vals / 3
    _, e8 = quant.mxfp4(x, rule="ceil")
    e = e8[:, 0].astype(np.int64) - 127
    for a, k in zip(vals[::97], e[::97]):
        fa = Fraction(float(a))
        assert fa <= 6 * Fraction(2) ** int(k) and fa > 6 * Fraction(2) ** (int(k) - 1), (a, k)
    # the "ocp" rule puts the maximum in [4, 8) instead
    _, e8o = quant.mxfp4(x, rule="ocp")
    scaled = vals * np.ldexp(1.0, -(e8o[:, 0].astype(np.int64) - 127))
    assert np.all((scaled >= 4) & (scaled < 8))
