"""Rounding grids and quantisers.  Oracle: test infrastructure only.

Each rounding function is written from the number format's definition: find the binade of |x|,
take that binade's quantum, round |x|/quantum to the nearest integer with ties to even (np.rint),
multiply back, saturate where the format says so.  Per-element arithmetic that the device performs
in fp32 (x*r, 127/a, a/127, 448/a) is done here in numpy float32, which is correctly rounded.

Follows: pchao.org blog on DraftAttention2, section 方法概览 bullet 2 (retained blocks are assigned
16-bit, INT8, then a 4-bit format) and bullet 4 (quantisation is fused into operand preparation;
the attention kernel rescales by the quantisation scales at phase boundaries).

Readings:
  R16 INT8: one symmetric fp32 scale per (head, token block, tensor); codes in [-127, 127]; RNE.
  R17 4-bit: OCP MXFP4 -- 32 channels along D share an E8M0 scale 2^(floor(log2 amax) - 2);
      E2M1 codes, RNE, saturating at 6.  (The pages name NVFP4 as an example; MXFP4 is the 4-bit
      format the gfx950 scaled matrix cores consume.)
  R20 FP8 V: one fp32 scale per (head, channel) over real tokens; e4m3fn codes, RNE, saturating.
  R30 NVFP4 (selectable instead of MXFP4): groups of 16 channels, E4M3 group scales, one fp32
      scale per (head, tensor) over real tokens; the fp32 steps are listed at nvfp4().
  R26 all-zero blocks / groups / channels: INT8 codes 0 with scale 0; MX exponent -127;
      FP8 codes 0 with scale 0.  A block or channel whose maximum is so small that the fp32
      reciprocal of the quantiser (127/a, 448/a) overflows is treated the same way (below about
      3.7e-37 for INT8, 1.3e-36 for FP8 V): its values are zero for every practical purpose, and
      an infinite reciprocal would turn its zeros into NaN codes.
Sign of a code: the IEEE sign bit of the input, also when the magnitude rounds to zero.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ----------------------------------------------------------------------------------------------
# helpers


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite fp64 values that are normal in fp64, read from the
    exponent field (exact; no transcendental)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    return ((a.view(np.uint64) >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64) - 1023


def _round_to_quantum(mag: np.ndarray, quantum: np.ndarray) -> np.ndarray:
    """rint(mag / quantum) * quantum; quantum is a power of two so both steps are exact apart
    from the rounding itself."""
    return np.rint(mag / quantum) * quantum


# ----------------------------------------------------------------------------------------------
# bf16


def bf16_rne(x) -> np.ndarray:
    """Round fp64/fp32 values to bfloat16 (8 significant bits, fp32 exponent range), ties to even.
    Returned as fp64 values on the bf16 grid.  Inputs are finite and far below bf16 overflow."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    nz = mag > 0
    e = np.where(nz, _floor_log2(np.where(nz, mag, 1.0)), 0)
    q = np.ldexp(1.0, np.maximum(e, -126) - 7)   # subnormal quantum 2^-133
    return np.copysign(_round_to_quantum(mag, q), x)


# ----------------------------------------------------------------------------------------------
# FP8 e4m3fn (OCP): bias 7, 3 mantissa bits, no infinities, max finite 448, min normal 2^-6,
# subnormal quantum 2^-9.

E4M3_MAX = 448.0


def e4m3fn_rne_sat(x) -> np.ndarray:
    """Round to the e4m3fn grid, ties to even, saturating at +-448.  fp64 values out."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    nz = mag > 0
    e = np.where(nz, _floor_log2(np.where(nz, mag, 1.0)), 0)
    q = np.ldexp(1.0, np.maximum(e, -6) - 3)
    r = np.minimum(_round_to_quantum(mag, q), E4M3_MAX)
    return np.copysign(r, x)


def e4m3fn_encode(v: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """Byte codes of values already on the e4m3fn grid (|v| <= 448); `neg` gives the sign bit."""
    mag = np.abs(np.asarray(v, dtype=np.float64))
    sub = mag < 2.0 ** -6
    e = np.where(sub, -6, _floor_log2(np.where(mag > 0, mag, 1.0)))
    exp_field = np.where(sub, 0, e + 7)
    mant = np.where(sub, mag / 2.0 ** -9, mag / np.ldexp(1.0, e - 3) - 8.0)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return (code | (np.asarray(neg, bool).astype(np.int64) << 7)).astype(np.uint8)


def e4m3fn_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(ef == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, ef - 10))
    return s * mag


# ----------------------------------------------------------------------------------------------
# E2M1 (OCP FP4): grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}; codes 0..7 in that order, bit 3 = sign.

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_rne_sat(v) -> np.ndarray:
    """Round magnitudes to the E2M1 grid with ties to even, saturating at 6.  Returns the 3-bit
    magnitude code (0..7).  The binade quanta are 0.5 below 2, 1 in [2, 4), 2 from 4 on."""
    mag = np.abs(np.asarray(v, dtype=np.float64))
    q = np.where(mag < 2.0, 0.5, np.where(mag < 4.0, 1.0, 2.0))
    r = np.minimum(_round_to_quantum(mag, q), 6.0)
    return np.searchsorted(E2M1_GRID, r).astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# INT8 per block


def int8_block(x: np.ndarray):
    """Symmetric INT8 of one token block (all rows and channels share one scale).

    x: fp64 values of bf16 inputs (pad rows are 0).  Returns (codes int8, scale float32).
    a = max|x|; r = f32(127/a); code = clamp(rne(f32(x*r)), -127, 127); s = f32(a/127).
    a = 0, or r not finite (a below about 3.7e-37): codes 0, s = 0 (R26)."""
    a = F32(np.max(np.abs(x)))
    if a == 0:
        return np.zeros(x.shape, np.int8), F32(0.0)
    with np.errstate(over="ignore"):
        r = F32(127.0) / a
    if not np.isfinite(r):
        return np.zeros(x.shape, np.int8), F32(0.0)
    c = np.clip(np.rint(np.asarray(x, dtype=F32) * r), -127, 127)
    return c.astype(np.int8), F32(a / F32(127.0))


# ----------------------------------------------------------------------------------------------
# MXFP4 per (row, 32-channel group)


def mxfp4(x: np.ndarray, rule: str = "ocp"):
    """MXFP4 of rows x [..., D] (fp64 values of bf16), groups of 32 consecutive channels.

    Returns (codes uint8 [..., D] in 0..15 with bit 3 = sign, e8m0 uint8 [..., D/32]).
    rule "ocp" (R17, the path's rule): e = floor(log2 amax) - 2, so amax 2^-e lies in [4, 8) and
      the top of that binade saturates at 6.
    rule "ceil" (R17's listed alternative, compared in the quality sweep only): the smallest e with
      amax <= 6 * 2^e, i.e. ceil(log2(amax / 6)): nothing saturates, amax 2^-e lies in (3, 6].
    Either way e is clamped to [-127, 127], amax = 0 gives -127; byte = e + 127.
    code = E2M1_rne_sat(x * 2^-e) with the sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (D // 32, 32))
    a = np.max(np.abs(xg), axis=-1)
    fl = _floor_log2(np.where(a > 0, a, 1.0))
    if rule == "ocp":
        e = np.where(a > 0, fl - 2, -127)
    elif rule == "ceil":
        # log2(a / 6) lies in [fl - 2.59, fl - 1.59): the answer is fl - 2 when a <= 6 * 2^(fl - 2)
        e = np.where(a > 0, np.where(a <= 6.0 * np.ldexp(1.0, fl - 2), fl - 2, fl - 1), -127)
    else:
        raise ValueError(rule)
    e = np.clip(e, -127, 127)
    scaled = xg * np.ldexp(1.0, -e)[..., None]
    mag = e2m1_rne_sat(scaled)
    sign = np.signbit(xg).astype(np.uint8) << 3
    codes = (mag | sign).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_decode(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = E2M1_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    D = c.shape[-1]
    vg = v.reshape(c.shape[:-1] + (D // 32, 32))
    sc = np.ldexp(1.0, np.asarray(e8m0, dtype=np.int64) - 127)
    return (vg * sc[..., None]).reshape(c.shape)


# ----------------------------------------------------------------------------------------------
# NVFP4: the pages' example 4-bit format (pchao.org blog, section 方法概览 bullet 2: the low-bit
# level is, for example, NVFP4) -- E2M1 elements in groups of 16 consecutive channels, each group
# scaled by an E4M3 factor, on top of one fp32 factor for the whole tensor.  The two-level scaling
# is the format's definition; the fp32 order of the steps is reading R30.

NV_GROUP = 16
NV_TOP = F32(6.0 * 448.0)   # largest E2M1 value times largest E4M3 value


def nvfp4(x: np.ndarray, amax=None):
    """NVFP4 of rows x [..., D] (fp64 values of bf16 inputs), one tensor scale for all of x.

    amax = max|x| over the tensor (default: over x itself; pad rows are 0 and do not change it).
    R30, every step in fp32 (numpy float32 is correctly rounded):
      t    = f32(amax / 2688)                   tensor scale; 0 -> every code and scale is 0
      d    = f32(6 * t)
      s_g  = e4m3fn_rne_sat(f32(a_g / d))       group scale, a_g = max|x| over the group's 16
      step = f32(s_g * t);  inv = f32(1 / step) (0 when step is 0 or inv is not finite: the
                                                 group's magnitudes are then 0)
      code = E2M1_rne_sat(f32(|x| * inv)), bit 3 = the IEEE sign bit of x
    Returns (codes uint8 [..., D] 0..15, scale bytes uint8 [..., D/16] (e4m3fn), t float32)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if amax is None:
        amax = float(np.max(np.abs(x))) if x.size else 0.0
    t = F32(F32(amax) / NV_TOP)
    shape_g = x.shape[:-1] + (D // NV_GROUP,)
    if t == 0:
        return np.zeros(x.shape, np.uint8), np.zeros(shape_g, np.uint8), F32(0.0)
    d = F32(F32(6.0) * t)
    xg = x.reshape(x.shape[:-1] + (D // NV_GROUP, NV_GROUP))
    a_g = np.max(np.abs(xg), axis=-1).astype(F32)
    sg_val = e4m3fn_rne_sat((a_g / d).astype(F32).astype(np.float64))
    sg_code = e4m3fn_encode(sg_val, np.zeros(sg_val.shape, bool))
    step = (sg_val.astype(F32) * t).astype(F32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(step > 0, F32(1.0) / np.where(step > 0, step, F32(1.0)), F32(0.0)).astype(F32)
    inv = np.where(np.isfinite(inv), inv, F32(0.0)).astype(F32)
    scaled = (np.abs(xg).astype(F32) * inv[..., None]).astype(F32)
    mag = e2m1_rne_sat(scaled.astype(np.float64))
    sign = np.signbit(xg).astype(np.uint8) << 3
    codes = (mag | sign).reshape(x.shape)
    return codes, sg_code, t


def nvfp4_decode(codes: np.ndarray, sg_code: np.ndarray, t) -> np.ndarray:
    """Values of NVFP4 codes (exact fp64): E2M1 value x E4M3 group scale x tensor scale."""
    c = np.asarray(codes, dtype=np.int64)
    v = E2M1_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    D = c.shape[-1]
    vg = v.reshape(c.shape[:-1] + (D // NV_GROUP, NV_GROUP))
    sg = e4m3fn_decode(sg_code)
    return (vg * sg[..., None] * float(t)).reshape(c.shape)


def nvfp4_dequant(x: np.ndarray) -> np.ndarray:
    """NVFP4 round trip of rows x [..., D] with the tensor scale taken over x (quality sweep)."""
    return nvfp4_decode(*nvfp4(x))


# ----------------------------------------------------------------------------------------------
# FP8 V per channel


def fp8_v(v_real: np.ndarray, vp: np.ndarray):
    """Per-channel e4m3fn quantisation of V.

    v_real: [N, D] fp64 values of bf16 V (real tokens) -- defines the scale.
    vp:     [Np, D] packed V (pad rows 0) -- the rows that get codes.
    a_d = max|V[:, d]|; r = f32(448/a_d); codes = e4m3fn_rne_sat(f32(V*r)); s_d = f32(a_d/448).
    a_d = 0, or r not finite (a_d below about 1.3e-36): codes 0, s_d = 0 (R26).
    Returns (codes uint8 [Np, D], scale float32 [D])."""
    a = np.max(np.abs(v_real), axis=0).astype(F32)
    with np.errstate(over="ignore"):
        r_raw = (F32(448.0) / np.where(a == 0, F32(1), a)).astype(F32)
    zero = (a == 0) | ~np.isfinite(r_raw)
    r = np.where(zero, F32(0), r_raw).astype(F32)
    y = (np.asarray(vp, dtype=F32) * r[None, :]).astype(F32)
    vals = e4m3fn_rne_sat(y.astype(np.float64))
    codes = e4m3fn_encode(vals, np.signbit(vp))
    codes[:, zero] = 0
    s = np.where(zero, F32(0), a / F32(448.0)).astype(F32)
    return codes, s
