"""One attention layer end to end, per (batch, head).  Oracle: test infrastructure only.

Pipeline (pchao.org blog on DraftAttention2, Figure 2 caption and section 方法概览; pith.science
DraftAttention abstract for reorder -> attention -> restore):
  pack (reorder + pad) -> avg/max pool -> draft map + lambda mix -> rank + quota assignment
  -> quantise (INT8 per block, MXFP4 per 32-channel group, FP8 V per channel)
  -> phased attention per query block -> restore token order, round the output to bf16 (R25).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import layout, quant, draft, attention


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
        .view(np.float32).astype(np.float64)


@dataclass
class HeadResult:
    g: layout.Geometry
    D: int
    B: int
    valid: np.ndarray                 # [Nb, B] bool
    qp: np.ndarray                    # packed fp64 [Np, D]
    kp: np.ndarray
    vp: np.ndarray
    q_avg: np.ndarray                 # [Nb, D]
    q_max: np.ndarray
    k_avg: np.ndarray
    k_max: np.ndarray
    A: np.ndarray                     # [Nb, Nb] mixed draft map
    A_avg: np.ndarray
    A_max: np.ndarray
    rank: np.ndarray                  # [Nb, Nb]
    cuts: tuple                       # (c16, c8, c4)
    levels: np.ndarray                # [Nb, Nb] uint8
    q_i8: np.ndarray                  # [Np, D] int8
    q_i8_s: np.ndarray                # [Nb] f32
    k_i8: np.ndarray
    k_i8_s: np.ndarray
    q_fp4: np.ndarray                 # [Np, D] codes 0..15
    q_e8: np.ndarray                  # [Np, D/32] uint8
    k_fp4: np.ndarray
    k_e8: np.ndarray
    v_fp8: np.ndarray                 # [Np, D] uint8 e4m3fn codes
    v_s: np.ndarray                   # [D] f32
    fp4_format: str = "mxfp4"         # 4-bit operands: "mxfp4" or "nvfp4" (R17 / R30)
    q_nv: np.ndarray = None           # NVFP4 codes [Np, D] 0..15, E4M3 scale bytes [Np, D/16], tensor scale
    q_nv_s: np.ndarray = None
    q_nv_t: np.float32 = None
    k_nv: np.ndarray = None
    k_nv_s: np.ndarray = None
    k_nv_t: np.float32 = None
    q_fp4_val: np.ndarray = None      # dequantised 4-bit operands (exact fp64)
    k_fp4_val: np.ndarray = None
    v_fp8_val: np.ndarray = None      # V_fp8 * s_V (exact fp64)
    levels_override: Optional[np.ndarray] = None
    out_packed: np.ndarray = None     # [Np, D] fp64, NaN where not computed
    l_packed: np.ndarray = None       # [Np] softmax denominators, NaN where not computed
    computed_blocks: list = field(default_factory=list)

    @property
    def levels_used(self):
        return self.levels if self.levels_override is None else self.levels_override

    def out_bf16(self) -> np.ndarray:
        """Restored [N, D] output rounded to bf16 (NaN rows where not computed)."""
        return quant.bf16_rne(layout.unpack(self.out_packed, self.g))


class _Ops:
    """Operand view handed to the attention step."""

    def __init__(self, r: HeadResult):
        self.B, self.D = r.B, r.D
        self.valid = r.valid
        self.qp, self.kp, self.vp = r.qp, r.kp, r.vp
        self.q_i8, self.k_i8 = r.q_i8, r.k_i8
        self.q_i8_s, self.k_i8_s = r.q_i8_s, r.k_i8_s
        self.q_fp4_val, self.k_fp4_val, self.v_fp8_val = r.q_fp4_val, r.k_fp4_val, r.v_fp8_val
        self.levels = r.levels_used


def prepare_head(q_bits, k_bits, v_bits, *, T, H, W, rh, rw, lam, quota_bp,
                 levels_override=None, fp4_format: str = "mxfp4", mx_rule: str = "ocp") -> HeadResult:
    """Every step up to (not including) attention for one head.  q/k/v_bits: [N, D] bf16 bits.
    fp4_format: the 4-bit level's operands, OCP MXFP4 (R17) or NVFP4 (R30); mx_rule: MXFP4's
    scale rule (see quant.mxfp4; the path implements "ocp", "ceil" is compared in the sweep)."""
    g = layout.geometry(T, H, W, rh, rw)
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    D = q.shape[1]
    qp, kp, vp = layout.pack(q, g), layout.pack(k, g), layout.pack(v, g)
    valid = layout.valid_rows(g)

    q_avg, q_max = draft.pool(qp, valid)
    k_avg, k_max = draft.pool(kp, valid)
    A, A_avg, A_max = draft.draft_map(q_avg, q_max, k_avg, k_max, lam, D)
    rank = draft.rank_pairs(A)
    cuts = draft.cut_ranks(g.Nb * g.Nb, quota_bp)
    levels = draft.assign_levels(rank, cuts)

    B = g.B
    q_i8 = np.zeros((g.Np, D), np.int8)
    k_i8 = np.zeros((g.Np, D), np.int8)
    q_i8_s = np.zeros(g.Nb, np.float32)
    k_i8_s = np.zeros(g.Nb, np.float32)
    for b in range(g.Nb):
        s = slice(b * B, (b + 1) * B)
        q_i8[s], q_i8_s[b] = quant.int8_block(qp[s])
        k_i8[s], k_i8_s[b] = quant.int8_block(kp[s])
    q_fp4, q_e8 = quant.mxfp4(qp, rule=mx_rule)
    k_fp4, k_e8 = quant.mxfp4(kp, rule=mx_rule)
    v_fp8, v_s = quant.fp8_v(v, vp)

    r = HeadResult(g, D, B, valid, qp, kp, vp, q_avg, q_max, k_avg, k_max, A, A_avg, A_max,
                   rank, cuts, levels, q_i8, q_i8_s, k_i8, k_i8_s, q_fp4, q_e8, k_fp4, k_e8,
                   v_fp8, v_s)
    r.fp4_format = fp4_format
    if fp4_format == "nvfp4":
        # one tensor scale per (head, tensor): amax over the packed rows = over the real tokens
        r.q_nv, r.q_nv_s, r.q_nv_t = quant.nvfp4(qp)
        r.k_nv, r.k_nv_s, r.k_nv_t = quant.nvfp4(kp)
        r.q_fp4_val = quant.nvfp4_decode(r.q_nv, r.q_nv_s, r.q_nv_t)
        r.k_fp4_val = quant.nvfp4_decode(r.k_nv, r.k_nv_s, r.k_nv_t)
    elif fp4_format == "mxfp4":
        r.q_fp4_val = quant.mxfp4_decode(q_fp4, q_e8)
        r.k_fp4_val = quant.mxfp4_decode(k_fp4, k_e8)
    else:
        raise ValueError(fp4_format)
    r.v_fp8_val = quant.e4m3fn_decode(v_fp8) * v_s.astype(np.float64)[None, :]
    r.levels_override = levels_override
    r.out_packed = np.full((g.Np, D), np.nan)
    r.l_packed = np.full(g.Np, np.nan)
    return r


def attend(r: HeadResult, q_blocks=None, emulate_p_rounding: bool = True) -> HeadResult:
    ops = _Ops(r)
    blocks = range(r.g.Nb) if q_blocks is None else q_blocks
    for qb in blocks:
        rows, O, l = attention.attend_block(ops, int(qb), emulate_p_rounding)
        r.out_packed[rows] = O
        r.l_packed[rows] = l
        r.computed_blocks.append(int(qb))
    return r


def run_head(q_bits, k_bits, v_bits, *, T, H, W, rh, rw, lam, quota_bp, q_blocks=None,
             emulate_p_rounding: bool = True, levels_override=None,
             fp4_format: str = "mxfp4") -> HeadResult:
    r = prepare_head(q_bits, k_bits, v_bits, T=T, H=H, W=W, rh=rh, rw=rw, lam=lam,
                     quota_bp=quota_bp, levels_override=levels_override, fp4_format=fp4_format)
    return attend(r, q_blocks, emulate_p_rounding)


def run(Q, K, V, *, T, H, W, rh, rw, lam, quota_bp, heads=None, q_blocks=None,
        emulate_p_rounding: bool = True, fp4_format: str = "mxfp4"):
    """Q/K/V: [batch, heads, N, D] bf16 bits.  Returns {(b, h): HeadResult}."""
    out = {}
    Bt, Hh = Q.shape[:2]
    idx = [(b, h) for b in range(Bt) for h in range(Hh)] if heads is None else heads
    for b, h in idx:
        out[(b, h)] = run_head(Q[b, h], K[b, h], V[b, h], T=T, H=H, W=W, rh=rh, rw=rw, lam=lam,
                               quota_bp=quota_bp, q_blocks=q_blocks,
                               emulate_p_rounding=emulate_p_rounding, fp4_format=fp4_format)
    return out
