"""Phased mixed-precision block-sparse attention with shared online-softmax state.
Oracle: test infrastructure only.

Follows: newx.sg paper card, Abstract, and pchao.org blog, section 方法概览 (overview paragraph and
bullet 4): a query row's kept blocks of every precision update one running maximum, one running
sum and one output accumulator, with the quantisation scales applied where the precision changes,
instead of one partial result per precision merged afterwards.

Per query block qb, over its real query rows, with running max m = -inf, sum l = 0, output O = 0:
  for phase in (16-bit, 8-bit, 4-bit), for each key block kb of that level in ascending order:
    S  = 16-bit: Q_bf16 K_bf16^T / sqrt(D)
          8-bit: (q_codes . k_codes) * s_q * s_k / sqrt(D)
          4-bit: (dequantised 4-bit Q . dequantised 4-bit K) / sqrt(D), MXFP4 or NVFP4
    pad keys of kb get -inf
    m' = max(m, rowmax S); alpha = exp(m - m'); P = exp(S - m'); l = alpha*l + rowsum P
    16-bit: O = alpha*O + bf16(P) V_bf16
    low-bit: O = alpha*O + (e4m3(2^8 P) 2^-8) (V_fp8 * s_V)
    m = m'
  O = O / l where l > 0, else 0.

Readings:
  R15 a query block whose pairs are all skipped outputs 0.
  R18 P.V is bf16 on 16-bit blocks and FP8 e4m3 on 8- and 4-bit blocks.
  R19 P is scaled by the exact power of two 2^8 before the e4m3 rounding.
  R21 l sums the unrounded P.
  R22 one running-max update per key block, phases 16 -> 8 -> 4, ascending kb inside a phase.
  R23 pad keys are masked to -inf; pad query rows are not computed (they are dropped on restore).
  R24 softmax scale 1/sqrt(D).
`emulate_p_rounding=False` drops the bf16 / e4m3 rounding of P (used by the exact invariants).
"""
from __future__ import annotations

import numpy as np

from . import quant
from .draft import LEVEL_16, LEVEL_8, LEVEL_4

PHASES = (LEVEL_16, LEVEL_8, LEVEL_4)
P_SCALE = 2.0 ** 8


def block_scores(ops, level: int, qb: int, kb: int, rows: np.ndarray) -> np.ndarray:
    """S for the real query rows `rows` (packed row indices) of qb against all B keys of kb."""
    B, D = ops.B, ops.D
    ks = slice(kb * B, (kb + 1) * B)
    if level == LEVEL_16:
        return (ops.qp[rows] @ ops.kp[ks].T) / np.sqrt(float(D))
    if level == LEVEL_8:
        s_int = ops.q_i8[rows].astype(np.int64) @ ops.k_i8[ks].astype(np.int64).T
        return s_int.astype(np.float64) * float(ops.q_i8_s[qb]) * float(ops.k_i8_s[kb]) \
            / np.sqrt(float(D))
    if level == LEVEL_4:
        return (ops.q_fp4_val[rows] @ ops.k_fp4_val[ks].T) / np.sqrt(float(D))
    raise ValueError(level)


def attend_block(ops, qb: int, emulate_p_rounding: bool = True, phase_order=PHASES,
                 kb_order=None) -> tuple:
    """Output rows (fp64, before the final bf16 rounding) of the real query rows of block qb.
    Returns (rows, O, l).  `phase_order` / `kb_order` exist for the order-invariance tests."""
    B, D = ops.B, ops.D
    rows = qb * B + np.flatnonzero(ops.valid[qb])
    nq = rows.size
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    O = np.zeros((nq, D))
    for level in phase_order:
        kbs = np.flatnonzero(ops.levels[qb] == level)
        if kb_order is not None:
            kbs = kb_order(kbs)
        for kb in kbs:
            S = block_scores(ops, level, qb, int(kb), rows)
            S[:, ~ops.valid[kb]] = -np.inf
            m_new = np.maximum(m, S.max(axis=1))
            alpha = np.exp(m - m_new)
            P = np.exp(S - m_new[:, None])
            l = alpha * l + P.sum(axis=1)
            ks = slice(kb * B, (kb + 1) * B)
            if level == LEVEL_16:
                Pq = quant.bf16_rne(P) if emulate_p_rounding else P
                O = alpha[:, None] * O + Pq @ ops.vp[ks]
            else:
                Pq = quant.e4m3fn_rne_sat(P_SCALE * P) / P_SCALE if emulate_p_rounding else P
                O = alpha[:, None] * O + Pq @ ops.v_fp8_val[ks]
            m = m_new
    safe = np.where(l > 0, l, 1.0)
    O = np.where((l > 0)[:, None], O / safe[:, None], 0.0)
    return rows, O, l
