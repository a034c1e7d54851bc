"""Pooling, draft attention maps, lambda mix, per-head ranking and quota assignment.
Oracle: test infrastructure only.

Follows:
  * pooling -- newx.sg paper card, Abstract (the draft is computed from queries and keys pooled
    over 2D spatial regions, by mean and by maximum); pchao.org blog, section 方法概览 bullet 1
    (one mean descriptor and one per-channel maximum descriptor per region);
  * draft maps and mix -- same bullet (an Avg draft map and a Max draft map are formed, then mixed
    with weight lambda; lambda = 0 falls back to average-only guidance as in DraftAttention v1);
    Figure 2 caption (weighted mixture of the pooled draft maps guides block selection);
  * ranking and assignment -- section 方法概览 bullet 2 (within each head all region pairs are
    sorted by draft score and, by quota, given 16-bit, then INT8, then 4-bit; the rest are
    skipped; query regions may end up with different counts); newx.sg AI Summary (a shared
    sorting mechanism); section 实验如何设计？ (the Bit column gives 0/4/8/16 percentages).

Readings:
  R6  the average divides by the number of real (non-pad) tokens of the region.
  R7  the max is the per-channel signed maximum over the region's real tokens.
  R8  draft logits use the attention scale 1/sqrt(D).
  R9  softmax runs over key regions, per query region.
  R10 A = (1 - lambda) * softmax(L_avg) + lambda * softmax(L_max).
  R11 ranking is per (batch, head) over all Nb^2 pairs.
  R12 quotas are percentages (basis points here) of the Nb^2 pairs of a head.
  R13 cut ranks are cumulative from the top with round-half-up in integer arithmetic;
      the skip share is whatever remains.
  R14 total order: A descending, then pair index qb*Nb + kb ascending.
Level encoding: 0 = skip, 1 = 4-bit, 2 = 8-bit, 3 = 16-bit.
"""
from __future__ import annotations

import numpy as np

LEVEL_SKIP, LEVEL_4, LEVEL_8, LEVEL_16 = 0, 1, 2, 3


def pool(xp: np.ndarray, valid: np.ndarray):
    """Avg and max descriptors per block.  xp: packed [Nb*B, D] fp64 (pads 0); valid: [Nb, B].
    Returns (avg [Nb, D], max [Nb, D])."""
    Nb, B = valid.shape
    x = xp.reshape(Nb, B, -1)
    n = valid.sum(axis=1).astype(np.float64)
    s = np.where(valid[:, :, None], x, 0.0).sum(axis=1)
    avg = s / n[:, None]
    mx = np.where(valid[:, :, None], x, -np.inf).max(axis=1)
    return avg, mx


def softmax_rows(L: np.ndarray) -> np.ndarray:
    e = np.exp(L - L.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def draft_logits(qbar: np.ndarray, kbar: np.ndarray, D: int) -> np.ndarray:
    return (qbar @ kbar.T) / np.sqrt(float(D))


def draft_map(q_avg, q_max, k_avg, k_max, lam: float, D: int):
    """Mixed draft map A [Nb, Nb] and its two components."""
    a_avg = softmax_rows(draft_logits(q_avg, k_avg, D))
    a_max = softmax_rows(draft_logits(q_max, k_max, D))
    return (1.0 - lam) * a_avg + lam * a_max, a_avg, a_max


def cut_ranks(P: int, quota_bp) -> tuple:
    """(c16, c8, c4): number of top-ranked pairs at 16-bit, at >= 8-bit, at >= 4-bit.
    quota_bp = (skip, q4, q8, q16) in basis points; skip is the remainder."""
    _, q4, q8, q16 = (int(v) for v in quota_bp)

    def rnd(x):
        return (P * x + 5000) // 10000

    return rnd(q16), rnd(q16 + q8), rnd(q16 + q8 + q4)


def rank_pairs(A: np.ndarray) -> np.ndarray:
    """Rank of every pair (flattened qb*Nb + kb) in the total order (A desc, index asc)."""
    flat = A.ravel()
    idx = np.arange(flat.size, dtype=np.int64)
    order = np.lexsort((idx, -flat))
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = idx
    return rank.reshape(A.shape)


def assign_levels(rank: np.ndarray, cuts) -> np.ndarray:
    c16, c8, c4 = cuts
    lv = np.zeros(rank.shape, np.uint8)
    lv[rank < c4] = LEVEL_4
    lv[rank < c8] = LEVEL_8
    lv[rank < c16] = LEVEL_16
    return lv

