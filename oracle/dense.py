"""Exact dense softmax attention over all tokens, in fp64.  Oracle: test infrastructure only.

This is the quantity the draft-guided sparse mixed-precision operator approximates: the pages
measure their operator by its relative L2 output error against full attention at a given latency
(pchao.org blog on DraftAttention2, Figure 1 caption, panel (b), and the first item of the section
关键结果与论文证据).  O = softmax(Q K^T / sqrt(D)) V over every key token, with the bf16 inputs
taken exactly and no rounding anywhere.  It is evaluated for a chosen set of query rows so that a
full-size layer can be sampled on the CPU.
"""
from __future__ import annotations

import numpy as np

from .pipeline import bf16_bits_to_f64


def dense_attention_rows(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                         rows=None, chunk: int = 256) -> np.ndarray:
    """Rows `rows` (token indices; all when None) of softmax(Q K^T / sqrt(D)) V, fp64 [len, D].
    q_bits, k_bits, v_bits: [N, D] uint16 bf16 bit patterns of one (batch, head)."""
    N, D = k_bits.shape
    rows = np.arange(q_bits.shape[0]) if rows is None else np.asarray(rows)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    out = np.empty((len(rows), D), np.float64)
    for s in range(0, len(rows), chunk):
        q = bf16_bits_to_f64(q_bits[rows[s:s + chunk]])
        logits = (q @ k.T) / np.sqrt(float(D))
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[s:s + chunk] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out
