"""Region geometry, pack (reorder + pad) and unpack (restore).  Oracle: test infrastructure only.

Follows: pchao.org blog on DraftAttention2, Figure 3(a) caption (each spatial region of a frame
becomes one run of consecutive rows, with pad cells where the frame does not fill the region) and
section 方法概览 bullet 1 (the per-frame spatial regions); pith.science DraftAttention abstract
(the token order is changed before attention and changed back after it).

Readings (the pages are silent on these):
  R1  inputs are [batch, heads, N, D]; token n = (t*H + y)*W + x.
  R3  a region is rh rows (height) by rw columns (width) of one frame.
  R4  padding goes at high y / high x of each frame, pad values are 0, and a pad slot keeps its
      in-region raster position.
  R5  blocks are ordered region-raster (t, ry, rx); inside a block rows are (iy, ix) raster.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Geometry:
    T: int
    H: int
    W: int
    rh: int
    rw: int
    Hp: int
    Wp: int
    nby: int
    nbx: int
    Nb: int
    B: int
    Np: int

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


def geometry(T: int, H: int, W: int, rh: int, rw: int) -> Geometry:
    nby = -(-H // rh)
    nbx = -(-W // rw)
    Nb = T * nby * nbx
    B = rh * rw
    return Geometry(T, H, W, rh, rw, nby * rh, nbx * rw, nby, nbx, Nb, B, Nb * B)


def source_index(g: Geometry) -> np.ndarray:
    """For each packed row p in [0, Np): the source token n, or -1 for a pad slot."""
    p = np.arange(g.Np, dtype=np.int64)
    b, i = np.divmod(p, g.B)
    iy, ix = np.divmod(i, g.rw)
    t, rem = np.divmod(b, g.nby * g.nbx)
    ry, rx = np.divmod(rem, g.nbx)
    y = ry * g.rh + iy
    x = rx * g.rw + ix
    valid = (y < g.H) & (x < g.W)
    n = (t * g.H + y) * g.W + x
    return np.where(valid, n, -1)


def pack(x: np.ndarray, g: Geometry) -> np.ndarray:
    """[..., N, D] -> [..., Np, D]; pad rows are 0."""
    src = source_index(g)
    out = np.zeros(x.shape[:-2] + (g.Np, x.shape[-1]), dtype=x.dtype)
    ok = src >= 0
    out[..., ok, :] = x[..., src[ok], :]
    return out


def unpack(xp: np.ndarray, g: Geometry) -> np.ndarray:
    """Inverse of pack on real tokens: [..., Np, D] -> [..., N, D]; pad rows are dropped."""
    src = source_index(g)
    ok = src >= 0
    out = np.empty(xp.shape[:-2] + (g.N, xp.shape[-1]), dtype=xp.dtype)
    out[..., src[ok], :] = xp[..., ok, :]
    return out


def valid_rows(g: Geometry) -> np.ndarray:
    """[Nb, B] bool: which packed rows of each block hold a real token."""
    return (source_index(g) >= 0).reshape(g.Nb, g.B)
