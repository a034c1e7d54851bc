"""Pins for the oracle's region geometry, pack and unpack (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import layout
from video_dit_mixed_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_geometry_matches_stated_workload(name):
    w = synth.WORKLOADS[name]
    exp = json.load(open(os.path.join(GOLD, "geometry.json")))["cases"][name]
    g = layout.geometry(w.T, w.H, w.W, w.region_h, w.region_w)
    assert (g.B, g.Nb, g.Hp, g.Wp) == (exp["B"], exp["Nb"], exp["Hp"], exp["Wp"])
    assert g.Np == g.Nb * g.B


def _pack_by_loops(x, T, H, W, rh, rw):
    """Brute force: walk every token with explicit loops and place it."""
    nby, nbx = -(-H // rh), -(-W // rw)
    B = rh * rw
    out = np.zeros((T * nby * nbx * B, x.shape[1]), x.dtype)
    for t in range(T):
        for y in range(H):
            for xx in range(W):
                b = (t * nby + y // rh) * nbx + xx // rw
                p = b * B + (y % rh) * rw + (xx % rw)
                out[p] = x[(t * H + y) * W + xx]
    return out


@pytest.mark.parametrize("shape", [(2, 16, 16, 4, 4), (3, 5, 7, 2, 4), (2, 9, 17, 8, 16), (1, 3, 3, 1, 1)])
def test_pack_matches_loops_and_roundtrips(shape):
    T, H, W, rh, rw = shape
    g = layout.geometry(T, H, W, rh, rw)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((g.N, 3))
    xp = layout.pack(x, g)
    np.testing.assert_array_equal(xp, _pack_by_loops(x, T, H, W, rh, rw))
    np.testing.assert_array_equal(layout.unpack(xp, g), x)
    src = layout.source_index(g)
    real = src[src >= 0]
    assert real.size == g.N and np.unique(real).size == g.N      # bijection onto real slots
    assert np.all(xp[src < 0] == 0)                               # pad rows are zero
    assert layout.valid_rows(g).sum() == g.N


def test_padding_positions_hunyuan_shape():
    # 45 rows in 8-row regions: the last region row keeps 5 real rows, pads are its last 3 rows.
    g = layout.geometry(33, 45, 80, 8, 16)
    v = layout.valid_rows(g)
    last = v[(0 * g.nby + g.nby - 1) * g.nbx].reshape(8, 16)
    assert last[:5].all() and not last[5:].any()
    assert v.sum(axis=1).min() == 80


def test_padding_positions_fewstep_shape():
    # 84 columns in 16-column regions: the last region column keeps 4 real columns.
    g = layout.geometry(91, 48, 84, 8, 16)
    v = layout.valid_rows(g)
    last = v[g.nbx - 1].reshape(8, 16)
    assert last[:, :4].all() and not last[:, 4:].any()
    assert v.sum(axis=1).min() == 32
