"""Worker processes for oracle work that a single process would take minutes over (one full-size
head over every query block).  The pool is forked while the test session is being set up, before
any test touches the GPU, so the workers are plain CPU processes; each runs numpy with one BLAS
thread.  Test infrastructure only."""
from __future__ import annotations

import multiprocessing as mp

import numpy as np

_pool = None
WORKERS = 8


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def start(n: int = WORKERS):
    global _pool
    if _pool is None:
        _pool = mp.get_context("fork").Pool(n, initializer=_init)


def stop():
    global _pool
    if _pool is not None:
        _pool.terminate()
        _pool.join()
        _pool = None


def get():
    return _pool


def _attend_blocks(args):
    """One worker's share: the oracle's steps up to attention for one head, then attention over
    the given query blocks.  Returns (packed rows, fp64 outputs of those rows)."""
    from oracle import pipeline as opipe
    q, k, v, geo, blocks = args
    r = opipe.prepare_head(q, k, v, **geo)  # geo may carry fp4_format
    opipe.attend(r, q_blocks=blocks)
    rows = np.concatenate([qb * r.B + np.flatnonzero(r.valid[qb]) for qb in blocks])
    return rows, r.out_packed[rows]


def attend_head(q, k, v, geo: dict, blocks):
    """Oracle outputs (packed rows, values) of `blocks` of one head, split over the pool (or in
    this process when no pool was started)."""
    blocks = [int(x) for x in blocks]
    if _pool is None:
        return _attend_blocks((q, k, v, geo, blocks))
    n = len(_pool._pool)
    parts = [list(p) for p in np.array_split(np.asarray(blocks), n) if len(p)]
    res = _pool.map(_attend_blocks, [(q, k, v, geo, p) for p in parts])
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
