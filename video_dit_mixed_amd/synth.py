"""Seeded synthetic video-token workloads for draft-guided mixed-precision attention.

This module only draws random numbers and names workloads. It contains none of the method's
arithmetic (no packing, pooling, ranking, quantisation or attention), so the CPU oracle and the HIP
path can both be fed from it without sharing any method code.

Workloads (latent grid T x H x W, heads, head_dim, region rh x rw, lambda, quotas in basis points
for skip / 4-bit / 8-bit / 16-bit) follow the layer shapes of the experiments on
"DraftAttention2: Fast Video Diffusion with Low-Resolution-Guided Mixed-Precision Attention"
(pchao.org blog, sections "实验如何设计？" and "关键结果与论文证据": HunyuanVideo Table 1 quota mixes
85/0/7.5/7.5 and 80.7/14.4/4.8/0, and the few-step 1344x768, 362-frame MiniMax-H3 setting).

Field recipe per (batch*head, tensor):
  * coordinates t^ = t/(T-1), y^ = y/(H-1), x^ = x/(W-1) (0 when the axis has length 1);
  * Q and K: 8 Gaussian blobs, centre ~ U[0,1]^3, per-axis sigma ~ U[0.05,0.25],
    amplitude ~ N(0,1)^D; field = sum_b a_b exp(-1/2 sum_axis ((coord-c)/sigma)^2) + 0.3 N(0,1);
    4 outlier channels (shared by Q and K of a head) are then scaled by 8;
  * V ~ N(0,1);
  * fp32 -> bf16 round-to-nearest-even; layout [batch, heads, N, D], token n = (t*H + y)*W + x.
Random streams: numpy PCG64 seeded with [seed, batch*heads index, tensor id] where tensor id is
Q=0, K=1, V=2, outlier-channel choice=99.  The default seed of workload c (1-based) is 1000 + c.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_head", "make_inputs", "bf16_bits_to_f32",
           "f32_to_bf16_bits"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    region_h: int
    region_w: int
    lam: float
    # basis points (1/100 %) for skip, 4-bit, 8-bit, 16-bit; skip is informational (remainder)
    quota_bp: Tuple[int, int, int, int]
    batch: int = 1
    seed: int = 0
    fp4: str = "mxfp4"   # 4-bit operand format of the workload: "mxfp4" or "nvfp4"

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny CPU-seconds case: 2x16x16 latent, 4x4 regions (16-token blocks)
    "tiny_2x16x16": Workload("tiny_2x16x16", 2, 16, 16, 2, 64, 4, 4, 0.5, (2500, 2500, 2500, 2500),
                             seed=1001),
    # mid case: 8x24x40 latent, 8x8 regions (64-token blocks)
    "mid_8x24x40": Workload("mid_8x24x40", 8, 24, 40, 12, 64, 8, 8, 0.5, (3000, 2000, 2000, 3000),
                            seed=1002),
    # HunyuanVideo-shaped 720p layer, 85/0/7.5/7.5 mix
    "hunyuan720p_33x45x80": Workload("hunyuan720p_33x45x80", 33, 45, 80, 24, 128, 8, 16, 0.5,
                                     (8500, 0, 750, 750), seed=1003),
    # same shape, 4-bit-heavy mix 80.7/14.4/4.8/0 (printed values sum to 99.9 %)
    "hunyuan720p_4bit_33x45x80": Workload("hunyuan720p_4bit_33x45x80", 33, 45, 80, 24, 128, 8, 16,
                                          0.5, (8070, 1440, 480, 0), seed=1004),
    # few-step long video 1344x768, 362 frames -> 91x48x84 latent, 75/15/10/0
    "fewstep_91x48x84": Workload("fewstep_91x48x84", 91, 48, 84, 24, 128, 8, 16, 0.5,
                                 (7500, 1500, 1000, 0), seed=1005),
}
ORDER = list(WORKLOADS)


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _coords(w: Workload) -> np.ndarray:
    def ax(n):
        return np.arange(n, dtype=np.float64) / (n - 1) if n > 1 else np.zeros(n)
    t, y, x = np.meshgrid(ax(w.T), ax(w.H), ax(w.W), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)  # [N, 3], n = (t*H+y)*W+x


def _blob_field(rng: np.random.Generator, coords: np.ndarray, D: int) -> np.ndarray:
    centre = rng.uniform(0.0, 1.0, size=(8, 3))
    sigma = rng.uniform(0.05, 0.25, size=(8, 3))
    amp = rng.standard_normal(size=(8, D))
    z = (coords[:, None, :] - centre[None, :, :]) / sigma[None, :, :]   # [N, 8, 3]
    env = np.exp(-0.5 * np.sum(z * z, axis=2))                          # [N, 8]
    f = env @ amp                                                       # [N, D] fp64
    f += 0.3 * rng.standard_normal(size=f.shape, dtype=np.float32)
    return f


def make_head(w: Workload, bh: int, coords: np.ndarray | None = None):
    """bf16 bit patterns (uint16) of Q, K, V for one (batch*head) index, each [N, D]."""
    if coords is None:
        coords = _coords(w)
    D = w.head_dim
    seed = w.seed
    q = _blob_field(np.random.default_rng([seed, bh, 0]), coords, D)
    k = _blob_field(np.random.default_rng([seed, bh, 1]), coords, D)
    ch = np.random.default_rng([seed, bh, 99]).choice(D, 4, replace=False)
    q[:, ch] *= 8.0
    k[:, ch] *= 8.0
    v = np.random.default_rng([seed, bh, 2]).standard_normal(size=(w.N, D), dtype=np.float32)
    return (f32_to_bf16_bits(q.astype(np.float32)), f32_to_bf16_bits(k.astype(np.float32)),
            f32_to_bf16_bits(v))


def make_inputs(w: Workload, heads=None, threads: int = 8):
    """Full [batch, heads, N, D] uint16 (bf16 bits) Q, K, V.  `heads` restricts which
    batch*head indices are filled (others stay zero) for partial CPU work."""
    from concurrent.futures import ThreadPoolExecutor
    BH = w.batch * w.heads
    shape = (w.batch, w.heads, w.N, w.head_dim)
    Q = np.zeros(shape, np.uint16)
    K = np.zeros(shape, np.uint16)
    V = np.zeros(shape, np.uint16)
    coords = _coords(w)
    idx = list(range(BH)) if heads is None else list(heads)

    def one(bh):
        q, k, v = make_head(w, bh, coords)
        b, h = divmod(bh, w.heads)
        Q[b, h], K[b, h], V[b, h] = q, k, v

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, idx))
    return Q, K, V
