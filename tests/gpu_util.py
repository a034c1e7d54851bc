"""Helpers for the GPU parity tests: run the HIP path through the C ABI, decode workspace sections
into the oracle's logical layouts, and compare."""
from __future__ import annotations

import sys
import time

import numpy as np

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

REL_L2_TOL = 5e-3
MAX_ABS_TOL = 2e-2
SCORE_RTOL = 1e-12


def log(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_device(Q, K, V):
    import torch
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return t(Q), t(K), t(V)


def run_gpu(cfg: b.Config, q, k, v, check_shapes=True):
    """prepare -> draft_rank -> attention -> restore; returns (ws, out, layout)."""
    import torch
    if check_shapes:
        exp = (cfg.batch, cfg.heads, cfg.N, cfg.head_dim)
        for t in (q, k, v):
            assert tuple(t.shape) == exp and t.dtype == torch.bfloat16 and t.is_contiguous()
    ws = b.alloc_workspace(cfg, q.device)
    out = torch.empty_like(q)
    b.prepare(cfg, q, k, v, ws)
    b.draft_rank(cfg, ws)
    b.attention(cfg, ws)
    b.restore(cfg, ws, out)
    torch.cuda.synchronize()
    return ws, out, b.workspace_layout(cfg)


class Sections:
    """Host copies of workspace sections for one (batch*head) index, in oracle layouts."""

    def __init__(self, ws, L, bhi: int):
        import torch
        self.L = L
        Nb, B, Np, D, kp8 = L["Nb"], L["B"], L["Np"], L["D"], L["kp8"]
        BH = L["bh"]
        sec = lambda name, dt, shape: b.section(ws, L, name, dt, shape)[bhi].cpu().numpy()
        self.q_avg = sec("q_avg", torch.float64, (BH, Nb, D))
        self.q_max = sec("q_max", torch.float64, (BH, Nb, D))
        self.k_avg = sec("k_avg", torch.float64, (BH, Nb, D))
        self.k_max = sec("k_max", torch.float64, (BH, Nb, D))
        self.q_bf16 = sec("q_bf16", torch.int16, (BH, Np, D)).view(np.uint16)
        self.k_bf16 = sec("k_bf16", torch.int16, (BH, Np, D)).view(np.uint16)
        vt16 = sec("vt_bf16", torch.int16, (BH, Nb, D, B)).view(np.uint16)
        self.q_i8 = sec("q_i8", torch.int8, (BH, Np, D))
        self.k_i8 = sec("k_i8", torch.int8, (BH, Np, D))
        self.q_i8_s = sec("q_i8_scale", torch.float32, (BH, Nb))
        self.k_i8_s = sec("k_i8_scale", torch.float32, (BH, Nb))
        qf4 = sec("q_fp4", torch.uint8, (BH, Np, D // 2))
        kf4 = sec("k_fp4", torch.uint8, (BH, Np, D // 2))
        self.q_fp4, self.k_fp4 = unpack_nibbles(qf4), unpack_nibbles(kf4)
        self.q_e8 = sec("q_e8m0", torch.uint8, (BH, Np, D // 32))
        self.k_e8 = sec("k_e8m0", torch.uint8, (BH, Np, D // 32))
        vt8 = sec("vt_fp8", torch.uint8, (BH, Nb, D, kp8))
        self.v_s = sec("v_scale", torch.float32, (BH, D))
        self.scores = sec("scores", torch.float64, (BH, Nb, Nb))
        self.map = sec("map", torch.uint8, (BH, Nb, Nb))
        self.lists = sec("lists", torch.int16, (BH, Nb, Nb)).view(np.uint16)
        self.counts = sec("counts", torch.int32, (BH, Nb, 4))
        self.out_packed = sec("out", torch.int16, (BH, Np, D)).view(np.uint16)
        # NVFP4 sections exist only when the layout gives them room
        self.nv = L["off_q_nv_bf16"] != L["off_k_nv_bf16"]
        if self.nv:
            self.q_nv_s = sec("q_nv_scale", torch.uint8, (BH, Np, D // 16))
            self.k_nv_s = sec("k_nv_scale", torch.uint8, (BH, Np, D // 16))
            self.q_nv_bf16 = sec("q_nv_bf16", torch.int16, (BH, Np, D)).view(np.uint16)
            self.k_nv_bf16 = sec("k_nv_bf16", torch.int16, (BH, Np, D)).view(np.uint16)
            self.nv_t = sec("nv_tscale", torch.float32, (BH, 2))
        # sections of a precision no pair uses are never written: decode only the used ones
        need16 = L["c16"] > 0
        needlow = L["c4"] > L["c16"]
        self.vp_bf16 = unpermute_vt16(vt16, B) if need16 else None
        self.v_fp8 = unpermute_vt8(vt8, B) if needlow else None


def unpack_nibbles(x: np.ndarray) -> np.ndarray:
    lo = x & 0xF
    hi = x >> 4
    return np.stack([lo, hi], axis=-1).reshape(x.shape[:-1] + (x.shape[-1] * 2,))


def unpermute_vt16(vt: np.ndarray, B: int) -> np.ndarray:
    """[Nb][D][B] (16-key chunks stored 0-3, 8-11, 4-7, 12-15) -> packed rows [Nb*B][D]."""
    pos = np.arange(B)
    key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)
    Nb, D = vt.shape[0], vt.shape[1]
    out = np.empty((Nb, B, D), vt.dtype)
    out[:, key, :] = np.transpose(vt, (0, 2, 1))
    return out.reshape(Nb * B, D)


def unpermute_vt8(vt: np.ndarray, B: int) -> np.ndarray:
    """[Nb][D][kp8] (position 32g + 16a + 4b + e holds key 32a + 8b + 4g + e of each 64-key
    chunk) -> packed rows [Nb*B][D]; positions of keys >= B must be zero."""
    kp8 = vt.shape[2]
    pos = np.arange(kp8)
    p = pos % 64
    key = (pos // 64) * 64 + 32 * ((p >> 4) & 1) + 8 * ((p >> 2) & 3) + 4 * ((p >> 5) & 1) + (p & 3)
    Nb, D = vt.shape[0], vt.shape[1]
    full = np.empty((Nb, kp8, D), vt.dtype)
    full[:, key, :] = np.transpose(vt, (0, 2, 1))
    assert not full[:, B:, :].any(), "FP8 V^T positions beyond the block are not zero"
    return full[:, :B, :].reshape(Nb * B, D)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 values that are exactly bf16 -> bit patterns."""
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rel_l2(a, b):
    d = np.linalg.norm((a - b).ravel())
    n = np.linalg.norm(b.ravel())
    return d / n if n > 0 else d


def out_head(out, bhi, heads):
    bb, h = divmod(bhi, heads)
    return synth.bf16_bits_to_f32(out[bb, h].cpu().view(__import__("torch").int16).numpy()
                                  .view(np.uint16)).astype(np.float64)
