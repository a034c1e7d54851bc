"""Thin Python binding of libdap (include/dap.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; torch is used for device memory and the
current stream.  If the library is missing the import-time loader raises -- there is no fallback.

    cfg = Config(batch=1, heads=24, head_dim=128, T=33, H=45, W=80, region_h=8, region_w=16,
                 lam=0.5, quota_bp=(8500, 0, 750, 750))
    out = forward(cfg, q, k, v)            # q, k, v: cuda bf16 [batch, heads, N, D]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, astuple
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdap.so")

DAP_OK, DAP_E_INVALID, DAP_E_UNSUPPORTED, DAP_E_WORKSPACE, DAP_E_HIP, DAP_E_SCRATCH_LIMIT = range(6)
ABI_VERSION = 2
STAGE_PREPARED, STAGE_RANKED, STAGE_ATTENDED, STAGE_BROKEN = (0xDA900001, 0xDA900002, 0xDA900003,
                                                              0xDA9000FF)
FP4_MXFP4, FP4_NVFP4 = 0, 1
LEVEL_SKIP, LEVEL_4, LEVEL_8, LEVEL_16 = 0, 1, 2, 3
EXPORTED = ("dap_abi_version", "dap_workspace_bytes", "dap_workspace_layout", "dap_prepare",
            "dap_prepare_static_scratch", "dap_draft_rank", "dap_attention",
            "dap_attention_section_clocks", "dap_restore", "dap_status_string")
# dap_attention_section_clocks: counters per phase (16-bit, 8-bit, MXFP4, NVFP4), in this order
SECTION_CLOCK_PARTS = ("wait_k", "barrier_1", "qk_and_statistics", "wait_v", "barrier_2", "pv")
SECTION_CLOCK_WORDS = 32


class DapError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("region_h", ctypes.c_int32), ("region_w", ctypes.c_int32),
                ("lam", ctypes.c_double), ("quota_bp", ctypes.c_int32 * 4),
                ("fp4_format", ctypes.c_int32)]


_LAYOUT_INT32 = ["Hp", "Wp", "nby", "nbx", "Nb", "B", "Np", "kp8", "bh", "D"]
_LAYOUT_INT64 = ["pairs", "c16", "c8", "c4"]
_LAYOUT_OFFS = ["q_bf16", "k_bf16", "vt_bf16", "q_i8", "k_i8", "q_i8_scale", "k_i8_scale",
                "q_fp4", "k_fp4", "q_e8m0", "k_e8m0", "vt_fp8", "v_scale", "v_amax",
                "q_avg", "q_max", "k_avg", "k_max", "scores", "lmax", "rank_state", "rank_hist",
                "map", "lists", "counts", "out", "zeros", "order", "stage", "q_nv_scale",
                "k_nv_scale", "q_nv_bf16", "k_nv_bf16", "nv_tscale", "qk_amax"]


class _Layout(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int32) for n in _LAYOUT_INT32] +
                [(n, ctypes.c_int64) for n in _LAYOUT_INT64] +
                [("off_" + n, ctypes.c_uint64) for n in _LAYOUT_OFFS] +
                [("total_bytes", ctypes.c_uint64)])


@dataclass(frozen=True)
class Config:
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    region_h: int
    region_w: int
    lam: float
    quota_bp: Tuple[int, int, int, int]   # skip, 4-bit, 8-bit, 16-bit (basis points)
    fp4_format: int = FP4_MXFP4

    @classmethod
    def from_workload(cls, w, **override) -> "Config":
        kw = dict(batch=w.batch, heads=w.heads, head_dim=w.head_dim, T=w.T, H=w.H, W=w.W,
                  region_h=w.region_h, region_w=w.region_w, lam=w.lam, quota_bp=tuple(w.quota_bp),
                  fp4_format=FP4_NVFP4 if getattr(w, "fp4", "mxfp4") == "nvfp4" else FP4_MXFP4)
        kw.update(override)
        return cls(**kw)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    def c_struct(self) -> _Config:
        c = _Config()
        c.batch, c.heads, c.head_dim = self.batch, self.heads, self.head_dim
        c.T, c.H, c.W = self.T, self.H, self.W
        c.region_h, c.region_w = self.region_h, self.region_w
        c.lam = float(self.lam)
        for i, q in enumerate(self.quota_bp):
            c.quota_bp[i] = int(q)
        c.fp4_format = int(self.fp4_format)
        return c


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdap.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m video_dit_mixed_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.dap_abi_version.restype = ctypes.c_size_t
    lib.dap_abi_version.argtypes = []
    lib.dap_workspace_bytes.restype = ctypes.c_int
    lib.dap_workspace_bytes.argtypes = [P(_Config), P(ctypes.c_size_t)]
    lib.dap_workspace_layout.restype = ctypes.c_int
    lib.dap_workspace_layout.argtypes = [P(_Config), P(_Layout)]
    vp = ctypes.c_void_p
    lib.dap_prepare.restype = ctypes.c_int
    lib.dap_prepare.argtypes = [P(_Config), vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.dap_prepare_static_scratch.restype = ctypes.c_int
    lib.dap_prepare_static_scratch.argtypes = [P(_Config), vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.dap_draft_rank.restype = ctypes.c_int
    lib.dap_draft_rank.argtypes = [P(_Config), vp, ctypes.c_size_t, vp, vp, vp]
    lib.dap_attention.restype = ctypes.c_int
    lib.dap_attention.argtypes = [P(_Config), vp, ctypes.c_size_t, vp]
    lib.dap_attention_section_clocks.restype = ctypes.c_int
    lib.dap_attention_section_clocks.argtypes = [P(_Config), vp, ctypes.c_size_t, vp, vp]
    lib.dap_restore.restype = ctypes.c_int
    lib.dap_restore.argtypes = [P(_Config), vp, ctypes.c_size_t, vp, vp]
    lib.dap_status_string.restype = ctypes.c_char_p
    lib.dap_status_string.argtypes = [ctypes.c_int]
    if lib.dap_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {lib.dap_abi_version()}, this binding speaks "
                           f"{ABI_VERSION}: rebuild with `python -m video_dit_mixed_amd.build`")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dap_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != DAP_OK:
        raise DapError(status, where)


def abi_version() -> int:
    return int(load().dap_abi_version())


def workspace_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c_struct()
    _check(load().dap_workspace_bytes(ctypes.byref(c), ctypes.byref(n)), "dap_workspace_bytes")
    return int(n.value)


def workspace_layout(cfg: Config) -> dict:
    L = _Layout()
    c = cfg.c_struct()
    _check(load().dap_workspace_layout(ctypes.byref(c), ctypes.byref(L)), "dap_workspace_layout")
    return {name: getattr(L, name) for name, _ in _Layout._fields_}


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def _prod(xs) -> int:
    n = 1
    for x in xs:
        n *= int(x)
    return n


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _expect(t, name: str, dtype: str, shape=None, min_bytes: int = 0):
    """Host-side check of a torch tensor handed to the library as a bare pointer: the kernels
    assume a contiguous device buffer of exactly this element type and size.  Integers (raw device
    pointers) are passed through unchecked, as the C ABI takes them."""
    if t is None or not hasattr(t, "data_ptr"):
        return
    import torch
    want = getattr(torch, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype != "uint8" and t.dtype != want:
        raise ValueError(f"{name}: expected dtype {want}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_bytes and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: expected at least {min_bytes} bytes")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor, got device {t.device}")


def _io_shape(cfg: Config):
    return (cfg.batch, cfg.heads, cfg.N, cfg.head_dim)


def _pairs_shape(cfg: Config):
    nb = cfg.T * -(-cfg.H // cfg.region_h) * -(-cfg.W // cfg.region_w)
    return (cfg.batch * cfg.heads, nb, nb)


def prepare(cfg: Config, q, k, v, ws, stream=None):
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, "bfloat16", _io_shape(cfg))
    _expect(ws, "ws", "uint8")
    c = cfg.c_struct()
    _check(load().dap_prepare(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(ws), _nbytes(ws),
                              _stream(stream)), "dap_prepare")


def prepare_static_scratch(cfg: Config, q, k, v, ws, stream=None):
    """dap_prepare with its scratch in the library's static device array (no allocation)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, "bfloat16", _io_shape(cfg))
    _expect(ws, "ws", "uint8")
    c = cfg.c_struct()
    _check(load().dap_prepare_static_scratch(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(ws),
                                             _nbytes(ws), _stream(stream)),
           "dap_prepare_static_scratch")


def draft_rank(cfg: Config, ws, map_out=None, scores_out=None, stream=None):
    _expect(map_out, "map_out", "uint8", min_bytes=_prod(_pairs_shape(cfg)))
    _expect(scores_out, "scores_out", "float64", _pairs_shape(cfg))
    _expect(ws, "ws", "uint8")
    c = cfg.c_struct()
    _check(load().dap_draft_rank(ctypes.byref(c), _ptr(ws), _nbytes(ws), _ptr(map_out),
                                 _ptr(scores_out), _stream(stream)), "dap_draft_rank")


def attention(cfg: Config, ws, stream=None):
    _expect(ws, "ws", "uint8")
    c = cfg.c_struct()
    _check(load().dap_attention(ctypes.byref(c), _ptr(ws), _nbytes(ws), _stream(stream)),
           "dap_attention")


def attention_section_clocks(cfg: Config, ws, clocks, stream=None):
    """dap_attention with the kernel's shader-clock counters added into `clocks` (a zeroed int64
    device tensor of SECTION_CLOCK_WORDS; word 8 p + i is part i of phase p, word 8 p + 6 the
    wave-blocks of phase p, word 7 the summed wave lifetimes)."""
    _expect(ws, "ws", "uint8")
    _expect(clocks, "clocks", "int64", (SECTION_CLOCK_WORDS,))
    c = cfg.c_struct()
    _check(load().dap_attention_section_clocks(ctypes.byref(c), _ptr(ws), _nbytes(ws), _ptr(clocks),
                                               _stream(stream)), "dap_attention_section_clocks")


def restore(cfg: Config, ws, out, stream=None):
    _expect(out, "out", "bfloat16", _io_shape(cfg))
    _expect(ws, "ws", "uint8")
    c = cfg.c_struct()
    _check(load().dap_restore(ctypes.byref(c), _ptr(ws), _nbytes(ws), _ptr(out), _stream(stream)),
           "dap_restore")


def alloc_workspace(cfg: Config, device="cuda"):
    import torch
    return torch.empty(workspace_bytes(cfg), dtype=torch.uint8, device=device)


def forward(cfg: Config, q, k, v, ws=None, out=None, stream=None):
    """One layer: prepare -> draft_rank -> attention -> restore.  Returns (out, ws)."""
    import torch
    if ws is None:
        ws = alloc_workspace(cfg, q.device)
    if out is None:
        out = torch.empty_like(q)
    prepare(cfg, q, k, v, ws, stream)
    draft_rank(cfg, ws, stream=stream)
    attention(cfg, ws, stream)
    restore(cfg, ws, out, stream)
    return out, ws


def stage_words(ws, layout: dict):
    """(stage word, configuration tag) of a workspace, read back to the host (synchronises)."""
    import torch
    st = section(ws, layout, "stage", torch.int32, (2,)).cpu().numpy().view("uint32")
    return int(st[0]), int(st[1])


def section(ws, layout: dict, name: str, dtype, shape):
    """View of one workspace section (torch tensor sharing the workspace memory)."""
    import torch
    off = int(layout["off_" + name])
    itemsize = torch.empty(0, dtype=dtype).element_size()
    count = 1
    for s in shape:
        count *= int(s)
    return ws[off: off + count * itemsize].view(dtype).view(*shape)
