"""C-ABI checks that need no GPU: the library loads, exports every symbol the header declares,
validates arguments before any HIP call, and its workspace layout matches a re-derivation."""
import ctypes
import os
import re
import subprocess

import pytest

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dap.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dap_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(b.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = b.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dap_\w+)", out))
    assert set(_declared()) <= exported


def test_abi_version_and_status_strings():
    assert b.abi_version() == 2
    assert b.status_string(0) == "ok"
    assert "workspace" in b.status_string(3)


def _cfg(**kw):
    return b.Config.from_workload(synth.workload(0), **kw)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), b.DAP_E_UNSUPPORTED),
    (dict(region_h=3, region_w=3), b.DAP_E_UNSUPPORTED),
    (dict(lam=1.5), b.DAP_E_INVALID),
    (dict(lam=-0.1), b.DAP_E_INVALID),
    (dict(lam=float("nan")), b.DAP_E_INVALID),
    (dict(quota_bp=(5000, 3000, 2000, 1000)), b.DAP_E_INVALID),
    (dict(quota_bp=(0, -1, 0, 100)), b.DAP_E_INVALID),
    (dict(batch=0), b.DAP_E_INVALID),
    (dict(T=0), b.DAP_E_INVALID),
    (dict(T=200, H=48, W=96, region_h=8, region_w=16), b.DAP_E_UNSUPPORTED),   # > 4096 regions
    # extreme grids: rejected, with no 32-bit overflow on the way (H + region_h - 1, T * nby * nbx)
    (dict(T=1, H=2**31 - 1, W=16, region_h=8, region_w=16), b.DAP_E_UNSUPPORTED),
    (dict(T=2**31 - 1, H=2**31 - 1, W=2**31 - 1, region_h=8, region_w=16), b.DAP_E_UNSUPPORTED),
    (dict(T=4097, H=8, W=16, region_h=8, region_w=16), b.DAP_E_UNSUPPORTED),
    (dict(fp4_format=2), b.DAP_E_INVALID),
    (dict(fp4_format=-1), b.DAP_E_INVALID),
])
def test_validation_rejects(kw, status):
    with pytest.raises(b.DapError) as e:
        b.workspace_bytes(_cfg(**kw))
    assert e.value.status == status


def test_calls_validate_before_touching_the_device():
    """Null / misaligned pointers and short workspaces are refused on the host (no HIP call)."""
    lib = b.load()
    cfg = _cfg()
    c = cfg.c_struct()
    need = b.workspace_bytes(cfg)
    P = ctypes.byref
    assert lib.dap_prepare(P(c), None, None, None, None, need, None) == b.DAP_E_INVALID
    assert lib.dap_prepare(None, 256, 256, 256, 256, need, None) == b.DAP_E_INVALID
    assert lib.dap_prepare(P(c), 256, 256, 256, 256, need - 1, None) == b.DAP_E_WORKSPACE
    assert lib.dap_prepare(P(c), 256, 256, 257, 256, need, None) == b.DAP_E_INVALID
    assert lib.dap_draft_rank(P(c), 256, need - 1, None, None, None) == b.DAP_E_WORKSPACE
    assert lib.dap_draft_rank(P(c), 256, need, 3, None, None) == b.DAP_E_INVALID
    assert lib.dap_attention(P(c), 100, need, None) == b.DAP_E_INVALID
    assert lib.dap_restore(P(c), 256, need, None, None) == b.DAP_E_INVALID
    bad = _cfg(head_dim=32).c_struct()
    assert lib.dap_attention(P(bad), 256, need, None) == b.DAP_E_UNSUPPORTED
    assert lib.dap_prepare_static_scratch(P(c), None, 256, 256, 256, need, None) == b.DAP_E_INVALID
    assert lib.dap_prepare_static_scratch(P(c), 256, 256, 256, 256, need - 1, None) == b.DAP_E_WORKSPACE
    # the section-clock diagnostic: the workspace checks of dap_attention, then its counter buffer
    assert lib.dap_attention_section_clocks(P(c), 256, need - 1, 256, None) == b.DAP_E_WORKSPACE
    assert lib.dap_attention_section_clocks(P(c), 256, need, None, None) == b.DAP_E_INVALID
    assert lib.dap_attention_section_clocks(P(c), 256, need, 260, None) == b.DAP_E_INVALID
    assert lib.dap_attention_section_clocks(P(bad), 256, need, 256, None) == b.DAP_E_UNSUPPORTED


def test_static_scratch_limit_is_checked_on_the_host():
    """batch * heads * head_dim above the static array (65536 words) is refused before any HIP call."""
    lib = b.load()
    cfg = b.Config(batch=1, heads=513, head_dim=128, T=1, H=8, W=16, region_h=8, region_w=16,
                   lam=0.5, quota_bp=(0, 0, 0, 10000))
    c = cfg.c_struct()
    need = b.workspace_bytes(cfg)
    assert lib.dap_prepare_static_scratch(ctypes.byref(c), 256, 256, 256, 256, need, None) == \
        b.DAP_E_SCRATCH_LIMIT
    assert "static scratch" in b.status_string(b.DAP_E_SCRATCH_LIMIT)


def _layout_py(w):
    """Independent re-derivation of the documented workspace layout."""
    al = lambda x: (x + 255) // 256 * 256
    nby, nbx = -(-w.H // w.region_h), -(-w.W // w.region_w)
    Nb = w.T * nby * nbx
    B = w.region_h * w.region_w
    Np, D, bh = Nb * B, w.head_dim, w.batch * w.heads
    kp8 = -(-B // 64) * 64
    sizes = [("q_bf16", bh * Np * D * 2), ("k_bf16", bh * Np * D * 2), ("vt_bf16", bh * Np * D * 2),
             ("q_i8", bh * Np * D), ("k_i8", bh * Np * D), ("q_i8_scale", bh * Nb * 4),
             ("k_i8_scale", bh * Nb * 4), ("q_fp4", bh * Np * D // 2), ("k_fp4", bh * Np * D // 2),
             ("q_e8m0", bh * Np * D // 32), ("k_e8m0", bh * Np * D // 32),
             ("vt_fp8", bh * Nb * D * kp8), ("v_scale", bh * D * 4), ("v_amax", bh * D * 4),
             ("q_avg", bh * Nb * D * 8), ("q_max", bh * Nb * D * 8), ("k_avg", bh * Nb * D * 8),
             ("k_max", bh * Nb * D * 8), ("scores", bh * Nb * Nb * 8), ("lmax", bh * Nb * Nb * 8),
             ("rank_state", bh * 3 * 32), ("rank_hist", bh * 3 * 2048 * 4), ("map", bh * Nb * Nb),
             ("lists", bh * Nb * Nb * 2), ("counts", bh * Nb * 16), ("out", bh * Np * D * 2),
             ("zeros", 256), ("order", 8 * bh * -(-Nb // 8) * 4), ("stage", 8)]
    nv = 1 if getattr(w, "fp4", "mxfp4") == "nvfp4" else 0  # NVFP4 sections, empty for MXFP4
    sizes += [("q_nv_scale", nv * bh * Np * D // 16), ("k_nv_scale", nv * bh * Np * D // 16),
              ("q_nv_bf16", nv * bh * Np * D * 2), ("k_nv_bf16", nv * bh * Np * D * 2),
              ("nv_tscale", nv * bh * 8), ("qk_amax", nv * 2 * bh * D * 4)]
    off, o = {}, 0
    for name, n in sizes:
        off["off_" + name] = o
        o = al(o + n)
    P = Nb * Nb
    _, q4, q8, q16 = w.quota_bp
    rnd = lambda x: (P * x + 5000) // 10000
    return dict(off, total_bytes=o, Nb=Nb, B=B, Np=Np, kp8=kp8, Hp=nby * w.region_h,
                Wp=nbx * w.region_w, pairs=P, c16=rnd(q16), c8=rnd(q16 + q8), c4=rnd(q16 + q8 + q4))


@pytest.mark.parametrize("fp4", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_layout_matches_rederivation(name, fp4):
    w = synth.WORKLOADS[name].with_(fp4=fp4)
    L = b.workspace_layout(b.Config.from_workload(w))
    exp = _layout_py(w)
    for k, v in exp.items():
        assert L[k] == v, k
    assert b.workspace_bytes(b.Config.from_workload(w)) == exp["total_bytes"]
    assert all(L[k] % 256 == 0 for k in L if k.startswith("off_"))


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError):
        saved = b._lib
        try:
            b._lib = None
            b.load(str(tmp_path / "nope.so"))
        finally:
            b._lib = saved


def test_binding_checks_tensors_before_the_library_call():
    """The kernels read q/k/v/out as contiguous bf16 [batch, heads, N, D] buffers; the binding
    refuses anything else on the host (checked here with host tensors, before any device call)."""
    import torch
    cfg = _cfg()
    shape = (cfg.batch, cfg.heads, cfg.N, cfg.head_dim)
    good = torch.zeros(shape, dtype=torch.bfloat16)
    ws = torch.zeros(16, dtype=torch.uint8)
    cases = [
        (torch.zeros(shape, dtype=torch.float16), "dtype"),
        (torch.zeros(shape[:-1] + (shape[-1] + 2,), dtype=torch.bfloat16)[..., :shape[-1]], "contiguous"),
        (torch.zeros((cfg.batch * cfg.heads, cfg.N, cfg.head_dim), dtype=torch.bfloat16), "shape"),
        (good, "device"),
    ]
    for q, what in cases:
        with pytest.raises(ValueError, match=what):
            b.prepare(cfg, q, good, good, ws)
    with pytest.raises(ValueError, match="shape"):
        b.restore(cfg, ws, torch.zeros((1, 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bytes"):
        b.draft_rank(cfg, ws, map_out=torch.zeros(3, dtype=torch.uint8))
    with pytest.raises(ValueError, match="shape"):
        b.attention_section_clocks(cfg, 256, torch.zeros(31, dtype=torch.int64))
    with pytest.raises(ValueError, match="dtype"):
        b.attention_section_clocks(cfg, 256, torch.zeros(b.SECTION_CLOCK_WORDS, dtype=torch.int32))


def _oracle_imports(path):
    """(enclosing top-level function or None, line) of every import of the oracle package in a file."""
    import ast
    tree = ast.parse(open(path).read(), filename=path)
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            inner = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) and fn is None else fn
            names = []
            if isinstance(child, ast.Import):
                names = [a.name for a in child.names]
            elif isinstance(child, ast.ImportFrom):
                names = [child.module or ""]
            if any(n == "oracle" or n.startswith("oracle.") for n in names):
                found.append((fn, child.lineno))
            visit(child, inner)

    visit(tree, None)
    return found


def test_product_path_never_reaches_the_oracle():
    """The oracle is test infrastructure: no module of the package imports it, and bench.py and the
    entry points reach it only from the CPU-baseline leg and from smoke() (the check against it)."""
    import glob
    pkg = glob.glob(os.path.join(ROOT, "video_dit_mixed_amd", "**", "*.py"), recursive=True)
    assert pkg
    for p in pkg:
        assert _oracle_imports(p) == [], p
    assert {fn for fn, _ in _oracle_imports(os.path.join(ROOT, "bench.py"))} == {"_cpu_baseline_head"}
    assert {fn for fn, _ in _oracle_imports(os.path.join(ROOT, "__graft_entry__.py"))} <= {"smoke", "build"}
