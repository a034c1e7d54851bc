"""GPU: dap_prepare_static_scratch (the preparation with its scratch in the library's static device
array, for callers that cannot allocate) gives exactly what dap_prepare gives -- every workspace
section it writes, and the whole layer after it -- on two calls in a row, the second with a smaller
input, so the array's contents from the first call must not leak into the second.  With MXFP4 the
scratch is the V channel maxima; with NVFP4 also the Q and K channel maxima."""
import numpy as np
import pytest

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

# sections dap_prepare writes (v_amax and qk_amax are the scratch that the variant keeps elsewhere)
PREP_SECTIONS = ["q_bf16", "k_bf16", "vt_bf16", "q_i8", "k_i8", "q_i8_scale", "k_i8_scale",
                 "q_fp4", "k_fp4", "q_e8m0", "k_e8m0", "vt_fp8", "v_scale", "q_avg", "q_max",
                 "k_avg", "k_max", "zeros", "stage"]
NV_SECTIONS = ["q_nv_scale", "k_nv_scale", "q_nv_bf16", "k_nv_bf16", "nv_tscale"]


def _section_bytes(ws, L, name):
    import torch
    names = [n for n in b._LAYOUT_OFFS]
    offs = sorted((L["off_" + n], n) for n in names)
    i = [n for _, n in offs].index(name)
    end = offs[i + 1][0] if i + 1 < len(offs) else L["total_bytes"]
    return ws[L["off_" + name]:end]


@pytest.mark.parametrize("fp4", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("seq", [("mid_8x24x40", "tiny_2x16x16")])
def test_static_scratch_prepare_matches_prepare(seq, fp4):
    import torch
    for name in seq:
        w = synth.workload(name).with_(fp4=fp4)
        assert w.quota_bp[1] > 0  # the 4-bit level, and with it NVFP4's scratch, is in use
        cfg = b.Config.from_workload(w)
        L = b.workspace_layout(cfg)
        log(f"workload {name}, {fp4}: bh*D = {cfg.batch * cfg.heads * cfg.head_dim}")
        q, k, v = to_device(*synth.make_inputs(w))
        nbytes = b.workspace_bytes(cfg)
        ws_ref = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=q.device)
        ws_new = ws_ref.clone()
        b.prepare(cfg, q, k, v, ws_ref)
        b.prepare_static_scratch(cfg, q, k, v, ws_new)
        torch.cuda.synchronize()
        for sec in PREP_SECTIONS + (NV_SECTIONS if fp4 == "nvfp4" else []):
            a, c = _section_bytes(ws_ref, L, sec), _section_bytes(ws_new, L, sec)
            assert a.numel() > 0 or sec in ("q_e8m0", "k_e8m0")
            assert torch.equal(a, c), f"{name}: section {sec} differs"
        # the variant leaves the workspace's own scratch sections alone
        assert bool((_section_bytes(ws_new, L, "v_amax") == 0xA5).all())
        if fp4 == "nvfp4":
            qa = _section_bytes(ws_new, L, "qk_amax")
            assert qa.numel() == 2 * cfg.batch * cfg.heads * cfg.head_dim * 4
            assert bool((qa == 0xA5).all())
            assert not bool((_section_bytes(ws_ref, L, "qk_amax") == 0xA5).all())
        outs = []
        for ws in (ws_ref, ws_new):
            out = torch.empty_like(q)
            b.draft_rank(cfg, ws)
            b.attention(cfg, ws)
            b.restore(cfg, ws, out)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"{name}: layer output differs"
        assert float(outs[1].float().abs().max()) > 0
