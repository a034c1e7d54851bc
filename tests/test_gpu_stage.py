"""GPU: the workspace's stage word enforces the call order reorder/pack -> draft + rank ->
attention -> restore (pith.science, "DraftAttention: Fast Video Diffusion via Low-Resolution
Attention Guidance", Abstract).  Calls made out of order, or on a workspace another configuration
left behind, finish normally, produce zeros and leave the stage broken until the next prepare; a
correct sequence afterwards gives the same bits as on a fresh workspace."""
import numpy as np
import pytest

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

from gpu_util import log, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _setup(quota=None):
    import torch
    w = synth.workload(1).with_(heads=2)
    if quota is not None:
        w = w.with_(quota_bp=quota)
    cfg = b.Config.from_workload(w)
    q, k, v = to_device(*synth.make_inputs(w))
    ws = torch.full((b.workspace_bytes(cfg),), 0xFF, dtype=torch.uint8, device=q.device)
    out = torch.full_like(q, float("nan"))
    return cfg, b.workspace_layout(cfg), q, k, v, ws, out


def _packed_out(ws, L):
    import torch
    return b.section(ws, L, "out", torch.int16, (L["bh"], L["Np"], L["D"]))


def test_full_sequence_reaches_attended():
    import torch
    cfg, L, q, k, v, ws, out = _setup()
    b.prepare(cfg, q, k, v, ws)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_PREPARED
    b.draft_rank(cfg, ws)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_RANKED
    b.attention(cfg, ws)
    b.restore(cfg, ws, out)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_ATTENDED
    assert bool(torch.isfinite(out.float()).all()) and float(out.float().abs().max()) > 0


@pytest.mark.parametrize("calls", ["attention", "prepare+attention", "draft_rank+attention"])
def test_out_of_order_calls_give_zeros(calls):
    import torch
    cfg, L, q, k, v, ws, out = _setup()
    log(f"calls: {calls} on a workspace of 0xFF bytes")
    if "prepare" in calls:
        b.prepare(cfg, q, k, v, ws)
    if "draft_rank" in calls:
        b.draft_rank(cfg, ws)
    b.attention(cfg, ws)
    b.restore(cfg, ws, out)
    torch.cuda.synchronize()
    st = b.stage_words(ws, L)[0]
    assert st == b.STAGE_BROKEN, hex(st)
    assert not bool(_packed_out(ws, L).any())
    assert not bool(out.view(torch.int16).any())


def test_stage_of_another_configuration_does_not_count():
    """A workspace fully processed under one quota mix is handed to attention and restore under
    another: the configuration tag differs, so both produce zeros."""
    import torch
    cfg_a, L, q, k, v, ws, out = _setup()
    b.forward(cfg_a, q, k, v, ws=ws, out=out)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_ATTENDED
    cfg_b = b.Config.from_workload(synth.workload(1).with_(heads=2, quota_bp=(5000, 0, 0, 5000)))
    assert b.workspace_layout(cfg_b)["off_out"] == L["off_out"]
    b.attention(cfg_b, ws)
    out_b = torch.full_like(out, float("nan"))
    b.restore(cfg_b, ws, out_b)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_BROKEN
    assert not bool(_packed_out(ws, L).any()) and not bool(out_b.view(torch.int16).any())


def test_broken_workspace_recovers_with_a_full_sequence():
    import torch
    cfg, L, q, k, v, ws, out = _setup()
    _, ref, _ = run_gpu(cfg, q, k, v)          # fresh workspace
    b.attention(cfg, ws)                       # out of order: broken
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_BROKEN
    b.forward(cfg, q, k, v, ws=ws, out=out)
    torch.cuda.synchronize()
    assert b.stage_words(ws, L)[0] == b.STAGE_ATTENDED
    assert torch.equal(out, ref)
