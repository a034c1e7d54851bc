"""GPU: one layer captured into a HIP graph replays to the eager result bit for bit.

The four calls launch kernels only (memory the library clears is cleared by its own fill kernels,
never by a memset node), so a caller can capture a whole layer.  Each replay runs after eager work
of the program's own -- a zero fill of the output and, for the allocation-free preparation, an eager
preparation of another layer that leaves different contents in the library's static scratch array --
and is checked against the eager output each time."""
import pytest

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def _layer(cfg, q, k, v, ws, out, static):
    (b.prepare_static_scratch if static else b.prepare)(cfg, q, k, v, ws)
    b.draft_rank(cfg, ws)
    b.attention(cfg, ws)
    b.restore(cfg, ws, out)


@pytest.mark.parametrize("static", [False, True], ids=["prepare", "prepare_static_scratch"])
@pytest.mark.parametrize("wi", [0, 1])
def test_layer_replays_from_a_graph(wi, static):
    import torch
    w = synth.workload(wi)
    cfg = b.Config.from_workload(w)
    log(f"graph capture: {w.name}, {'static scratch' if static else 'workspace scratch'}")
    q, k, v = to_device(*synth.make_inputs(w))
    dev = q.device
    ws_ref, out_ref = b.alloc_workspace(cfg, dev), torch.empty_like(q)
    _layer(cfg, q, k, v, ws_ref, out_ref, static)
    torch.cuda.synchronize()
    assert float(out_ref.float().abs().max()) > 0

    # another layer (other inputs, another shape) whose eager runs sit between the replays
    w2 = synth.workload(1 - wi).with_(seed=synth.workload(1 - wi).seed + 7)
    cfg2 = b.Config.from_workload(w2)
    q2, k2, v2 = to_device(*synth.make_inputs(w2))
    ws2, out2 = b.alloc_workspace(cfg2, dev), torch.empty_like(q2)

    ws, out = b.alloc_workspace(cfg, dev), torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (the static array is looked up here)
        _layer(cfg, q, k, v, ws, out, static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(cfg, q, k, v, ws, out, static)
    torch.cuda.synchronize()

    for rep in range(3):
        out.zero_()
        _layer(cfg2, q2, k2, v2, ws2, out2, static)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"replay {rep}")
        assert torch.equal(out, out_ref), f"replay {rep} differs from the eager layer"
        assert b.stage_words(ws, b.workspace_layout(cfg))[0] == b.STAGE_ATTENDED
