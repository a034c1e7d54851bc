"""GPU: the section-clock diagnostic runs the same attention as dap_attention.

`dap_attention_section_clocks` is a second instance of the attention kernel that reads the shader
clock around each part of the key-block loop.  Its output must equal dap_attention's bit for bit
(the clock reads change no arithmetic), it must leave the stage word at ATTENDED, and its counters
must be consistent with the block map: the wave-blocks counted per phase are the waves of a row
times the kept blocks of that level, summed over rows, and no wave spends more cycles in the parts
than it lives."""
import pytest

from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_2x16x16", {}, "mxfp4"),                                # 16-token blocks, one wave per row
    ("mid_8x24x40", {}, "nvfp4"),                                 # 64-token blocks, two waves
    ("mid_8x24x40", {"region_h": 8, "region_w": 16}, "mxfp4"),    # 128-token blocks, four waves
    ("mid_8x24x40", {"region_h": 8, "region_w": 16}, "nvfp4"),
]


@pytest.mark.parametrize("name,geo,fp4", CASES, ids=[f"{n}-{g.get('region_w', 'own')}-{f}" for n, g, f in CASES])
def test_section_clocks_match_attention(name, geo, fp4):
    import torch
    w = synth.workload(name).with_(fp4=fp4, **geo)
    cfg = b.Config.from_workload(w)
    L = b.workspace_layout(cfg)
    log(f"section clocks: {w.name} regions {w.region_h}x{w.region_w} {fp4}")
    q, k, v = to_device(*synth.make_inputs(w))
    ws = b.alloc_workspace(cfg, q.device)
    b.prepare(cfg, q, k, v, ws)
    b.draft_rank(cfg, ws)
    b.attention(cfg, ws)
    torch.cuda.synchronize()
    shape = (L["bh"], L["Np"], L["D"])
    ref = b.section(ws, L, "out", torch.int16, shape).clone()

    clk = torch.zeros(b.SECTION_CLOCK_WORDS, dtype=torch.int64, device=q.device)
    b.section(ws, L, "out", torch.int16, shape).zero_()
    b.attention_section_clocks(cfg, ws, clk)
    torch.cuda.synchronize()
    got = b.section(ws, L, "out", torch.int16, shape)
    assert torch.equal(got, ref), "the clocked kernel's output differs from dap_attention's"
    assert b.stage_words(ws, L)[0] == b.STAGE_ATTENDED

    c = clk.cpu().numpy().astype("uint64").reshape(4, 8)
    counts = b.section(ws, L, "counts", torch.int32, (L["bh"], L["Nb"], 4)).cpu().numpy()
    B = w.region_h * w.region_w
    waves = max(B // 32, 1)
    p4 = 3 if fp4 == "nvfp4" else 2
    want = {0: counts[..., 0].sum(), 1: counts[..., 1].sum(), p4: counts[..., 2].sum()}
    log(f"blocks per phase {want}; counters {c.tolist()}")
    for p in range(4):
        assert int(c[p, 6]) == waves * int(want.get(p, 0)), f"phase {p}: wave-blocks"
        if want.get(p, 0):
            assert all(int(x) > 0 for x in c[p, [2, 5]]), f"phase {p}: Q K^T and P V cycles"
        else:
            assert not c[p, :6].any(), f"phase {p} ran no block but counted cycles"
    assert int(c[:, :6].sum()) <= int(c[0, 7]), "parts exceed the waves' lifetimes"
