"""CPU: the benchmark's roofline arithmetic and its traffic-file guard.

T_roof is the time the kept block pairs of a layer would take at the MI355X dense matrix-core peaks
of their precisions (bf16 2.5, int8 and fp8 5.0, fp4 10.1 PFLOP/s), one Q K^T and one P V of
2 B^2 D flops each per pair; NVFP4's Q K^T is priced at the bf16 peak, the precision it runs in."""
import json
import os

import pytest

import bench
from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quota_counts.json")


def _layout(w):
    return b.workspace_layout(b.Config.from_workload(w))


def test_roofline_of_the_720p_mix_by_hand():
    w = synth.workload("hunyuan720p_33x45x80")
    flops, t_roof, (n16, n8, n4) = bench.roofline_terms(_layout(w), w.batch * w.heads, w.head_dim)
    assert (n16, n8, n4) == (73508, 73507, 0)
    pair = 4 * 128 * 128 * 128                      # both contractions of one 128-token pair, D 128
    assert flops == 24 * (73508 + 73507) * pair
    t = 24 * (73508 * pair / 2.5e15 + 73507 * (pair / 2 / 5.0e15 + pair / 2 / 5.0e15))
    assert t_roof == pytest.approx(t, rel=1e-12)
    assert t_roof * 1e3 == pytest.approx(8.8794, abs=5e-5)


@pytest.mark.parametrize("fp4,qk_peak", [("mxfp4", 10.1e15), ("nvfp4", 2.5e15)])
def test_roofline_prices_the_4bit_level_by_format(fp4, qk_peak):
    w = synth.workload("hunyuan720p_4bit_33x45x80").with_(fp4=fp4)
    flops, t_roof, (n16, n8, n4) = bench.roofline_terms(_layout(w), w.batch * w.heads, w.head_dim,
                                                        w.fp4)
    assert (n16, n8, n4) == (0, 47045, 141134)
    half = 2 * 128 * 128 * 128
    t = 24 * (n8 * (half / 5.0e15 + half / 5.0e15) + n4 * (half / qk_peak + half / 5.0e15))
    assert t_roof == pytest.approx(t, rel=1e-12)
    assert flops == 24 * (n8 + n4) * 2 * half


def test_pair_counts_follow_the_golden_quota_counts():
    """The kept-pair counts the roofline is priced on are the hand-computed cuts of every workload."""
    gold = json.load(open(GOLDEN))["counts"]
    for name, want in gold.items():
        w = synth.workload(name)
        _, _, got = bench.roofline_terms(_layout(w), w.batch * w.heads, w.head_dim)
        assert got == (want["n16"], want["n8"], want["n4"]), name


def test_traffic_is_reported_only_for_the_kernel_it_was_taken_on():
    body = "# comment = ignored\nworkload = hunyuan720p_33x45x80\nsource_sha256_16 = {}\nhbm_bytes_per_launch = 12345\n"
    d = bench.source_digest()
    assert bench.parse_traffic(body.format(d), "hunyuan720p_33x45x80", d) == 12345.0
    assert bench.parse_traffic(body.format(d), "fewstep_91x48x84", d) is None     # another workload
    assert bench.parse_traffic(body.format("0" * 16), "hunyuan720p_33x45x80", d) is None  # another kernel
    assert bench.parse_traffic("", "hunyuan720p_33x45x80", d) is None


def test_lds_feed_needs_the_built_program(monkeypatch, capsys):
    """`bench.py --lds-feed` runs only what build() compiled; a missing program is an error, not a build."""
    from video_dit_mixed_amd import build as bld
    monkeypatch.setattr(bld, "LDS_FEED_BENCH", os.path.join(os.path.dirname(__file__), "no_such_program"))
    assert bench.lds_feed() == 1
    assert "not built" in capsys.readouterr().err
