"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: pooled descriptors, quantised codes and scales, block maps, per-row lists and the restore
permutation bit-exact; draft scores within 1e-12 relative; outputs within rel-L2 5e-3 and
max-abs 2e-2 over real tokens.  Full-size workloads compare every head-level result of two sampled
heads and the outputs of sampled query blocks (edge blocks with padding, the longest and shortest
rows, and seeded random ones); the other heads carry copies of the sampled heads' inputs."""
import numpy as np
import pytest

import oracle
from oracle import draft as odraft, layout as olayout, pipeline as opipe
from video_dit_mixed_amd import binding as b
from video_dit_mixed_amd import synth

from gpu_util import (Sections, bf16_bits, log, rel_l2, run_gpu, to_device, MAX_ABS_TOL,
                      REL_L2_TOL, SCORE_RTOL)

pytestmark = pytest.mark.gpu


def _inputs(w, exact_heads=None):
    """Exact generator output for `exact_heads` (all when None); the other heads copy them."""
    if exact_heads is None:
        return synth.make_inputs(w)
    Q, K, V = synth.make_inputs(w, heads=exact_heads)
    BH = w.batch * w.heads
    src = list(exact_heads)
    for i in range(BH):
        if i in exact_heads:
            continue
        j = src[i % len(src)]
        bb, h = divmod(i, w.heads)
        sb, sh = divmod(j, w.heads)
        Q[bb, h], K[bb, h], V[bb, h] = Q[sb, sh], K[sb, sh], V[sb, sh]
    return Q, K, V


def _oracle_head(w, Q, K, V, bhi):
    bb, h = divmod(bhi, w.heads)
    return opipe.prepare_head(Q[bb, h], K[bb, h], V[bb, h], T=w.T, H=w.H, W=w.W, rh=w.region_h,
                              rw=w.region_w, lam=w.lam, quota_bp=w.quota_bp, fp4_format=w.fp4)


def _nv_value_bits(codes, scale_bytes):
    """bf16 bits of E2M1 value x E4M3 group scale with the code's sign (exact in bf16)."""
    from oracle import quant
    c = codes.astype(np.int64)
    mag = quant.E2M1_GRID[c & 7] * np.repeat(quant.e4m3fn_decode(scale_bytes), 16, axis=-1)
    bits = (mag.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits | ((c & 8) << 12).astype(np.uint16)


def _check_prep(S: Sections, r, L):
    need16 = L["c16"] > 0
    need8 = L["c8"] > L["c16"]
    need4 = L["c4"] > L["c8"]
    for name in ("q_avg", "q_max", "k_avg", "k_max"):
        np.testing.assert_array_equal(getattr(S, name), getattr(r, name), err_msg=name)
    if need16:
        np.testing.assert_array_equal(S.q_bf16, bf16_bits(r.qp), err_msg="q bf16 pack")
        np.testing.assert_array_equal(S.k_bf16, bf16_bits(r.kp), err_msg="k bf16 pack")
        np.testing.assert_array_equal(S.vp_bf16, bf16_bits(r.vp), err_msg="v bf16 pack")
    if need8:
        np.testing.assert_array_equal(S.q_i8, r.q_i8, err_msg="q int8")
        np.testing.assert_array_equal(S.k_i8, r.k_i8, err_msg="k int8")
        np.testing.assert_array_equal(S.q_i8_s.view(np.uint32), r.q_i8_s.view(np.uint32))
        np.testing.assert_array_equal(S.k_i8_s.view(np.uint32), r.k_i8_s.view(np.uint32))
    if need4 and r.fp4_format == "nvfp4":
        assert S.nv
        for name, got_c, got_s, got_b, t_idx, rc, rs, rt in (
                ("q", S.q_fp4, S.q_nv_s, S.q_nv_bf16, 0, r.q_nv, r.q_nv_s, r.q_nv_t),
                ("k", S.k_fp4, S.k_nv_s, S.k_nv_bf16, 1, r.k_nv, r.k_nv_s, r.k_nv_t)):
            np.testing.assert_array_equal(got_c, rc, err_msg=f"{name} nvfp4 codes")
            np.testing.assert_array_equal(got_s, rs, err_msg=f"{name} nvfp4 e4m3 scales")
            assert S.nv_t[t_idx].view(np.uint32) == np.float32(rt).view(np.uint32), f"{name} tensor scale"
            np.testing.assert_array_equal(got_b, _nv_value_bits(rc, rs), err_msg=f"{name} nvfp4 bf16")
    elif need4:
        np.testing.assert_array_equal(S.q_fp4, r.q_fp4, err_msg="q mxfp4 codes")
        np.testing.assert_array_equal(S.k_fp4, r.k_fp4, err_msg="k mxfp4 codes")
        np.testing.assert_array_equal(S.q_e8, r.q_e8, err_msg="q e8m0")
        np.testing.assert_array_equal(S.k_e8, r.k_e8, err_msg="k e8m0")
    if need8 or need4:
        np.testing.assert_array_equal(S.v_fp8, r.v_fp8, err_msg="v fp8 codes")
        np.testing.assert_array_equal(S.v_s.view(np.uint32), r.v_s.view(np.uint32))


def _check_map(S: Sections, r, L):
    rel = np.abs(S.scores - r.A) / np.maximum(np.abs(r.A), 1e-300)
    assert rel.max() <= SCORE_RTOL, f"draft scores rel err {rel.max():.3e}"
    cuts = (int(L["c16"]), int(L["c8"]), int(L["c4"]))
    assert cuts == r.cuts
    # rank on the GPU's own scores: exact, no exceptions
    own = odraft.assign_levels(odraft.rank_pairs(S.scores), cuts)
    np.testing.assert_array_equal(S.map, own, err_msg="rank of the device's own scores")
    # against the oracle's map: the only admissible difference is a pair within 1e-12 of a cut
    diff = np.argwhere(S.map != r.levels)
    if diff.size:
        flat = r.A.ravel()
        order = np.lexsort((np.arange(flat.size), -flat))
        cut_scores = [flat[order[c - 1]] for c in cuts if 0 < c <= flat.size]
        bad = [tuple(p) for p in diff
               if not any(abs(r.A[tuple(p)] - cs) <= 1e-12 * cs for cs in cut_scores)]
        log(f"map differs at {len(diff)} pairs, {len(bad)} not near a cut")
        assert not bad
    # per-row lists and counts
    for qb in range(L["Nb"]):
        row = S.map[qb]
        n16, n8, n4 = (int((row == lv).sum()) for lv in (3, 2, 1))
        assert tuple(S.counts[qb]) == (n16, n8, n4, 0)
        lst = S.lists[qb]
        np.testing.assert_array_equal(lst[:n16], np.flatnonzero(row == 3))
        np.testing.assert_array_equal(lst[n16:n16 + n8], np.flatnonzero(row == 2))
        np.testing.assert_array_equal(lst[n16 + n8:n16 + n8 + n4], np.flatnonzero(row == 1))


def _check_out(S: Sections, r, blocks, precomputed=None):
    """Outputs of `blocks` against the oracle; `precomputed` = (rows, fp64 outputs) from the
    oracle worker pool, else the oracle runs here."""
    B = r.B
    rows = np.concatenate([qb * B + np.flatnonzero(r.valid[qb]) for qb in blocks])
    if precomputed is None:
        opipe.attend(r, q_blocks=blocks)
    else:
        r.out_packed[precomputed[0]] = precomputed[1]
    ref = r.out_packed[rows]
    from oracle import quant
    ref = quant.bf16_rne(ref)
    got = synth.bf16_bits_to_f32(S.out_packed[rows]).astype(np.float64)
    e_rel = rel_l2(got, ref)
    e_max = np.abs(got - ref).max() if rows.size else 0.0
    empty = sum(1 for qb in blocks if S.counts[qb][:3].sum() == 0)
    log(f"out rows={rows.size} rel_l2={e_rel:.3e} max_abs={e_max:.3e} empty_rows={empty}")
    assert e_rel <= REL_L2_TOL and e_max <= MAX_ABS_TOL
    return e_rel, e_max


def _check_restore(out, S_out_packed_all, L, w):
    """The restored output equals the packed output under the oracle's token permutation."""
    g = olayout.geometry(w.T, w.H, w.W, w.region_h, w.region_w)
    src = olayout.source_index(g)
    ok = src >= 0
    got = out.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    for bhi, packed in S_out_packed_all:
        bb, h = divmod(bhi, w.heads)
        exp = np.empty((g.N, w.head_dim), np.uint16)
        exp[src[ok]] = packed[ok]
        np.testing.assert_array_equal(got[bb, h], exp)


def _sample_blocks(r, S, k=12, seed=0):
    Nb = r.g.Nb
    kept = S.counts[:, :3].sum(1)
    edge = [qb for qb in range(Nb) if not r.valid[qb].all()]
    pick = {0, Nb - 1, int(np.argmax(kept)), int(np.argmin(kept))}
    pick |= set(edge[:2]) | set(edge[-2:])
    rng = np.random.default_rng(seed)
    pick |= set(rng.choice(Nb, size=min(k, Nb), replace=False).tolist())
    return sorted(pick)


def _geo_kw(w):
    return dict(T=w.T, H=w.H, W=w.W, rh=w.region_h, rw=w.region_w, lam=w.lam, quota_bp=w.quota_bp,
                fp4_format=w.fp4)


def _run_case(w, exact_heads=None, sample_blocks=None, check_heads=None, inputs=None,
              all_blocks_heads=()):
    """`sample_blocks`: compare that many sampled query blocks per checked head (None: all);
    heads in `all_blocks_heads` are compared over every query block, with the oracle's attention
    split over the worker pool."""
    log(f"case {w.name} quota={w.quota_bp} lam={w.lam} batch={w.batch} fp4={w.fp4}")
    Q, K, V = _inputs(w, exact_heads) if inputs is None else inputs
    cfg = b.Config.from_workload(w)
    q, k, v = to_device(Q, K, V)
    log("gpu run")
    ws, out, L = run_gpu(cfg, q, k, v)
    heads = check_heads if check_heads is not None else range(w.batch * w.heads)
    packed = []
    for bhi in heads:
        log(f"head {bhi}: oracle")
        r = _oracle_head(w, Q, K, V, bhi)
        S = Sections(ws, L, bhi)
        _check_prep(S, r, L)
        _check_map(S, r, L)
        pre = None
        if sample_blocks is None or bhi in all_blocks_heads:
            blocks = list(range(r.g.Nb))
            if bhi in all_blocks_heads:
                import oracle_pool
                bb, h = divmod(bhi, w.heads)
                log(f"head {bhi}: oracle attention over all {r.g.Nb} query blocks "
                    f"({'pool' if oracle_pool.get() else 'this process'})")
                pre = oracle_pool.attend_head(Q[bb, h], K[bb, h], V[bb, h], _geo_kw(w), blocks)
        else:
            blocks = _sample_blocks(r, S, sample_blocks, bhi)
        _check_out(S, r, blocks, pre)
        packed.append((bhi, S.out_packed))
    _check_restore(out, packed, L, w)
    _check_order(ws, L)
    return ws, out


def _check_order(ws, L):
    """The attention work order covers every (head, query block) exactly once; each die's slice
    holds a block of every head with that die's share of the head's rows."""
    import torch
    Nb, BH = L["Nb"], L["bh"]
    stride = BH * -(-Nb // 8)
    tab = b.section(ws, L, "order", torch.int32, (8, stride)).cpu().numpy().view(np.uint32)
    seen = []
    q, rem = divmod(Nb, 8)
    for x in range(8):
        # snake deal of the cost-ranked rows: one row per die per round, the last partial round
        # going to dies 0.. (even round count) or ..7 (odd)
        size = q + int(x >= 8 - rem if q % 2 else x < rem)
        items = tab[x, :BH * size]
        assert np.all((items >> 16).reshape(BH, size) == np.arange(BH)[:, None])
        seen.append(items)
    allitems = np.sort(np.concatenate(seen))
    exp = np.sort((np.arange(BH)[:, None].astype(np.uint32) << 16 | np.arange(Nb)[None, :]).ravel())
    np.testing.assert_array_equal(allitems, exp)


# ------------------------------------------------------------------------------------ workloads

def test_parity_tiny_all_heads():
    _run_case(synth.workload(0))


def test_parity_mid_sampled_heads():
    w = synth.workload(1)
    _run_case(w, exact_heads=[0, 5, 11], check_heads=[0, 11])


# ------------------------------------------------------------------------------------ phases alone

@pytest.mark.parametrize("quota", [(0, 0, 0, 10000), (0, 0, 10000, 0), (0, 10000, 0, 0),
                                   (5000, 5000, 0, 0), (4000, 2000, 2000, 2000)])
@pytest.mark.parametrize("wi", [0, 1])
def test_single_and_mixed_levels(wi, quota):
    w = synth.workload(wi).with_(quota_bp=quota, heads=2)
    _run_case(w)


def test_dense_equals_plain_attention_on_gpu():
    """Quotas 0/0/0/100: every pair is 16-bit, so the output is dense attention up to bf16 P."""
    import torch
    w = synth.workload(1).with_(quota_bp=(0, 0, 0, 10000), heads=2)
    Q, K, V = synth.make_inputs(w)
    cfg = b.Config.from_workload(w)
    q, k, v = to_device(Q, K, V)
    _, out, _ = run_gpu(cfg, q, k, v)
    qf, kf, vf = (t.float().cpu() for t in (q, k, v))
    ref = torch.softmax(qf @ kf.transpose(-1, -2) / np.sqrt(w.head_dim), dim=-1) @ vf
    got = out.float().cpu()
    rel = float((got - ref).norm() / ref.norm())
    log(f"dense rel_l2={rel:.3e}")
    assert rel <= REL_L2_TOL


def test_all_skip_outputs_zero():
    w = synth.workload(0).with_(quota_bp=(10000, 0, 0, 0))
    Q, K, V = synth.make_inputs(w)
    _, out, _ = run_gpu(b.Config.from_workload(w), *to_device(Q, K, V))
    assert float(out.float().abs().max()) == 0.0


@pytest.mark.parametrize("lam", [0.0, 1.0])
def test_lambda_endpoints(lam):
    _run_case(synth.workload(0).with_(lam=lam))


def test_batch_two():
    _run_case(synth.workload(0).with_(batch=2))


@pytest.mark.parametrize("fp4", ["mxfp4", "nvfp4"])
def test_ragged_odd_grid(fp4):
    # regions that leave padding on both axes and an odd frame count (64-token blocks, D = 128)
    w = synth.Workload("ragged", 3, 13, 21, 2, 128, 8, 8, 0.5, (3000, 2500, 2500, 2000), seed=77,
                       fp4=fp4)
    _run_case(w)


def test_deterministic_bitwise():
    import torch
    w = synth.workload(1).with_(heads=3)
    Q, K, V = synth.make_inputs(w)
    cfg = b.Config.from_workload(w)
    q, k, v = to_device(Q, K, V)
    ws1, out1, _ = run_gpu(cfg, q, k, v)
    ws2, out2, _ = run_gpu(cfg, q, k, v)
    L = b.workspace_layout(cfg)
    assert torch.equal(out1, out2)
    for name, dt, shape in (("map", torch.uint8, (L["bh"], L["Nb"], L["Nb"])),
                            ("scores", torch.float64, (L["bh"], L["Nb"], L["Nb"]))):
        assert torch.equal(b.section(ws1, L, name, dt, shape), b.section(ws2, L, name, dt, shape))


def test_workspace_contents_do_not_leak_between_layers():
    """The workspace is caller-owned scratch: whatever it holds before a layer (all-ones bytes, or
    the lists, counters, maps and operands of a previous layer with other inputs and quotas) must not
    change a single output bit, block-map entry or draft score."""
    import torch
    w = synth.workload(1).with_(heads=3)
    w_prev = w.with_(seed=w.seed + 1, quota_bp=(1000, 3000, 3000, 3000))
    cfg, cfg_prev = b.Config.from_workload(w), b.Config.from_workload(w_prev)
    q, k, v = to_device(*synth.make_inputs(w))
    qp, kp, vp = to_device(*synth.make_inputs(w_prev))
    nbytes = max(b.workspace_bytes(cfg), b.workspace_bytes(cfg_prev))
    L = b.workspace_layout(cfg)
    secs = (("map", torch.uint8, (L["bh"], L["Nb"], L["Nb"])),
            ("scores", torch.float64, (L["bh"], L["Nb"], L["Nb"])))
    results = []
    for before in ("zeros", "ones", "previous layer"):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
        if before == "ones":
            ws.fill_(0xFF)
        elif before == "previous layer":
            b.forward(cfg_prev, qp, kp, vp, ws=ws)
        log(f"workspace before the layer: {before}")
        out, _ = b.forward(cfg, q, k, v, ws=ws)
        torch.cuda.synchronize()
        results.append((out, [b.section(ws, L, n, dt, s).clone() for n, dt, s in secs]))
    for out, sec in results[1:]:
        assert torch.equal(out, results[0][0])
        for a, r in zip(sec, results[0][1]):
            assert torch.equal(a, r)


def test_calls_follow_the_callers_stream():
    """Every call is ordered on the stream it is handed: the inputs are produced on a side stream
    behind a long spin, and the whole layer is enqueued on that stream with no host wait in between;
    the result must equal the default-stream run bit for bit."""
    import torch
    w = synth.workload(1).with_(heads=3)
    cfg = b.Config.from_workload(w)
    q, k, v = to_device(*synth.make_inputs(w))
    _, ref_out, _ = run_gpu(cfg, q, k, v)
    ws = torch.full((b.workspace_bytes(cfg),), 0xFF, dtype=torch.uint8, device=q.device)
    out = torch.full_like(q, float("nan"))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)  # a bounded spin of about 20 ms on the side stream
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        b.forward(cfg, q2, k2, v2, ws=ws, out=out, stream=s.cuda_stream)
    s.synchronize()
    assert torch.equal(out, ref_out)


# ------------------------------------------------------------------------------------ 16-token blocks
# 3 x 13 x 21 latent: every region shape leaves padding on both axes (4x4: 16 x 24 padded grid,
# 2x8: 14 x 24, 1x16: 13 x 32); one wave per query block, head_dim 64 and 128.

@pytest.mark.parametrize("quota", [(0, 0, 0, 10000), (0, 0, 10000, 0), (0, 10000, 0, 0),
                                   (2000, 2000, 3000, 3000)])
@pytest.mark.parametrize("region", [(4, 4), (2, 8), (1, 16)])
@pytest.mark.parametrize("D", [128, 64])
def test_block16(D, region, quota):
    rh, rw = region
    w = synth.Workload("b16", 3, 13, 21, 2, D, rh, rw, 0.5, quota, seed=4249)
    _run_case(w)


# ------------------------------------------------------------------------------------ 128-token blocks
# 128-token blocks (the full-size configurations) at CPU-checkable sizes.
# 20 x 36 latent with 8 x 16 regions: the last region row holds 4 real rows (keys 64..127 of its
# blocks are all padding) and the last region column 4 real columns.

@pytest.mark.parametrize("quota", [(0, 0, 0, 10000), (0, 0, 10000, 0), (0, 10000, 0, 0),
                                   (2000, 2000, 3000, 3000), (7000, 1000, 1000, 1000)])
@pytest.mark.parametrize("dims", [(128, 8, 16), (64, 8, 16), (128, 4, 32), (128, 16, 8)])
def test_block128_small(dims, quota):
    D, rh, rw = dims
    w = synth.Workload("b128", 2, 20, 36, 2, D, rh, rw, 0.5, quota, seed=4242)
    _run_case(w)


@pytest.mark.parametrize("quota", [(0, 0, 0, 10000), (5000, 1500, 1500, 2000)])
def test_block128_long_rows(quota):
    # 80 key blocks per head: long rows that cycle both tile buffers many times
    w = synth.Workload("b128long", 4, 40, 64, 2, 128, 8, 16, 0.5, quota, seed=4243)
    _run_case(w)


@pytest.mark.parametrize("quota", [(5000, 1500, 1500, 2000), (8500, 0, 750, 750)])
def test_all_draft_scores_tied(quota):
    # Head 0 has Q = 0, so every pooled logit is 0 and every draft score is exactly 1/Nb: the
    # ranking falls back to the pair index and every pair shares every cut's key prefix (the rank
    # candidate list overflows and that head keeps scanning all pairs).  Head 1 is ordinary.
    w = synth.Workload("ties", 4, 40, 64, 2, 128, 8, 16, 0.5, quota, seed=4244)
    Q, K, V = synth.make_inputs(w)
    Q[0, 0] = 0
    _run_case(w, inputs=(Q, K, V))


@pytest.mark.parametrize("geom", [(4, 40, 64, 128, 8, 16), (4, 24, 40, 64, 8, 8)])
def test_zero_blocks_and_channels(geom):
    # Exact zeros where a scale becomes 0: two V channels of head 0 (FP8 scale 0, so the
    # accumulator's unit change multiplies those channels by 0), one key region of head 0 (INT8 block
    # scale 0, E8M0 code 0, pooled descriptor 0) and one query region of head 1.  Every precision
    # is used; 128-token blocks load tiles straight into LDS, 64-token blocks through registers.
    T, H, W, D, rh, rw = geom
    w = synth.Workload("zeros", T, H, W, 2, D, rh, rw, 0.5, (4000, 2000, 2000, 2000), seed=4245)
    Q, K, V = synth.make_inputs(w)
    V[0, 0, :, 3] = 0
    V[0, 0, :, D - 5] = 0

    def region_tokens(t, ry, rx):
        ys, xs = np.meshgrid(np.arange(ry * rh, (ry + 1) * rh), np.arange(rx * rw, (rx + 1) * rw),
                             indexing="ij")
        return ((t * H + ys) * W + xs).ravel()

    K[0, 0, region_tokens(0, 1, 2), :] = 0
    Q[0, 1, region_tokens(1, 2, 1), :] = 0
    _run_case(w, inputs=(Q, K, V))


def _scaled_bits(bits, k):
    """bf16 bits of the values times 2^-k (rounded to bf16; tiny results may be subnormal)."""
    f = synth.bf16_bits_to_f32(bits).astype(np.float64) * 2.0 ** -k
    return synth.f32_to_bf16_bits(f.astype(np.float32))


@pytest.mark.parametrize("geom", [(4, 40, 64, 128, 8, 16), (4, 24, 40, 64, 8, 8)])
def test_vanishing_blocks_and_channels(geom):
    # Values so small that a quantiser's fp32 reciprocal (127/a, 448/a) overflows: such a block or
    # channel quantises to zero.  Head 0: one key region near 2^-123 (INT8 reciprocal overflows)
    # and three V channels near 2^-116 (FP8 reciprocal finite, but the reciprocal of its scale
    # is not: the accumulator's unit change must not overflow), 2^-119 (at the bound) and 2^-122
    # (reciprocal overflows).  Head 1: one query region near 2^-114 (INT8 scale tiny but nonzero).
    T, H, W, D, rh, rw = geom
    w = synth.Workload("vanish", T, H, W, 2, D, rh, rw, 0.5, (4000, 2000, 2000, 2000), seed=4248)
    Q, K, V = synth.make_inputs(w)

    def region_tokens(t, ry, rx):
        ys, xs = np.meshgrid(np.arange(ry * rh, (ry + 1) * rh), np.arange(rx * rw, (rx + 1) * rw),
                             indexing="ij")
        return ((t * H + ys) * W + xs).ravel()

    kt = region_tokens(0, 1, 2)
    K[0, 0, kt, :] = _scaled_bits(K[0, 0, kt, :], 128)
    qt = region_tokens(1, 2, 1)
    Q[0, 1, qt, :] = _scaled_bits(Q[0, 1, qt, :], 119)
    for d, k in ((3, 118), (7, 121), (D - 5, 124)):
        V[0, 0, :, d] = _scaled_bits(V[0, 0, :, d], k)
    _run_case(w, inputs=(Q, K, V))


@pytest.mark.parametrize("geom", [(4, 40, 64, 128, 8, 16), (4, 24, 40, 64, 8, 8)])
def test_very_sparse(geom):
    # 0.1 % of the pairs kept (16-bit and 8-bit): most query blocks have no kept pair and must
    # output 0, the others attend to one or two key blocks.
    T, H, W, D, rh, rw = geom
    w = synth.Workload("sparse", T, H, W, 2, D, rh, rw, 0.5, (9990, 0, 5, 5), seed=4247)
    _run_case(w)


def test_max_regions():
    # The largest supported map: 4096 regions per head (one 8x16 region per frame), so pair
    # indices use all 24 bits and list entries reach 4095; sampled query blocks.
    w = synth.Workload("maxnb", 4096, 8, 16, 1, 64, 8, 16, 0.5, (5000, 1500, 1500, 2000), seed=4246)
    _run_case(w, exact_heads=[0], sample_blocks=8, check_heads=[0])


# ------------------------------------------------------------------------------------ full size

@pytest.mark.parametrize("wi", [2, 3, 4])
def test_parity_full_size(wi):
    w = synth.workload(wi)
    _run_case(w, exact_heads=[0, w.heads - 1], sample_blocks=10, check_heads=[0, w.heads - 1])


@pytest.mark.oracle_pool
def test_parity_full_size_one_head_every_block():
    # the 720p layer (85/0/7.5/7.5): head 0 over all 990 query blocks, the last head sampled
    w = synth.workload(2)
    _run_case(w, exact_heads=[0, w.heads - 1], sample_blocks=10, check_heads=[0, w.heads - 1],
              all_blocks_heads=(0,))


# ------------------------------------------------------------------------------------ NVFP4
# The pages' example 4-bit format (pchao.org blog, section 方法概览 bullet 2) selected instead of
# MXFP4: codes, E4M3 group scales, tensor scales and the bf16 operands of the 4-bit Q K^T are
# bit-exact; outputs within the usual tolerance.

@pytest.mark.parametrize("quota", [(0, 10000, 0, 0), (2000, 2000, 3000, 3000), (7000, 1000, 1000, 1000)])
@pytest.mark.parametrize("dims", [(128, 8, 16), (64, 8, 16), (128, 4, 32)])
def test_nvfp4_block128_small(dims, quota):
    D, rh, rw = dims
    w = synth.Workload("b128nv", 2, 20, 36, 2, D, rh, rw, 0.5, quota, seed=4250, fp4="nvfp4")
    _run_case(w)


@pytest.mark.parametrize("wi,D", [(0, 64), (0, 128), (1, 64), (1, 128)])
def test_nvfp4_block16_and_64(wi, D):
    w = synth.workload(wi).with_(quota_bp=(2500, 5000, 1000, 1500), head_dim=D, heads=2, fp4="nvfp4")
    _run_case(w)


def test_nvfp4_zero_tensor():
    # head 0 has Q = 0: its tensor scale is 0, every NVFP4 code and scale of Q is 0
    w = synth.Workload("nvzero", 4, 40, 64, 2, 128, 8, 16, 0.5, (5000, 3000, 1000, 1000), seed=4251,
                       fp4="nvfp4")
    Q, K, V = synth.make_inputs(w)
    Q[0, 0] = 0
    _run_case(w, inputs=(Q, K, V))


def test_nvfp4_vanishing_tensors():
    # Tensors so small that NVFP4's fp32 steps leave the normal range (R30's zero rule): head 0's Q
    # near 2^-116 (subnormal tensor scale, ordinary codes), head 1's K near 2^-128 (subnormal tensor
    # scale, group steps whose reciprocal overflows: codes 0 under nonzero group scales), head 2's Q
    # near 2^-132 (bf16 subnormals, mostly zeros), head 3's K near 2^-122 (subnormal steps with finite
    # reciprocals).  Codes, group scales and tensor scales must match the oracle bit for bit.
    w = synth.Workload("nvvanish", 4, 40, 64, 4, 128, 8, 16, 0.5, (4000, 3000, 1500, 1500), seed=4252,
                       fp4="nvfp4")
    Q, K, V = synth.make_inputs(w)
    Q[0, 0] = _scaled_bits(Q[0, 0], 120)
    K[0, 1] = _scaled_bits(K[0, 1], 132)
    Q[0, 2] = _scaled_bits(Q[0, 2], 136)
    K[0, 3] = _scaled_bits(K[0, 3], 126)
    _run_case(w, inputs=(Q, K, V))


@pytest.mark.parametrize("wi", [3, 4])
def test_nvfp4_full_size(wi):
    w = synth.workload(wi).with_(fp4="nvfp4")
    _run_case(w, exact_heads=[0, w.heads - 1], sample_blocks=10, check_heads=[0, w.heads - 1])
