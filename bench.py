"""Benchmark: one attention layer of draft-guided mixed-precision block-sparse attention on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --sweep [--workloads A,B,...] [--out FILE]
    python bench.py --section-clocks [--workload NAME] [--quota Q] [--fp4 F]   # where the waves' cycles go
    python bench.py --lds-feed                                                 # matrix-core / LDS program

The --sweep mode measures every workload (all five by default), one JSON line per case:
  * the workload's own quota: per-call median and minimum over R timed layers (R = 20, 5 for the
    91x48x84 few-step shape), ms/layer as the median of the per-layer sum of the four calls,
    T_roof / T_attention and its real-token variant (N/Np)^2, prepare and restore in GB/s of
    algorithmic HBM bytes, draft_rank against the draft's fp64 flops, and the shader clock sampled
    from sysfs during the timed layers;
  * phase-isolated maps (the same kept-pair count, all at one precision) for 128-token blocks, so
    each precision's MFMA utilisation is seen alone;
  * the dense baseline (no skipped pair, all 16-bit) for 128-token blocks, and the speedup of the
    workload's own quota over it, per attention call and per layer.
With --fp4 nvfp4 the 4-bit level runs in NVFP4: the sweep then takes only the workloads with 4-bit
pairs, their own quota and the 4-bit isolated map.

A step is one pass of the whole path over one batch of synthetic input, inputs resident in HBM:
dap_prepare -> dap_draft_rank -> dap_attention -> dap_restore.  Prints one JSON line:
  value         ms per layer (wall clock over K steps, synchronised on both sides)
  roofline      the attention kernel against the precision-weighted MFMA roofline: algorithmic
                flops per launch (4*B^2*D per kept block pair) over its average duration from
                HIP events on the launch stream; peak = flops / T_roof with T_roof the time every
                kept pair would take at the dense peak of its own precisions (bf16 2.5 PF/s;
                int8 and fp8 5.0 P/s; fp4 10.1 PF/s; NVFP4's Q.K^T, run as exact bf16, at 2.5);
                frac_at_sampled_sclk rescales the peaks (quoted at 2.4 GHz) to the median shader
                clock sampled from sysfs during the timed steps (the "sclk" object)
  cpu_baseline  the CPU oracle on a bounded sample of the same workload (a process pool over heads,
                one worker per core), extrapolated to a layer
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2.5e15, "i8": 5.0e15, "fp8": 5.0e15, "fp4": 10.1e15}
DEFAULT_WORKLOAD = "hunyuan720p_33x45x80"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_hbm_traffic.txt")


def roofline_terms(L: dict, heads_total: int, D: int, fp4: str = "mxfp4"):
    """(algorithmic flops, T_roof seconds) of the attention kernel for one layer.  NVFP4's Q.K^T
    is priced at the bf16 peak: its E4M3 group scales are not powers of two, so the scaled fp4
    MFMA (E8M0 scales only) cannot take them and the kernel contracts the exact bf16 values."""
    B = L["B"]
    n16 = L["c16"]
    n8 = L["c8"] - L["c16"]
    n4 = L["c4"] - L["c8"]
    half = 2.0 * B * B * D  # one of the two contractions of a block pair
    flops = heads_total * (n16 + n8 + n4) * 2 * half
    t_roof = heads_total * (n16 * (2 * half / PEAK["bf16"]) +
                            n8 * (half / PEAK["i8"] + half / PEAK["fp8"]) +
                            n4 * (half / PEAK["bf16" if fp4 == "nvfp4" else "fp4"] +
                                  half / PEAK["fp8"]))
    return flops, t_roof, (n16, n8, n4)


def source_digest() -> str:
    p = os.path.join(ROOT, "video_dit_mixed_amd", "csrc", "dap_attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def parse_traffic(text: str, workload: str, digest: str):
    """HBM bytes per attention launch from the text of a counter summary, if it was taken on the
    kernel source with this digest for this workload; else None."""
    kv = {}
    for line in text.splitlines():
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("workload") != workload or kv.get("source_sha256_16") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, if it was taken on the
    current kernel source for this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    return parse_traffic(open(TRAFFIC_FILE).read(), workload, source_digest())


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline_head(args):
    """Pool worker: the oracle on one head of the workload -- every step before attention, then
    attention over query blocks in a seeded random order until `budget_s` has passed.  Returns
    (head, prepare seconds, attention seconds, blocks done, Nb)."""
    from oracle import pipeline as opipe
    from video_dit_mixed_amd import synth
    w, bh, budget_s, blas_threads = args
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(blas_threads)
    except Exception:  # pragma: no cover
        limit = None
    q, k, v = synth.make_head(w, bh)
    t0 = time.perf_counter()
    r = opipe.prepare_head(q, k, v, T=w.T, H=w.H, W=w.W, rh=w.region_h, rw=w.region_w,
                           lam=w.lam, quota_bp=w.quota_bp)
    t_prep = time.perf_counter() - t0
    Nb = r.g.Nb
    order = np.random.default_rng([7, bh]).permutation(Nb)
    done = 0
    t1 = time.perf_counter()
    while done < Nb and (time.perf_counter() - t1) < budget_s:
        opipe.attend(r, q_blocks=[int(order[done])])
        done += 1
    t_att = time.perf_counter() - t1
    del limit
    return bh, t_prep, t_att, done, Nb


class CpuBaseline:
    """The CPU oracle timed on this host's cores: a process pool over heads (heads are independent
    and carry equal work), one worker per core the process may run on (up to the head count),
    BLAS threads split between the workers.  The pool is forked when the object is made, which
    must happen before the GPU is touched, so the workers are plain CPU processes."""

    def __init__(self, w, budget_s: float = 12.0):
        import multiprocessing as mp
        self.w = w
        self.budget_s = budget_s
        self.cores = len(os.sched_getaffinity(0))
        heads = w.batch * w.heads
        self.workers = max(1, min(self.cores, heads))
        self.blas = max(1, self.cores // self.workers)
        self.pool = mp.get_context("fork").Pool(self.workers)

    def run(self):
        w = self.w
        heads = w.batch * w.heads
        sample = list(range(self.workers))          # one head per worker, all at once
        t0 = time.perf_counter()
        res = self.pool.map(_cpu_baseline_head,
                            [(w, bh, self.budget_s, self.blas) for bh in sample], chunksize=1)
        wall = time.perf_counter() - t0
        self.pool.close()
        self.pool.join()
        full = [tp + ta * nb / max(done, 1) for _, tp, ta, done, nb in res]
        rounds = -(-heads // self.workers)
        per_layer_s = rounds * statistics.mean(full)
        done = [d for _, _, _, d, _ in res]
        nb = res[0][4]
        return {"value": round(per_layer_s * 1e3, 1), "unit": "ms/layer", "cores": self.cores,
                "kind": "oracle", "cpu_model": _cpu_model(), "workers": self.workers,
                "blas_threads_per_worker": self.blas, "heads_sampled": len(sample),
                "sample": f"{len(sample)} of {heads} heads in parallel (one per worker): every "
                          f"step before attention in full ({statistics.mean([r[1] for r in res]):.1f} s "
                          f"per head) and {min(done)}-{max(done)} of {nb} query blocks through "
                          f"attention ({self.budget_s:.0f} s budget); per head extrapolated "
                          f"linearly to {nb} blocks, per layer x {rounds} rounds of "
                          f"{self.workers} heads; {wall:.0f} s wall for the sample"}


# ------------------------------------------------------------------------------------------ sweep
HBM_PEAK = 8.0e12
FP64_PEAK = 78.6e12


def algorithmic_bytes(L: dict, w):
    """HBM bytes the method must move, per layer (the layout's sizes, every head):
    prepare reads Q, K, V and writes the packed bf16 copies, int8 Q/K with per-block scales,
    MXFP4 Q/K with E8M0 scales, fp8 V^T, the four pooled fp64 descriptors, then reads V once
    more for the per-channel amax; restore reads the packed output and writes the token-order one;
    the draft scores are the fp64 [Nb, Nb] map per head."""
    heads = w.batch * w.heads
    N, Np, Nb, D = w.N, L["Np"], L["Nb"], w.head_dim
    prep = heads * (3 * N * D * 2 + 3 * Np * D * 2 + 2 * Np * D + 2 * Nb * 4 +
                    2 * (Np * D // 2 + Np * D // 32) + Np * D + D * 4 + 4 * Nb * D * 8 +
                    N * D * 2)
    restore = heads * (Np * D * 2 + N * D * 2)
    draft_flops = heads * 4.0 * Nb * Nb * D
    score_bytes = heads * Nb * Nb * 8
    return prep, restore, draft_flops, score_bytes


class SclkSampler(threading.Thread):
    """Samples the GPU shader clock from sysfs while a timed region runs (amdgpu exposes the
    current SCLK as hwmon freq1_input in Hz; pp_dpm_sclk marks the active level with '*').
    Best effort: reports nothing where neither file is readable."""

    def __init__(self, period_s: float = 0.02):
        super().__init__(daemon=True)
        self.period = period_s
        self.samples = {}
        self._halt = threading.Event()
        self.sources = self._find()

    @staticmethod
    def _find():
        import glob
        out = []
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                if open(os.path.join(dev, "vendor")).read().strip() != "0x1002":
                    continue
            except OSError:
                continue
            for f in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "freq1_input"))):
                out.append((dev, "hwmon", f))
            p = os.path.join(dev, "pp_dpm_sclk")
            if os.path.exists(p):
                out.append((dev, "dpm", p))
        return out

    def _read(self, kind, path):
        txt = open(path).read()
        if kind == "hwmon":
            return int(txt.strip()) / 1e6
        for line in txt.splitlines():
            if line.rstrip().endswith("*"):
                tok = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                return float(tok.replace("mhz", ""))
        return None

    def run(self):
        if not self.sources:
            self._run_smi()
            return
        while not self._halt.is_set():
            for dev, kind, path in self.sources:
                try:
                    v = self._read(kind, path)
                except (OSError, ValueError, IndexError):
                    v = None
                if v is not None:
                    self.samples.setdefault((dev, kind), []).append(v)
            self._halt.wait(self.period)

    def _run_smi(self):
        """Fallback where sysfs is not readable: poll `rocm-smi --showclocks`."""
        import re
        import subprocess
        pat = re.compile(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", re.I)
        while not self._halt.is_set():
            try:
                txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                     timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            for m in pat.finditer(txt):
                self.samples.setdefault(("rocm-smi", "showclocks"), []).append(float(m.group(1)))
            self._halt.wait(self.period * 10)

    def stop(self):
        self._halt.set()
        self.join(timeout=2)
        # the card under load is the one with the highest median clock
        best = None
        for (dev, kind), xs in self.samples.items():
            med = statistics.median(xs)
            if best is None or med > best["median_mhz"]:
                best = {"median_mhz": round(med, 1), "min_mhz": round(min(xs), 1),
                        "max_mhz": round(max(xs), 1), "samples": len(xs),
                        "source": f"{os.path.basename(os.path.dirname(dev)) or dev} {kind}"}
        return best


def time_layers(b, cfg, q, k, v, ws, out, warmup: int, reps: int, stream):
    """HIP events around each of the four calls for `reps` layers after `warmup` untimed ones.
    Returns per-call lists (ms) and the per-layer sums."""
    import torch
    calls = [lambda: b.prepare(cfg, q, k, v, ws), lambda: b.draft_rank(cfg, ws),
             lambda: b.attention(cfg, ws), lambda: b.restore(cfg, ws, out)]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    sampler = SclkSampler()
    sampler.start()
    for i in range(reps):
        evs[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    sclk = sampler.stop()
    names = ["prepare", "draft_rank", "attention", "restore"]
    per = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
    per["layer"] = [e[0].elapsed_time(e[4]) for e in evs]
    return per, sclk


def measure_case(b, w, quota, q, k, v, dev, warmup, reps, stream, label):
    import torch
    cfg = b.Config.from_workload(w, quota_bp=tuple(quota))
    L = b.workspace_layout(cfg)
    ws = b.alloc_workspace(cfg, dev)
    out = torch.empty_like(q)
    per, sclk = time_layers(b, cfg, q, k, v, ws, out, warmup, reps, stream)
    del ws, out
    torch.cuda.empty_cache()
    heads = w.batch * w.heads
    flops, t_roof, (n16, n8, n4) = roofline_terms(L, heads, w.head_dim, w.fp4)
    med = {n: statistics.median(x) for n, x in per.items()}
    mn = {n: min(x) for n, x in per.items()}
    prep_b, rest_b, dflops, sbytes = algorithmic_bytes(L, w)
    real = (w.N / L["Np"]) ** 2
    t_attn = med["attention"] * 1e-3
    r = {"case": label, "workload": w.name, "fp4": w.fp4, "quota_bp_skip_4_8_16": list(quota), "reps": reps,
         "warmup": warmup, "B": L["B"], "Nb": L["Nb"], "Np": L["Np"], "N": w.N,
         "kept_pairs_per_head_16_8_4": [n16, n8, n4],
         "median_ms": {n: round(x, 4) for n, x in med.items()},
         "min_ms": {n: round(x, 4) for n, x in mn.items()},
         "ms_per_layer": round(med["layer"], 4),
         "t_roof_ms": round(t_roof * 1e3, 4),
         "t_roof_over_t_attn": round(t_roof / t_attn, 4) if t_attn > 0 else None,
         "t_roof_over_t_attn_real_tokens": round(real * t_roof / t_attn, 4) if t_attn > 0 else None,
         "real_token_share": round(real, 4),
         "t_roof_over_layer": round(t_roof * 1e3 / med["layer"], 4),
         "attn_tflops": round(flops / t_attn / 1e12, 2) if t_attn > 0 else None,
         "prepare_gbs": round(prep_b / (med["prepare"] * 1e-3) / 1e9, 1),
         "prepare_frac_hbm": round(prep_b / (med["prepare"] * 1e-3) / HBM_PEAK, 4),
         "restore_gbs": round(rest_b / (med["restore"] * 1e-3) / 1e9, 1),
         "restore_frac_hbm": round(rest_b / (med["restore"] * 1e-3) / HBM_PEAK, 4),
         "draft_rank_fp64_tflops": round(dflops / (med["draft_rank"] * 1e-3) / 1e12, 3),
         "draft_rank_score_gbs": round(sbytes / (med["draft_rank"] * 1e-3) / 1e9, 1),
         "algorithmic_bytes": {"prepare": prep_b, "restore": rest_b, "scores": sbytes},
         "draft_fp64_flops": dflops, "sclk": sclk}
    if sclk and sclk.get("median_mhz"):
        r["t_roof_over_t_attn_at_sclk"] = round(t_roof * 2400.0 / sclk["median_mhz"] / t_attn, 4)
    return r


def sweep(args):
    import torch
    from video_dit_mixed_amd import binding as b
    from video_dit_mixed_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    names = args.workloads.split(",") if args.workloads else list(synth.ORDER)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    sink = open(args.out, "w") if args.out else None

    def emit(r):
        rows.append(r)
        line = json.dumps(r)
        print(line, flush=True)
        if sink:
            sink.write(line + "\n")
            sink.flush()

    for name in names:
        w = synth.workload(name).with_(fp4=args.fp4)
        if args.fp4 == "nvfp4" and w.quota_bp[1] == 0:
            continue  # no 4-bit pair in this workload: NVFP4 changes nothing
        reps = args.reps if args.reps else (5 if w.N > 200_000 else 20)
        print(f"# {name}: generating inputs", flush=True)
        Q, K, V = synth.make_inputs(w, threads=16)
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = to(Q), to(K), to(V)
        del Q, K, V
        base = measure_case(b, w, w.quota_bp, q, k, v, dev, args.warmup, reps, stream, "own")
        emit(base)
        kept = 10000 - w.quota_bp[0]
        if base["B"] == 128 and not args.own_only:
            levels = (("16", (w.quota_bp[0], 0, 0, kept)), ("8", (w.quota_bp[0], 0, kept, 0)),
                      ("4", (w.quota_bp[0], kept, 0, 0)))
            if args.fp4 == "nvfp4":
                levels = levels[2:]  # only the 4-bit level differs from the MXFP4 sweep
            for lvl, quota in levels:
                emit(measure_case(b, w, quota, q, k, v, dev, args.warmup, reps, stream,
                                  f"isolated_{lvl}bit"))
            if args.fp4 != "nvfp4":
                dense = measure_case(b, w, (0, 0, 0, 10000), q, k, v, dev, args.warmup, reps,
                                     stream, "dense_16bit")
                dense["speedup_attention"] = round(dense["median_ms"]["attention"] /
                                                   base["median_ms"]["attention"], 3)
                dense["speedup_layer"] = round(dense["ms_per_layer"] / base["ms_per_layer"], 3)
                emit(dense)
        del q, k, v
        torch.cuda.empty_cache()
    if sink:
        sink.close()


def lds_feed() -> int:
    """Runs the stand-alone matrix-core / LDS timing program that build() compiles next to
    libdap.so; it must have been built (no compilation happens here)."""
    import subprocess
    from video_dit_mixed_amd import build as bld
    if not os.path.exists(bld.LDS_FEED_BENCH):
        print(f"{bld.LDS_FEED_BENCH} is not built: run __graft_entry__.build() first", file=sys.stderr)
        return 1
    return subprocess.run([bld.LDS_FEED_BENCH]).returncode


def section_clocks(w) -> dict:
    """One attention launch of the section-clock diagnostic after two plain ones: per precision
    phase, the cycles per wave-block and the share of each part of the key-block loop (the
    clocked instance reads the shader clock, so its launch is a few per cent slower)."""
    import torch
    from video_dit_mixed_amd import binding as b
    from video_dit_mixed_amd import synth
    cfg = b.Config.from_workload(w)
    dev = torch.device("cuda:0")
    Q, K, V = synth.make_inputs(w, threads=16)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(Q), to(K), to(V)
    del Q, K, V
    ws = b.alloc_workspace(cfg, dev)
    b.prepare(cfg, q, k, v, ws)
    b.draft_rank(cfg, ws)
    for _ in range(2):
        b.attention(cfg, ws)
    clk = torch.zeros(b.SECTION_CLOCK_WORDS, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    b.attention_section_clocks(cfg, ws, clk, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    c = clk.cpu().numpy().astype(np.uint64).astype(np.float64).reshape(4, 8)
    names = ("16-bit", "8-bit", "4-bit MXFP4", "4-bit NVFP4")
    phases = {}
    for p in range(4):
        if c[p, 6] == 0:
            continue
        tot = c[p, :6].sum()
        phases[names[p]] = {"wave_blocks": int(c[p, 6]),
                            "cycles_per_wave_block": round(tot / c[p, 6], 1),
                            "share_of_wave_cycles": round(tot / c[0, 7], 4),
                            **{n: round(c[p, i] / tot, 4) for i, n in enumerate(b.SECTION_CLOCK_PARTS)}}
    return {"section_clocks": {"workload": w.name, "quota_bp": list(w.quota_bp), "fp4": w.fp4,
                               "clocked_launch_ms": round(e0.elapsed_time(e1), 3), "phases": phases}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quota", default=None,
                    help="override the workload's quotas: skip,4-bit,8-bit,16-bit in basis points "
                         "(for per-phase counter runs; the traffic figure is then not reported)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (a kernel of known "
                         "read/write size for scaling HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="measure every workload: own quota, phase-isolated maps, dense baseline")
    ap.add_argument("--workloads", default=None, help="comma-separated workloads for --sweep")
    ap.add_argument("--reps", type=int, default=0, help="timed layers per --sweep case")
    ap.add_argument("--own-only", action="store_true", help="--sweep: only each workload's quota")
    ap.add_argument("--out", default=None, help="--sweep: also write the JSON lines here")
    ap.add_argument("--fp4", choices=["mxfp4", "nvfp4"], default="mxfp4",
                    help="4-bit operand format (NVFP4: the pages' example format; MXFP4 default)")
    ap.add_argument("--lds-feed", action="store_true",
                    help="run the built lds_feed_bench program instead (matrix-core products fed "
                         "from LDS, one workgroup per compute unit) and print its JSON lines")
    ap.add_argument("--section-clocks", action="store_true",
                    help="instead of timing, run dap_attention_section_clocks once on the workload "
                         "(and --quota / --fp4) and print where the attention waves spend their cycles")
    args = ap.parse_args()
    if args.lds_feed:
        sys.exit(lds_feed())
    if args.gpus != 1:
        print(f"bench.py measures one GPU (got --gpus {args.gpus}): the operator shards by heads "
              f"with no communication inside it, and the multi-GPU path is not implemented.",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return

    import torch
    from video_dit_mixed_amd import binding as b
    from video_dit_mixed_amd import synth

    w = synth.workload(args.workload).with_(fp4=args.fp4)
    if args.quota:
        w = w.with_(quota_bp=tuple(int(x) for x in args.quota.split(",")))
    if args.section_clocks:
        print(json.dumps(section_clocks(w)), flush=True)
        return
    # the CPU baseline's workers are forked now, before anything touches the GPU
    cpu = None if args.no_cpu_baseline else CpuBaseline(w)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = b.Config.from_workload(w)
    L = b.workspace_layout(cfg)
    t_gen = time.perf_counter()
    Q, K, V = synth.make_inputs(w, threads=16)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(Q), to(K), to(V)
    ws = b.alloc_workspace(cfg, dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        b.prepare(cfg, q, k, v, ws)
        if ev is not None:
            ev[1].record(stream)
        b.draft_rank(cfg, ws)
        if ev is not None:
            ev[2].record(stream)
        b.attention(cfg, ws)
        if ev is not None:
            ev[3].record(stream)
        b.restore(cfg, ws, out)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    sampler = SclkSampler()
    sampler.start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = sampler.stop()
    ms_per_step = wall * 1e3 / args.steps
    names = ["prepare", "draft_rank", "attention", "restore"]
    per = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
    med = {n: statistics.median(v) for n, v in per.items()}

    heads_total = w.batch * w.heads
    flops, t_roof, (n16, n8, n4) = roofline_terms(L, heads_total, w.head_dim, w.fp4)
    t_attn = statistics.mean(per["attention"]) * 1e-3
    achieved = flops / t_attn
    peak = flops / t_roof
    traffic = read_traffic(w.name) if not args.quota and args.fp4 == "mxfp4" else None
    fp4_name = "nvfp4(bf16 mfma)+fp8" if w.fp4 == "nvfp4" else "mxfp4+fp8"
    dtype = "/".join(x for x, n in (("bf16", n16), ("i8+fp8", n8), (fp4_name, n4)) if n > 0)

    res = {
        "metric": "ms/layer + % precision-weighted MFMA roofline, mixed-precision draft attn",
        "value": round(ms_per_step, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded blob+noise+outlier-channel Q/K, N(0,1) V)",
        "config": {"workload": w.name, "fp4": w.fp4, "batch": w.batch, "tokens": w.N,
                   "latent": [w.T, w.H, w.W],
                   "heads": w.heads, "head_dim": w.head_dim,
                   "region": [w.region_h, w.region_w], "lambda": w.lam,
                   "quota_bp_skip_4_8_16": list(w.quota_bp), "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2),
                     "peak": round(peak / 1e12, 2), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel": "attn_kernel",
                     "t_roof_ms": round(t_roof * 1e3, 4),
                     "kept_pairs_per_head_16_8_4": [n16, n8, n4]},
        "sclk": sclk,
        "breakdown_ms_median": {n: round(v, 4) for n, v in med.items()},
        "t_roof_over_layer_ms": round(t_roof * 1e3 / ms_per_step, 4),
        "input_gen_s": round(t_gen, 1),
    }
    if sclk and sclk.get("median_mhz"):
        # the same fraction with the peaks scaled to the shader clock held during the timed steps
        res["roofline"]["frac_at_sampled_sclk"] = round(achieved / peak * 2400.0 / sclk["median_mhz"], 4)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 1 << 30
    if cpu is not None:
        del Q, K, V
        res["cpu_baseline"] = cpu.run()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
