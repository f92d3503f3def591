"""Benchmark of the verify/accept step on one MI355X.

One step = one verify pass over the workload b=128, K=7, V=262144, bf16
logits: sequences 0..63 greedy, 64..127 speculative sampling at T=0.8
(target block [128, 8, V], draft block [128, 7, V], draft tokens, seeds,
all resident in HBM).  By default the step is ONE mixed-rule call
(spec_mixed_accept, per-sequence temperature 0 or 0.8); `--step split` runs
it as a greedy call over 0..63 plus a sampling call over 64..127 on the same
stream.  Inputs rotate over several device copies so no step reads bytes a
previous step left in the 256 MB last-level cache.

Timed regions (HIP events on the call stream, synchronised on both sides):
  1. `--steps` steps, nothing else recorded: the headline value;
  2. the same steps with the library's stage events recorded around every
     kernel: per-kernel times and the row pass's achieved HBM bandwidth;
  3. (mixed) the same steps as split calls, for reference.
Then the CPU oracle is timed on a bounded sample of the same workload.

Prints one JSON line.  Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--step mixed|split]
  python bench.py --copy-calibration BYTES   (rocprof counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
SEG_BYTES = 16384          # one row-pass segment (the bonus draw re-reads one)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(step, seconds: float, chunk: int = 50):
    """Run `step` in chunks of untimed calls until `seconds` of wall time have
    passed (the GPU's clocks ramp up under sustained load, whatever the
    warm-up count).  Returns (wall seconds, steps run)."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while True:
        for _ in range(chunk):
            step(k)
            k += 1
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            return el, k


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def source_digest() -> str:
    """sha256[:16] over every kernel source file (sorted by name)."""
    d = os.path.join(ROOT, "lossless_draft_verification_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".inc")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, valid
    only while the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel, {}).get(workload)
    if not ent or ent.get("source_sha256_16") != source_digest():
        return None
    return ent.get("bytes_per_launch")


def markov_loop_traffic(K: int):
    """HBM bytes of the Markov position loop (K correction and select
    launches) from the counters of one launch of each, or None."""
    a = load_traffic("markov_stream", "markov_b128_V262144_r256")
    c = load_traffic("draft_select", "markov_b128_V262144_r256")
    return None if a is None or c is None else K * (a + c)


def cpu_baseline(case, greedy_idx, sample_idx, budget_s: float):
    """Time the CPU oracle (single thread) on whole sequences of the workload,
    alternating greedy and sampling sequences until the budget is spent."""
    import oracle
    orc = oracle.default()
    tg = ts = 0.0
    ng = ns = 0
    t_begin = time.perf_counter()
    k = 0
    while k == 0 or (time.perf_counter() - t_begin < budget_s and k < min(len(greedy_idx), len(sample_idx))):
        g = case.take([greedy_idx[k]])
        t0 = time.perf_counter()
        orc.greedy_accept(g.target, g.draft_tokens)
        tg += time.perf_counter() - t0
        ng += 1
        s = case.take([sample_idx[k]])
        t0 = time.perf_counter()
        orc.sample_accept(s.target, s.draft, s.draft_tokens, s.T, s.seeds)
        ts += time.perf_counter() - t0
        ns += 1
        k += 1
    per_block = 0.5 * (tg / ng) + 0.5 * (ts / ns)
    return {
        "value": 1.0 / per_block, "unit": "verify blocks/s", "cores": 1, "kind": "oracle",
        "sample": f"{ng} greedy + {ns} sampling sequences of the same workload, whole sequences, "
                  f"mixed 50/50 as in the workload (single-threaded C oracle in double precision, "
                  f"gcc -O2): greedy {tg / ng * 1e3:.1f} ms/seq, sampling {ts / ns * 1e3:.1f} ms/seq; "
                  f"host CPU: {cpu_model()}, {os.cpu_count()} logical CPUs visible",
    }


KERNEL_KEYS = {"row_pass_listed": "row_pass", "row_pass": "row_pass", "scan_kernel": "scan",
               "residual_kernel": "residual_mass",
               "draw_kernel": "draw_token", "stream_copy_kernel": "stream_copy",
               "lm_head_dl_kernel": "lm_head_gemm", "markov_stream_kernel": "markov_stream",
               "draft_select_kernel": "draft_select"}

# Counter passes over the other bench modes: (-o prefix, kernels, workload key,
# profile file the counters are appended to, bench arguments).
EXTRA_PMC = [
    ("fused", ("lm_head_gemm",), "fused_b128_V262144_D3840", "lm_head_fused_verify_b128_V262144_D3840.md",
     "--fused --steps 2 --warmup 1 --no-cpu-baseline --no-reference"),
    ("markov", ("markov_stream", "draft_select"), "markov_b128_V262144_r256",
     "markov_block_decode_b128_V262144_r256.md", "--markov --steps 2 --warmup 1 --no-cpu-baseline"),
    ("ragged", ("row_pass",), "c5_mixed_ragged", "verify_c5_ragged.md",
     "--ragged --steps 3 --warmup 1 --no-cpu-baseline --no-reference"),
    ("sharded", ("row_pass",), "c5_mixed_sharded8", "verify_c5_vocab_sharded8.md",
     "--sharded 8 --steps 3 --warmup 1 --no-cpu-baseline --no-reference"),
]


def _short(name: str) -> str:
    for k, v in KERNEL_KEYS.items():
        if k in name:
            return v
    return name.split("(")[0][-40:]


def summarize_rocprof(rdir: str, workload: str = "c5_mixed", nbytes_copy: int = 536870912, out_dir: str = "") -> int:
    """Turn rocprofv3 CSV output (a kernel trace and --pmc FETCH_SIZE /
    WRITE_SIZE passes over the bench and over --copy-calibration, written
    under `rdir` by the commands listed in the summary) into
    profiles/verify_c5_mixed.md and profiles/traffic.json."""
    import csv
    import statistics
    prof = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    tr = os.path.join(rdir, "prof", "mixed_c5_kernel_trace.csv")
    rows = list(csv.DictReader(open(tr)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = {}
    for r in rows:
        k = _short(r["Kernel_Name"])
        dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counter(path):
        out = {}
        for r in csv.DictReader(open(path)):
            out.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return out

    pmc = os.path.join(rdir, "pmc")
    fb, wb = (counter(os.path.join(pmc, f"bench_{c}_counter_collection.csv")) for c in ("FETCH_SIZE", "WRITE_SIZE"))
    fc, wc = (counter(os.path.join(pmc, f"copy_{c}_counter_collection.csv")) for c in ("FETCH_SIZE", "WRITE_SIZE"))
    kib = nbytes_copy / 1024.0
    f_scale = kib / statistics.median(fc["stream_copy"])
    w_scale = kib / statistics.median(wc["stream_copy"])
    digest = source_digest()
    lines = ["# Kernel durations and HBM traffic: verify step, workload c5 (mixed call)", "",
             "b=128, K=7, V=262144, bf16; sequences 0..63 greedy, 64..127 sampling at T=0.8, one",
             "spec_mixed_accept call per step.  Kernel source sha256[:16] = `%s`." % digest, "",
             "Commands (run from /tmp, repository at $R, rocprofv3 output under $OUT):", "",
             "    rocprofv3 --kernel-trace --stats -d $OUT/prof -o mixed_c5 --output-format csv \\",
             "        -- python3 $R/bench.py --steps 200 --warmup 1000 --no-cpu-baseline --no-reference",
             "    rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc -o bench_FETCH_SIZE --output-format csv \\",
             "        -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-reference",
             "    rocprofv3 --pmc WRITE_SIZE  (same, -o bench_WRITE_SIZE)",
             "    rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc -o copy_FETCH_SIZE --output-format csv \\",
             "        -- python3 $R/bench.py --copy-calibration %d" % nbytes_copy,
             "    rocprofv3 --pmc WRITE_SIZE  (same, -o copy_WRITE_SIZE)",
             "    python bench.py --summarize-rocprof $OUT            # writes this file", "",
             "## Kernel trace (rocprofv3 --kernel-trace), last 200 steps", "",
             "| kernel | launches | median us | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for k, v in dur.items():
        if k not in KERNEL_KEYS.values():
            continue
        v = v[-200:]
        lines.append(f"| {k} | {len(v)} | {statistics.median(v):.2f} | {statistics.mean(v):.2f} | "
                     f"{min(v):.2f} | {max(v):.2f} |")
    lines += ["", "## Counters (rocprofv3 --pmc, one counter per run), KiB per dispatch", "",
              f"Calibration: spec_stream_copy of {nbytes_copy} bytes reads FETCH_SIZE "
              f"{statistics.median(fc['stream_copy']):.0f} KiB and WRITE_SIZE "
              f"{statistics.median(wc['stream_copy']):.0f} KiB for {kib:.0f} KiB moved each way, so "
              f"FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}.", "",
              "| kernel | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | HBM bytes per launch (scaled) |",
              "|---|---|---|---|"]
    traffic = {}
    for k in fb:
        if k not in ("row_pass", "scan", "residual_mass", "draw_token"):
            continue
        f_med, w_med = statistics.median(fb[k]), statistics.median(wb.get(k, [0.0]))
        byts = (f_med * f_scale + w_med * w_scale) * 1024.0
        traffic[k] = {workload: {"bytes_per_launch": byts, "fetch_kib": f_med, "write_kib": w_med,
                                 "fetch_scale": f_scale, "write_scale": w_scale, "source_sha256_16": digest}}
        lines.append(f"| {k} | {f_med:.0f} | {w_med:.0f} | {byts:.0f} |")
    lines += ["", "Algorithmic bytes of the row pass per launch: 771751936 (every logit read once).", ""]
    lines += residual_counter_section(pmc)
    with open(os.path.join(prof, "verify_c5_mixed.md"), "w") as f:
        f.write("\n".join(lines))
    # the fused and Markov paths' kernels, appended to their trace summaries
    for mode, keys, wl, fname, bargs in EXTRA_PMC:
        fp, wp = (os.path.join(pmc, f"{mode}_{c}_counter_collection.csv") for c in ("FETCH_SIZE", "WRITE_SIZE"))
        if not (os.path.exists(fp) and os.path.exists(wp)):
            continue
        fm, wm = counter(fp), counter(wp)
        sec = ["", f"## Counters of the `{bargs.split()[0]}` bench (rocprofv3 --pmc, one counter per run), "
                   "KiB per dispatch", "",
               "Commands (scaled as in verify_c5_mixed.md: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f):" % (f_scale, w_scale),
               "",
               f"    rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc -o {mode}_FETCH_SIZE --output-format csv \\",
               f"        -- python3 $R/bench.py {bargs}",
               f"    rocprofv3 --pmc WRITE_SIZE  (same, -o {mode}_WRITE_SIZE)", "",
               "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | HBM bytes per dispatch (scaled) |",
               "|---|---|---|---|---|"]
        for k in keys:
            if k not in fm:
                continue
            f_med, w_med = statistics.median(fm[k]), statistics.median(wm.get(k, [0.0]))
            byts = (f_med * f_scale + w_med * w_scale) * 1024.0
            traffic.setdefault(k, {})[wl] = {"bytes_per_launch": byts, "fetch_kib": f_med, "write_kib": w_med,
                                             "fetch_scale": f_scale, "write_scale": w_scale,
                                             "source_sha256_16": digest}
            sec.append(f"| {k} | {len(fm[k])} | {f_med:.0f} | {w_med:.0f} | {byts:.0f} |")
        with open(os.path.join(prof, fname), "a") as f:
            f.write("\n".join(sec) + "\n")
    gemm = gemm_counter_section(pmc)
    if gemm:
        with open(os.path.join(prof, "lm_head_fused_verify_b128_V262144_D3840.md"), "a") as f:
            f.write("\n".join(gemm) + "\n")
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print("\n".join(lines))
    return 0


# Instruction and cycle counters of the residual pass (two rocprofv3 --pmc
# passes, at most eight SQ counters each, over residual_kernel only).
RES_PMC = [
    ("res_sqA", "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES "
                "SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD"),
    ("res_sqB", "SQ_THREAD_CYCLES_VALU SQ_ACTIVE_INST_ANY SQ_INSTS_SALU SQ_INSTS_SMEM SQ_ACTIVE_INST_VMEM "
                "SQ_ACTIVE_INST_SCA SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_ADD_F32 GRBM_GUI_ACTIVE"),
]


def residual_counter_section(pmc: str) -> list:
    """Markdown lines for the residual pass's SQ counters (median over the
    dispatches of each counter, summed over the chip), or [] if the passes
    are absent."""
    import csv
    import statistics
    vals = {}
    for prefix, _ in RES_PMC:
        path = os.path.join(pmc, f"{prefix}_counter_collection.csv")
        if not os.path.exists(path):
            return []
        per = {}
        for r in csv.DictReader(open(path)):
            if "residual_kernel" not in r["Kernel_Name"]:
                continue
            key = (r["Counter_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (name, _), v in per.items():
            vals.setdefault(name, []).append(v)
    med = {k: statistics.median(v) for k, v in vals.items()}
    g = med.get
    lines = ["## Residual pass: instruction and cycle counters (rocprofv3 --pmc), median per dispatch", "",
             "Commands (two passes; at most eight SQ counters fit in one):", ""]
    for prefix, ctrs in RES_PMC:
        lines += [f"    rocprofv3 --pmc {ctrs} \\",
                  f"        --kernel-include-regex residual_kernel -d $OUT/pmc -o {prefix} --output-format csv \\",
                  "        -- python3 $R/bench.py --steps 3 --warmup 1 --settle 0 --no-cpu-baseline --no-reference"]
    lines += ["", "| counter | value |", "|---|---|"]
    for k in sorted(med):
        lines.append(f"| {k} | {med[k]:.0f} |")
    pairs = 59 * 262144                      # element pairs of the 59 rejected row pairs of c5
    if g("SQ_INSTS_VALU") and g("SQ_WAVE_CYCLES"):
        lines += ["", "Derived (c5 rejects 59 row pairs of 262144 entries: 15.47M element pairs):", "",
                  f"- VALU instructions per element pair (wave instructions x 64 lanes / pairs): "
                  f"{g('SQ_INSTS_VALU') * 64 / pairs:.1f}, of which transcendental "
                  f"{g('SQ_INSTS_VALU_TRANS_F32', 0) * 64 / pairs:.2f}",
                  f"- share of resident wave-cycles issuing VALU (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES): "
                  f"{g('SQ_ACTIVE_INST_VALU', 0) / g('SQ_WAVE_CYCLES'):.2f}",
                  f"- share waiting on any instruction's dependency (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES): "
                  f"{g('SQ_WAIT_INST_ANY', 0) / g('SQ_WAVE_CYCLES'):.2f}",
                  f"- VALU issue cycles per SIMD (4 per wave64 instruction, 1024 SIMDs): "
                  f"{g('SQ_INSTS_VALU') * 4 / 1024:.0f}, that is "
                  f"{g('SQ_INSTS_VALU') * 4 / 1024 / 2.4e3:.2f} us at 2.4 GHz"]
    return lines + [""]


# Matrix-pipe and clock counters of the fused GEMM (one rocprofv3 --pmc pass
# over lm_head_dl_kernel), with its dispatches' own timestamps.
GEMM_PMC = ("gemm_sq", "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES")
GEMM_FLOPS = 2 * 1024 * 3840 * 262144          # b*(K+1) x D x V, two flops per product
XCDS, SIMDS, FLOPS_PER_SIMD_CYCLE, NOMINAL_GHZ = 8, 1024, 1024, 2.4


def gemm_counter_section(pmc: str) -> list:
    """Markdown lines for the fused GEMM's SQ/GRBM counters: per dispatch the
    clock (GRBM_GUI_ACTIVE summed over the XCDs / XCDs / duration) and the
    matrix pipe's busy share at that clock (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs
    over clock x duration); medians over the dispatches after the first
    third (the clock ramps over the first ones).  [] if the pass is absent."""
    import csv
    import statistics
    path = os.path.join(pmc, f"{GEMM_PMC[0]}_counter_collection.csv")
    if not os.path.exists(path):
        return []
    per = {}
    for r in csv.DictReader(open(path)):
        if "lm_head_dl_kernel" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [per[k] for k in sorted(per, key=int)]
    disp = [d for d in disp if d.get("GRBM_GUI_ACTIVE") and d.get("SQ_VALU_MFMA_BUSY_CYCLES") and d["dur"] > 0]
    if not disp:
        return []
    steady = disp[len(disp) // 3:]
    ghz = [d["GRBM_GUI_ACTIVE"] / XCDS / d["dur"] / 1e9 for d in steady]
    busy = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / (d["GRBM_GUI_ACTIVE"] / XCDS) for d in steady]
    dur = [d["dur"] * 1e3 for d in steady]
    ideal = GEMM_FLOPS / FLOPS_PER_SIMD_CYCLE
    mfma = statistics.median(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in steady)
    lines = ["", "## Matrix pipe and clock of the GEMM (rocprofv3 --pmc), dispatches after the first third", "",
             "Command:", "",
             f"    rocprofv3 --pmc {GEMM_PMC[1]} --kernel-include-regex lm_head_dl \\",
             f"        -d $OUT/pmc -o {GEMM_PMC[0]} --output-format csv \\",
             "        -- python3 $R/bench.py --fused --steps 2 --warmup 1 --settle 0 --no-cpu-baseline --no-reference", "",
             "| measure | median | range |", "|---|---|---|",
             f"| duration (ms) | {statistics.median(dur):.3f} | {min(dur):.3f}-{max(dur):.3f} |",
             f"| clock, GRBM_GUI_ACTIVE / {XCDS} XCDs / duration (GHz) | {statistics.median(ghz):.3f} | "
             f"{min(ghz):.3f}-{max(ghz):.3f} |",
             f"| matrix pipe busy at that clock | {statistics.median(busy):.3f} | {min(busy):.3f}-{max(busy):.3f} |",
             "",
             f"SQ_VALU_MFMA_BUSY_CYCLES reads {mfma:.0f} per dispatch; the product needs {ideal:.0f} SIMD-cycles "
             f"of v_mfma_f32_32x32x16_bf16 ({GEMM_FLOPS:.3e} flops at {FLOPS_PER_SIMD_CYCLE} per SIMD-cycle), so the "
             "counter is the matrix pipe's work itself. The same work at the nominal "
             f"{NOMINAL_GHZ} GHz is the {NOMINAL_GHZ * FLOPS_PER_SIMD_CYCLE * SIMDS / 1e3:.0f} TFLOP/s bf16 peak.", ""]
    return lines


TRACE_SUMMARIES = [
    # (trace dir, -o prefix, profile file, title, workload text, bench arguments)
    ("prof_fused", "fused", "lm_head_fused_verify_b128_V262144_D3840.md",
     "Kernel durations: fused lm_head + verify",
     "b=128, K=7, V=262144, D=3840, bf16 hidden states and lm_head weight, softcap 30, float32 drafter "
     "logits; sequences 0..63 greedy, 64..127 sampled at T=0.8; one spec_fused_mixed_accept call per step.",
     "--fused --steps 50 --warmup 5 --no-cpu-baseline --no-reference"),
    ("prof_markov", "markov", "markov_block_decode_b128_V262144_r256.md",
     "Kernel durations: draft-side Markov block decode",
     "b=128, K=7, V=262144, r=256, D=3840; float32 base logits, bf16 Markov tables, confidence head; "
     "sequences 0..63 greedy, 64..127 sampled at T=0.8; one spec_markov_block_decode call per step "
     "(7 positions: the streaming correction kernel and the per-sequence select kernel each).",
     "--markov --steps 30 --warmup 3 --no-cpu-baseline"),
    ("prof_ragged", "ragged", "verify_c5_ragged.md",
     "Kernel durations: verify step with per-sequence draft lengths",
     "workload c5 (b=128, K=7, V=262144, bf16, 64 greedy + 64 sampled) with draft lengths drawn uniformly "
     "from 0..7, one spec_mixed_accept call per step (the listed row pass streams only rows inside each "
     "block).",
     "--ragged --steps 200 --warmup 200 --no-cpu-baseline --no-reference"),
    ("prof_sharded", "sharded", "verify_c5_vocab_sharded8.md",
     "Kernel durations: vocabulary-sharded verify, 8 shards",
     "workload c5 (b=128, K=7, V=262144, bf16, 64 greedy + 64 sampled) with the vocabulary in 8 shards of "
     "32768 columns, one spec_sharded_mixed_accept call per step.",
     "--sharded 8 --steps 200 --warmup 200 --no-cpu-baseline --no-reference"),
]


def summarize_traces(rdir: str, out_dir: str = "") -> None:
    """profiles/*.md summaries of the kernel traces of the fused, Markov and
    sharded paths (whichever are present under rdir)."""
    import csv
    digest = source_digest()
    for sub, prefix, fname, title, workload, bargs in TRACE_SUMMARIES:
        path = os.path.join(rdir, sub, f"{prefix}_kernel_stats.csv")
        if not os.path.exists(path):
            continue
        rows = list(csv.DictReader(open(path)))
        lines = [f"# {title}", "", workload, f"Kernel source sha256[:16] = `{digest}`.", "",
                 "Command (run from /tmp, repository at $R, rocprofv3 output under $OUT):", "",
                 f"    rocprofv3 --kernel-trace --stats -d $OUT/{sub} -o {prefix} --output-format csv \\",
                 f"        -- python3 $R/bench.py {bargs}",
                 "    python bench.py --summarize-rocprof $OUT            # writes this file", "",
                 "## rocprofv3 --stats (kernel stats), all launches of the run", "",
                 "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
        for r in rows:
            name = r["Name"]
            if "anonymous namespace" not in name:
                continue
            short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), fname), "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote profiles/{fname}")


def copy_calibration(nbytes: int) -> int:
    import torch
    import lossless_draft_verification_amd as L
    dev = torch.device("cuda:0")
    src = torch.full((nbytes // 4,), 1.0, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        L.stream_copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5,
                      "expected_fetch_bytes": nbytes, "expected_write_bytes": nbytes}), flush=True)
    return 0


def cpu_baseline_fused(case, budget_s: float):
    """Time the fused-verify oracle (numpy float64 lm_head GEMM + the C
    accept) on pairs of sequences (one greedy, one sampling) of the workload
    until the budget is spent."""
    import numpy as np
    import oracle.fused as OF
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = 1
    g_idx = np.nonzero(case.temps == 0.0)[0]
    s_idx = np.nonzero(case.temps > 0.0)[0]
    spent, blocks, k = 0.0, 0, 0
    while k == 0 or (spent < budget_s and k < min(len(g_idx), len(s_idx))):
        idx = [int(g_idx[k]), int(s_idx[k])]
        t0 = time.perf_counter()
        OF.fused_mixed_accept(case.hidden[idx], case.weight, case.softcap, case.draft[idx],
                              case.draft_tokens[idx], case.temps[idx], case.seeds[idx])
        spent += time.perf_counter() - t0
        blocks += 2
        k += 1
    return {
        "value": blocks / spent, "unit": "verify blocks/s", "cores": cores, "kind": "oracle",
        "sample": f"{blocks} sequences (greedy/sampling pairs) of the fused workload, each pair a separate "
                  f"oracle call: float64 lm_head product (numpy/OpenBLAS, {cores} threads) + the "
                  f"single-threaded C accept; {spent / blocks * 1e3:.0f} ms per sequence; host CPU: "
                  f"{cpu_model()}",
    }


def main_fused(args) -> int:
    """The fused verify workload: target logits formed from hidden states and
    the lm_head weight inside the call."""
    import numpy as np
    import torch
    import workloads as W
    import lossless_draft_verification_amd as L

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    log("generating the fused workload: " + W.FUSED_TEXT)
    t0 = time.time()
    case = W.fused_config()
    log(f"generated in {time.time() - t0:.1f}s")
    b, K, V, D, cap = case.b, case.K, case.V, case.D, case.softcap
    M = b * (K + 1)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    h, w = bf(case.hidden), bf(case.weight)
    d = torch.from_numpy(case.draft).to(dev)
    x = torch.from_numpy(case.draft_tokens).to(dev)
    temps = torch.from_numpy(case.temps).to(dev)
    seeds = torch.from_numpy(case.seeds.view(np.int64)).to(dev)
    out = L.AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                         torch.empty(b, K + 1, dtype=torch.int32, device=dev),
                         p_draft=torch.empty(b, K, device=dev), q_draft=torch.empty(b, K, device=dev),
                         argmax=torch.empty(b, K + 1, dtype=torch.int32, device=dev))
    ws = torch.empty(L.fused_workspace_bytes(b, K, V, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(k, evs=None):
        L.set_stage_events(evs)
        L.fused_mixed_accept(h, w, d, x, temps, seeds, softcap=cap, out=out, workspace=ws, stream=stream)

    def mk_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)
        return evs

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(n):
            fn(k)
        end.record(stream)
        torch.cuda.synchronize()
        L.set_stage_events(None)
        return start.elapsed_time(end)

    log(f"warmup {args.warmup} fused steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    settle_s, settle_steps = settle(step, args.settle, chunk=10)
    log(f"settled clocks: {settle_steps} untimed steps in {settle_s:.2f}s")
    log(f"region 1: {args.steps} timed fused steps")
    total_ms = timed(step, args.steps)
    ms_per_step = total_ms / args.steps
    log("region 2: the same steps with stage events")
    names = ["lm_head_gemm", "tile_merge", "draft_row_pass", "scan", "residual_mass", "draw_token"]
    evs = [mk_events(7) for _ in range(args.steps)]
    staged_ms = timed(lambda k: step(k, evs[k]), args.steps)
    stage = {nm: float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(args.steps)]))
             for j, nm in enumerate(names)}
    gemm_flops = 2.0 * M * D * V
    achieved = gemm_flops / (stage["lm_head_gemm"] * 1e-3) / 1e12

    n_all = out.n_accepted.cpu().numpy()
    sidx = np.nonzero(case.temps > 0.0)[0]
    n_s = n_all[sidx]
    rejected = int(((n_s >= 0) & (n_s < K)).sum())
    bonus = int((n_s == K).sum())
    bs = len(sidx)
    step_bytes = (V * D * 2 + M * D * 2 + bs * (K + 1) * V * 4 + bs * K * V * 4
                  + rejected * 2 * V * 4 + bonus * SEG_BYTES)

    reference = None
    if not args.no_reference:
        log("reference: hipBLASLt GEMM (bf16 in, fp32 out) + softcap + spec_mixed_accept")
        h2 = h.view(M, D)
        out_r = L.AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                               torch.empty(b, K + 1, dtype=torch.int32, device=dev),
                               p_draft=torch.empty(b, K, device=dev), q_draft=torch.empty(b, K, device=dev),
                               argmax=torch.empty(b, K + 1, dtype=torch.int32, device=dev))
        ws_r = torch.empty(L.mixed_workspace_bytes(b, K, V, torch.float32), dtype=torch.uint8, device=dev)
        try:
            z = torch.mm(h2, w.t(), out_dtype=torch.float32)
            gemm_kind = "torch.mm(bf16, bf16, out_dtype=float32)"
        except Exception as e:                      # no fp32-output bf16 product in this torch
            log(f"torch.mm out_dtype unavailable ({type(e).__name__}); reference GEMM in bf16 out")
            z = None
            gemm_kind = "torch.mm(bf16, bf16) -> bf16, then .float()"

        def gemm():
            if z is not None:
                return torch.mm(h2, w.t(), out_dtype=torch.float32)
            return torch.mm(h2, w.t()).float()

        def ref_step(k):
            zz = gemm()
            zz.div_(cap).tanh_().mul_(cap)
            L.mixed_accept(zz.view(b, K + 1, V), d, x, temps, seeds, out=out_r, workspace=ws_r, stream=stream)

        for k in range(min(args.warmup, 20)):
            ref_step(k)
        n_ref = max(1, min(args.steps, 200))
        ref_ms = timed(ref_step, n_ref) / n_ref
        for k in range(5):
            gemm()
        gemm_ms = timed(lambda k: gemm(), n_ref) / n_ref
        same = bool((out_r.n_accepted == out.n_accepted).all().item())
        reference = {"unfused_ms_per_step": ref_ms, "unfused_blocks_per_s": b / (ref_ms * 1e-3),
                     "library_gemm": gemm_kind, "library_gemm_ms": gemm_ms,
                     "library_gemm_TFLOPs": gemm_flops / (gemm_ms * 1e-3) / 1e12,
                     "same_accepted_lengths_as_fused": same}

    result = {
        "metric": "fused verify blocks/s (lm_head GEMM + verify), b=128 K=7 V=262144 D=3840",
        "value": b / (ms_per_step * 1e-3),
        "unit": "verify blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": settle_s,
        "settle_steps": settle_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused: " + W.FUSED_TEXT, "b": b, "K": K, "V": V, "D": D, "softcap": cap,
                   "greedy_sequences": int((case.temps == 0.0).sum()), "sampling_sequences": bs,
                   "step": "one spec_fused_mixed_accept call", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "lm_head_dl_kernel", "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": load_traffic("lm_head_gemm", "fused_b128_V262144_D3840"),
                     "algorithmic_flops_per_launch": gemm_flops,
                     "avg_launch_ms": stage["lm_head_gemm"]},
        "step_hbm": {"algorithmic_bytes_per_step": step_bytes,
                     "achieved_GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
                     "rejected_sequences": rejected, "bonus_sequences": bonus},
        "stage_ms": stage,
        "staged_ms_per_step": staged_ms / args.steps,
        "reference": reference,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"timing the fused oracle (budget {args.cpu_budget:.0f}s)")
        result["cpu_baseline"] = cpu_baseline_fused(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_markov(case, budget_s: float):
    """Time the Markov block-decode oracle on small batches of the workload."""
    import numpy as np
    import oracle.markov as OM
    spent, blocks, k = 0.0, 0, 0
    while k == 0 or (spent < budget_s and 2 * k + 2 <= case.b):
        idx = [2 * k, 2 * k + 1]
        t0 = time.perf_counter()
        OM.block_decode(case.base[idx], case.anchors[idx], case.w1, case.w2, case.temps[idx], case.seeds[idx],
                        hidden=case.hidden[idx], conf_w=case.conf_w, conf_b=case.conf_b, threshold=0.6)
        spent += time.perf_counter() - t0
        blocks += 2
        k += 1
    return {"value": blocks / spent, "unit": "draft blocks/s", "cores": os.cpu_count() or 1, "kind": "oracle",
            "sample": f"{blocks} sequences of the Markov workload in pairs (one greedy, one sampled): float64 "
                      f"correction by numpy, C-oracle draws; {spent / blocks * 1e3:.0f} ms per sequence; "
                      f"host CPU: {cpu_model()}"}


def main_markov(args) -> int:
    """The draft-side block decode with the Markov head (the step that
    produces the verify's draft block)."""
    import numpy as np
    import torch
    import workloads as W
    import lossless_draft_verification_amd as L

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    log("generating the Markov workload: " + W.MARKOV_TEXT)
    t0 = time.time()
    case = W.markov_config()
    log(f"generated in {time.time() - t0:.1f}s")
    b, K, V, r, D = case.b, case.K, case.V, case.r, case.D

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    base = torch.from_numpy(case.base).to(dev)
    anchors = torch.from_numpy(case.anchors).to(dev)
    w1, w2, hid, cw = bf(case.w1), bf(case.w2), bf(case.hidden), bf(case.conf_w)
    temps = torch.from_numpy(case.temps).to(dev)
    seeds = torch.from_numpy(case.seeds.view(np.int64)).to(dev)
    out = L.DraftBlock(torch.empty(b, K, dtype=torch.int32, device=dev),
                       torch.empty(b, K, V, dtype=torch.float32, device=dev),
                       torch.empty(b, K, dtype=torch.float32, device=dev), torch.empty(b, dtype=torch.int32, device=dev))
    ws = torch.empty(L.markov_workspace_bytes(b, K, V, r), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(k, evs=None):
        L.set_stage_events(evs)
        L.markov_block_decode(base, anchors, w1, w2, temps, seeds, hidden=hid, conf_w=cw, conf_b=case.conf_b,
                              threshold=0.6, out=out, workspace=ws, stream=stream)

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(n):
            fn(k)
        end.record(stream)
        torch.cuda.synchronize()
        L.set_stage_events(None)
        return start.elapsed_time(end)

    log(f"warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    settle_s, settle_steps = settle(step, args.settle, chunk=10)
    log(f"settled clocks: {settle_steps} untimed steps in {settle_s:.2f}s")
    total_ms = timed(step, args.steps)
    ms = total_ms / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        for q in e:
            q.record(stream)
    staged = timed(lambda k: step(k, evs[k]), args.steps)
    loop_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    conf_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # per position: the W2 table, the base row and the corrected row of every
    # sequence, the gathered W1 rows; then one bonus-free draw segment per
    # sampled sequence (16 KiB fp32)
    bs = int((case.temps > 0.0).sum())
    per_pos = V * r * 2 + b * V * 4 * 2 + b * r * 2 + bs * SEG_BYTES
    loop_bytes = K * per_pos
    achieved = loop_bytes / (loop_ms * 1e-3) / 1e9
    # The correction kernel's traffic is two streams read for one written.  A
    # plain stream of that mix at the same size (two 134 MB float32 rows added
    # into a third, torch's elementwise kernel) is the reference for it.
    mix = [torch.empty(b * V, dtype=torch.float32, device=dev) for _ in range(3)]
    for _ in range(3):
        torch.add(mix[0], mix[1], out=mix[2])
    mix_ts = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.add(mix[0], mix[1], out=mix[2])
        e1.record(stream)
        e1.synchronize()
        mix_ts.append(e0.elapsed_time(e1))
    mix_gbs = 3 * b * V * 4 / (float(np.median(mix_ts)) * 1e-3) / 1e9
    del mix
    result = {
        "metric": "draft blocks/s (Markov-head block decode), b=128 K=7 V=262144 r=256",
        "value": b / (ms * 1e-3), "unit": "draft blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_s": settle_s, "settle_steps": settle_steps,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "markov: " + W.MARKOV_TEXT, "b": b, "K": K, "V": V, "r": r, "D": D,
                   "confidence_threshold": 0.6, "step": "one spec_markov_block_decode call",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "position loop (markov_stream_kernel + draft_select_kernel, 7 positions)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": markov_loop_traffic(K), "algorithmic_bytes_per_launch": loop_bytes,
                     "avg_launch_ms": loop_ms,
                     "ceiling": {"kernel": "torch.add over two 134 MB float32 rows into a third (2 reads : 1 write, "
                                           "the correction kernel's mix)",
                                 "GBs": mix_gbs, "peak_frac": mix_gbs / HBM_PEAK_GBS, "frac": achieved / mix_gbs}},
        "stage_ms": {"position_loop": loop_ms, "confidence": conf_ms},
        "staged_ms_per_step": staged / args.steps,
        "mean_draft_length": float(out.lengths.float().mean().item()),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"timing the Markov oracle (budget {args.cpu_budget:.0f}s)")
        result["cpu_baseline"] = cpu_baseline_markov(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def read_ceiling(stream, nbytes: int = 1 << 30, launches: int = 20) -> dict:
    """The achievable read bandwidth beside the spec peak: spec_stream_read
    (the row pass's load shape) over 1 GiB, larger than every cache, median of
    `launches` event-timed launches on the bench's stream."""
    import numpy as np
    import torch
    import lossless_draft_verification_amd as L
    src = torch.empty(nbytes, dtype=torch.uint8, device=stream.device)
    sink = torch.zeros(1, dtype=torch.int32, device=stream.device)
    for _ in range(3):
        L.stream_read(src, sink, stream=stream)
    ts = []
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.stream_read(src, sink, stream=stream)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del src
    return {"kernel": "stream_read_kernel (read-only, 1 GiB, the row pass's load shape)",
            "GBs": nbytes / (ms * 1e-3) / 1e9, "peak_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000, help="untimed steps first")
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="after the warm-up, untimed steps for at least this much wall time, "
                         "whatever --warmup is, so the GPU clocks have ramped up before timing")
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--step", choices=["mixed", "split"], default="mixed")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--markov", action="store_true",
                    help="the draft-side Markov block decode instead of the verify")
    ap.add_argument("--fused", action="store_true",
                    help="the fused verify workload (lm_head GEMM inside the call) instead of c5")
    ap.add_argument("--sharded", type=int, default=0, metavar="G",
                    help="mixed step over G vocabulary shards in separate buffers")
    ap.add_argument("--ragged", action="store_true",
                    help="mixed step with per-sequence draft lengths drawn uniformly from 0..K")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true", help="skip the split-call reference region")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--summarize-rocprof", default="", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 CSVs under DIR and exit")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_traces(args.summarize_rocprof)
        return summarize_rocprof(args.summarize_rocprof)
    if (args.ragged or args.sharded) and args.step != "mixed":
        print("--ragged and --sharded need --step mixed", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the verify step shards by sequence with no exchange; see the design notes).",
              file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.fused:
        return main_fused(args)
    if args.markov:
        return main_markov(args)

    import numpy as np
    import torch
    import workloads as W
    import lossless_draft_verification_amd as L

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")

    log(f"generating workload {args.workload}: {W.CONFIG_TEXT[args.workload]}")
    t0 = time.time()
    case = W.config(args.workload)
    log(f"generated in {time.time() - t0:.1f}s")
    K, V, b = case.K, case.V, case.b
    if args.workload == 1:
        temps_np = np.full(b, case.T)                # one sequence: sampling rule
    else:
        temps_np = np.where(case.rule == W.GREEDY, 0.0, case.T)
    gidx, sidx = np.nonzero(temps_np == 0.0)[0], np.nonzero(temps_np > 0.0)[0]
    has_g, has_s = len(gidx) > 0, len(sidx) > 0
    for idx in (gidx, sidx):
        assert len(idx) == 0 or (np.diff(idx) == 1).all(), "each rule must own a contiguous range"

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    tgt0, drf0 = to_dev(case.target), to_dev(case.draft)
    copies = [(tgt0, drf0)] + [(tgt0.clone(), drf0.clone()) for _ in range(args.copies - 1)]
    x = torch.from_numpy(case.draft_tokens).to(dev)
    seeds = torch.from_numpy(case.seeds.view(np.int64)).to(dev)
    temps = torch.from_numpy(temps_np.astype(np.float64)).to(dev)
    klen_np = (np.random.default_rng(54).integers(0, K + 1, size=b).astype(np.int32) if args.ragged
               else np.full(b, K, np.int32))
    klen = torch.from_numpy(klen_np).to(dev) if args.ragged else None
    dt = tgt0.dtype
    g0, g1 = (int(gidx[0]), int(gidx[-1]) + 1) if has_g else (0, 0)
    s0, s1 = (int(sidx[0]), int(sidx[-1]) + 1) if has_s else (0, 0)
    bg, bs = g1 - g0, s1 - s0

    def res(n, samp, greedy):
        return L.AcceptResult(torch.empty(n, dtype=torch.int32, device=dev),
                              torch.empty(n, K + 1, dtype=torch.int32, device=dev),
                              p_draft=torch.empty(n, K, device=dev) if samp else None,
                              q_draft=torch.empty(n, K, device=dev) if samp else None,
                              argmax=torch.empty(n, K + 1, dtype=torch.int32, device=dev) if greedy else None)

    out_m = res(b, True, True)
    ws_m = torch.zeros(L.mixed_workspace_bytes(b, K, V, dt), dtype=torch.uint8, device=dev)
    shard_copies, ws_sh, widths = None, None, None
    if args.sharded:
        G = args.sharded
        unit = 8192 if V % (8192 * G) == 0 else 1
        base = V // (unit * G) * unit
        widths = [base] * (G - 1) + [V - base * (G - 1)]
        cuts = np.cumsum([0] + widths)
        shard_copies = [([t[:, :, a:c].contiguous() for a, c in zip(cuts[:-1], cuts[1:])],
                         [d[:, :, a:c].contiguous() for a, c in zip(cuts[:-1], cuts[1:])]) for t, d in copies]
        copies = copies[:1]
        torch.cuda.empty_cache()
        ws_sh = torch.zeros(L.sharded_workspace_bytes(widths, b, K, dt), dtype=torch.uint8, device=dev)
    out_g = res(max(bg, 1), False, True)
    ws_g = torch.zeros(L.workspace_bytes(max(bg, 1), K, V, dt, False), dtype=torch.uint8, device=dev)
    out_s = res(max(bs, 1), True, False)
    ws_s = torch.zeros(L.workspace_bytes(max(bs, 1), K, V, dt, True), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step_mixed(k, evs=None):
        L.set_stage_events(evs)
        if shard_copies is not None:
            ts, ds = shard_copies[k % len(shard_copies)]
            L.sharded_mixed_accept(ts, ds, x, temps, seeds, draft_lengths=klen, out=out_m, workspace=ws_sh,
                                   stream=stream)
            return
        t, d = copies[k % len(copies)]
        L.mixed_accept(t, d, x, temps, seeds, draft_lengths=klen, out=out_m, workspace=ws_m, stream=stream)

    def step_split(k, gev=None, sev=None):
        t, d = copies[k % len(copies)]
        if has_g:
            L.set_stage_events(gev)
            L.greedy_accept(t[g0:g1], x[g0:g1], out=out_g, workspace=ws_g, stream=stream)
        if has_s:
            L.set_stage_events(sev)
            L.speculative_sample_accept(t[s0:s1], d[s0:s1], x[s0:s1], case.T, seeds[s0:s1], out=out_s,
                                        workspace=ws_s, stream=stream)

    def mk_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)          # creates the underlying hipEvent
        return evs

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(n):
            fn(k)
        end.record(stream)
        torch.cuda.synchronize()
        L.set_stage_events(None)
        return start.elapsed_time(end)

    mixed = args.step == "mixed"
    main_step = (lambda k: step_mixed(k)) if mixed else (lambda k: step_split(k))
    log(f"warmup {args.warmup} steps ({args.step})")
    for k in range(args.warmup):
        main_step(k)
    torch.cuda.synchronize()
    settle_s, settle_steps = settle(main_step, args.settle)
    log(f"settled clocks: {settle_steps} untimed steps in {settle_s:.2f}s")

    log(f"region 1: {args.steps} timed steps")
    total_ms = timed(main_step, args.steps)
    ms_per_step = total_ms / args.steps
    blocks_per_s = b * args.steps / (total_ms * 1e-3)

    log("region 2: the same steps with stage events")
    stage = {}
    names = ["row_pass", "scan", "residual_mass", "draw_token"]
    if mixed:
        evs = [mk_events(5) for _ in range(args.steps)]
        staged_ms = timed(lambda k: step_mixed(k, evs[k]), args.steps)
        for j, nm in enumerate(names):
            stage[nm] = float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(args.steps)]))
    else:
        gevs = [mk_events(3) for _ in range(args.steps)] if has_g else [None] * args.steps
        sevs = [mk_events(5) for _ in range(args.steps)] if has_s else [None] * args.steps
        staged_ms = timed(lambda k: step_split(k, gevs[k], sevs[k]), args.steps)
        if has_g:
            for j, nm in enumerate(names[:2]):
                stage["greedy_" + nm] = float(np.mean([gevs[k][j].elapsed_time(gevs[k][j + 1])
                                                       for k in range(args.steps)]))
        if has_s:
            for j, nm in enumerate(names):
                stage["sample_" + nm] = float(np.mean([sevs[k][j].elapsed_time(sevs[k][j + 1])
                                                       for k in range(args.steps)]))

    reference = None
    if mixed and not args.no_reference and has_g and has_s:
        log("region 3: the same steps as two split calls (reference)")
        for k in range(min(args.warmup, 100)):
            step_split(k)
        ref_ms = timed(lambda k: step_split(k), args.steps) / args.steps
        reference = {"split_calls_ms_per_step": ref_ms, "split_calls_blocks_per_s": b / (ref_ms * 1e-3)}

    # outcome of the (identical) steps, for the algorithmic byte count
    if mixed:
        n_all = out_m.n_accepted.cpu().numpy()
        n_s = n_all[sidx] if has_s else np.zeros(0, np.int32)
    else:
        n_s = out_s.n_accepted.cpu().numpy()[:bs] if has_s else np.zeros(0, np.int32)
    ks = klen_np[sidx] if has_s else np.zeros(0, np.int32)
    rejected = int(((n_s >= 0) & (n_s < ks)).sum())
    bonus = int((n_s == ks).sum())
    es = 2 if dt == torch.bfloat16 else 4
    # rows each sequence's block holds: Ks + 1 target rows, plus Ks draft rows when sampled
    bytes_greedy = int((klen_np[gidx].astype(np.int64) + 1).sum()) * V * es if has_g else 0
    bytes_sample_pass = int((2 * ks.astype(np.int64) + 1).sum()) * V * es
    # per sampling sequence: one pass over its 2K+1 rows, plus the rejected
    # row pair read again for the residual, or one segment of the bonus row
    bytes_step = bytes_greedy + bytes_sample_pass + rejected * 2 * V * es + bonus * SEG_BYTES
    if mixed:
        dom, dom_bytes, dom_ms = "row_pass", bytes_greedy + bytes_sample_pass, stage["row_pass"]
    elif has_s:
        dom, dom_bytes, dom_ms = "row_pass", bytes_sample_pass, stage["sample_row_pass"]
    else:
        dom, dom_bytes, dom_ms = "row_pass", bytes_greedy, stage["greedy_row_pass"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    ceiling = read_ceiling(stream)
    wl_key = (f"c{args.workload}_{args.step}" + ("_ragged" if args.ragged else "")
              + (f"_sharded{args.sharded}" if args.sharded else ""))
    traffic = load_traffic(dom, wl_key)

    result = {
        "metric": "verify blocks/s and achieved HBM GB/s (% of peak), b=128 K=7 V=262144 bf16",
        "value": blocks_per_s,
        "unit": "verify blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": settle_s,
        "settle_steps": settle_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if es == 2 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"c{args.workload}: {W.CONFIG_TEXT[args.workload]}" + (
                "; per-sequence draft lengths uniform on 0..K (seeded)" if args.ragged else "") + (
                f"; vocabulary split into {args.sharded} shards of widths {widths}" if args.sharded else ""),
            "mean_draft_length": float(klen_np.mean()),
            "b": b, "K": K, "V": V, "temperature": case.T,
            "greedy_sequences": bg, "sampling_sequences": bs,
            "step": (f"one spec_sharded_mixed_accept call over {args.sharded} shards" if args.sharded else
                     "one spec_mixed_accept call (per-sequence temperature 0 / 0.8)" if mixed else
                     "spec_greedy_accept over the greedy sequences + spec_sample_accept over the "
                     "sampling sequences, one stream"),
            "input_copies_rotated": len(shard_copies) if shard_copies is not None else len(copies),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_ms": dom_ms,
            "ceiling": dict(ceiling, frac=achieved / ceiling["GBs"]),
        },
        "step_hbm": {
            "algorithmic_bytes_per_step": bytes_step,
            "achieved_GBs": bytes_step / (ms_per_step * 1e-3) / 1e9,
            "frac": bytes_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "rejected_sequences": rejected, "bonus_sequences": bonus,
        },
        "stage_ms": stage,
        "staged_ms_per_step": staged_ms / args.steps,
        "reference": reference,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle (budget {args.cpu_budget:.0f}s)")
        gi = gidx if has_g else sidx
        si = sidx if has_s else gidx
        result["cpu_baseline"] = cpu_baseline(case, gi, si, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
