#!/usr/bin/env python3
"""Throughput of one MiniMax-H3-Image DiT block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4096]

One step = one h3dit_block_forward over the whole joint sequence (all nine
steps of the block: modulation, RoPE table, RMSNorm1, QKV+RoPE GEMM,
attention, output projection, RMSNorm2, MLP up+GELU, MLP down), inputs and
weights resident in HBM before the timed region starts. Prints ONE JSON line.

The K timed steps are plain h3dit_block_forward calls between two HIP events.
Per-kernel times come from a second pass of K steps in which the library also
records HIP events between its kernel launches on the same stream
(h3dit_block_forward_timed), averaged over those steps; that pass also gives
the median, minimum and maximum of the single forwards and its own mean (the
events' records add a little to it). The roofline object reports the slowest
kernel.

The cpu_baseline leg times the float64 CPU oracle on a bounded sample of the
same workload (a few sampled query rows; keys and values still cover every
token) and extrapolates linearly in the number of rows to a whole block.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 (MXFP8 scaled) MFMA: twice the bf16 rate
GEMM_STAGES = ("qkv_rope_gemm", "out_proj_gemm", "mlp_up_gelu_gemm", "mlp_down_gemm")
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "DiT block tokens/s + TFLOP/s (% bf16 MFMA peak), 4096/16384 image tokens"

STAGES = ["modulation", "rope_table", "rmsnorm1", "qkv_rope_gemm", "attention", "out_proj_gemm",
          "rmsnorm2", "mlp_up_gelu_gemm", "mlp_down_gemm"]


def stage_work(cfg):
    """Algorithmic FLOPs / HBM bytes of each kernel of one block (per launch)."""
    T, D, A, F = cfg.n_tokens, cfg.hidden, cfg.attn_width, cfg.ffn
    xb = 4 if cfg.x_dtype == "fp32" else 2
    flops = {
        "modulation": 2.0 * 6 * D * D,
        "qkv_rope_gemm": 2.0 * T * D * 3 * A,
        "attention": 4.0 * T * T * A,
        "out_proj_gemm": 2.0 * T * A * D,
        "mlp_up_gelu_gemm": 2.0 * T * D * F,
        "mlp_down_gemm": 2.0 * T * F * D,
    }
    nbytes = {
        "modulation": 2.0 * 6 * D * D + 4 * D + 8 * 6 * D,
        "rope_table": 8.0 * T + 4.0 * T * 128,
        "rmsnorm1": (xb + 2.0) * T * D,
        "rmsnorm2": (4.0 + 2.0) * T * D,
        "qkv_rope_gemm": 2.0 * T * D + 2.0 * 3 * A * D + 2.0 * T * 3 * A + 4.0 * T * 128,
        "attention": 2.0 * T * 3 * A + 2.0 * T * A,
        "out_proj_gemm": 2.0 * T * A + 2.0 * D * A + (xb + 4.0) * T * D,
        "mlp_up_gelu_gemm": 2.0 * T * D + 2.0 * F * D + 2.0 * T * F,
        "mlp_down_gemm": 2.0 * T * F + 2.0 * D * F + 8.0 * T * D,
    }
    return flops, nbytes


def block_flops(cfg) -> float:
    T, D, A, F = cfg.n_tokens, cfg.hidden, cfg.attn_width, cfg.ffn
    return 2.0 * T * (3 * A * D + A * D + 2 * D * F) + 4.0 * T * T * A + 2.0 * 6 * D * D


class ClockSampler:
    """Samples the GPU's current shader clock and board power from sysfs
    (pp_dpm_sclk: the level marked '*' is the present clock; hwmon power1_input
    in microwatts) every few milliseconds on a host thread, while the GPU works
    through already-queued forwards. Reports nothing where the files are absent."""

    def __init__(self, period_s: float = 0.004, root: str = "/sys/class/drm"):
        import glob
        import threading
        self.period = period_s
        dev = sorted(glob.glob(os.path.join(root, "card*", "device", "pp_dpm_sclk")))
        self.sclk = dev[0] if dev else None
        pw = sorted(glob.glob(os.path.join(os.path.dirname(dev[0]), "hwmon", "*", "power1_input"))) if dev else []
        self.power = pw[0] if pw else None
        self.mhz, self.watts = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            with open(self.sclk) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        self.mhz.append(float(line.split(":")[1].strip().lower().split("mhz")[0]))
            if self.power:
                with open(self.power) as f:
                    self.watts.append(float(f.read()) * 1e-6)
        except (OSError, ValueError, IndexError):
            pass

    def _run(self):
        while not self._stop.is_set():
            self._read()
            self._stop.wait(self.period)

    def __enter__(self):
        if self.sclk:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.sclk:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.mhz:
            return None
        m = sorted(self.mhz)
        out = {"mean_mhz": round(sum(m) / len(m)), "median_mhz": round(m[len(m) // 2]),
               "min_mhz": round(m[0]), "max_mhz": round(m[-1]), "samples": len(m),
               "source": "pp_dpm_sclk, sampled during the timed forwards"}
        if self.watts:
            out["mean_board_power_w"] = round(sum(self.watts) / len(self.watts), 1)
        return out


def measure(cfg, steps: int, warmup: int, linears: str = "bf16"):
    import torch
    from joint_attention_dit_amd import binding as B
    from joint_attention_dit_amd.inputs import make_inputs

    inp = make_inputs(cfg, seed=0)
    blk = B.Block(cfg, inp, device="cuda:0", linears=linears)
    del inp
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        blk.forward(stream)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(steps)]
    for row in ev:          # torch creates the underlying hipEvent_t on first record
        for e in row:
            e.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    assert all(e.cuda_event for row in ev for e in row)
    # the headline: K plain forwards (the clock sampled meanwhile on the host)
    with ClockSampler() as clock:
        start.record(stream)
        for _ in range(steps):
            blk.forward(stream)
        end.record(stream)
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # per-kernel times: K forwards with the library's events between its launches
    start.record(stream)
    for k in range(steps):
        blk.forward_timed([e.cuda_event for e in ev[k]], stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms_timed = start.elapsed_time(end) / steps
    stage_ms = {s: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)) / steps
                for i, s in enumerate(STAGES)}
    # each block forward on its own, first to last stage event: spread over the timed steps
    per_step = sorted(ev[k][0].elapsed_time(ev[k][-1]) for k in range(steps))
    spread = {"median_ms": round(per_step[steps // 2] if steps % 2 else
                                 0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2]), 4),
              "min_ms": round(per_step[0], 4), "max_ms": round(per_step[-1], 4),
              "mean_ms_with_stage_events": round(ms_timed, 4),
              "of": "single forwards of the pass with stage events",
              "sclk": clock.summary()}
    out_ok = bool(torch.isfinite(blk.out).all().item())
    del blk
    torch.cuda.empty_cache()
    return ms, stage_ms, out_ok, spread


def summarize(cfg, ms, stage_ms, linears: str = "bf16"):
    flops, nbytes = stage_work(cfg)
    total = block_flops(cfg)
    tflops = total / (ms * 1e-3) / 1e12
    # each product kernel against the matrix-core peak of its own operand type
    peak = {s: (PEAK_FP8_TFLOPS if linears == "mxfp8" and s in GEMM_STAGES else PEAK_BF16_TFLOPS)
            for s in STAGES}
    kernels = {}
    for s in STAGES:
        t = stage_ms[s] * 1e-3
        k = {"ms": round(stage_ms[s], 4)}
        if s in flops and s != "modulation":
            k["tflops"] = round(flops[s] / t / 1e12, 1)
            k["pct_mfma_peak"] = round(100 * flops[s] / t / 1e12 / peak[s], 1)
        else:
            k["gbs"] = round(nbytes[s] / t / 1e9, 1)
            k["pct_hbm_peak"] = round(100 * nbytes[s] / t / 1e9 / PEAK_HBM_GBS, 1)
        kernels[s] = k
    dom = max(STAGES, key=lambda s: stage_ms[s])
    t = stage_ms[dom] * 1e-3
    if dom in flops and dom != "modulation":
        ach = flops[dom] / t / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak[dom],
                "unit": "TFLOP/s", "frac": round(ach / peak[dom], 4),
                "traffic": measured_traffic(dom) if linears == "bf16" or dom not in GEMM_STAGES
                else None,
                "traffic_unit": "HBM bytes per launch", "algorithmic_per_launch": flops[dom]}
    else:
        ach = nbytes[dom] / t / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom), "traffic_unit": "HBM bytes per launch",
                "algorithmic_per_launch": nbytes[dom]}
    return tflops, kernels, roof


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_4096.md")
KERNEL_SOURCES = {
    "attention": "attention.hip", "qkv_rope_gemm": "gemm.hip", "out_proj_gemm": "gemm.hip",
    "mlp_up_gelu_gemm": "gemm.hip", "mlp_down_gemm": "gemm.hip", "modulation": "modulation.hip",
    "rmsnorm1": "rmsnorm_modulate.hip", "rmsnorm2": "rmsnorm_modulate.hip",
    "rope_table": "rope_table.hip",
}
# dispatch order of one block forward (h3dit_block_forward launches in this order)
KERNEL_ORDER = ["modulation", "rope_table", "rmsnorm1", "qkv_rope_gemm", "attention",
                "out_proj_gemm", "rmsnorm2", "mlp_up_gelu_gemm", "mlp_down_gemm"]
COPY_BYTES = 1 << 30   # the plain copy used to calibrate the HBM byte counters


def source_digest(stage: str) -> str:
    """Digest of the kernel's source file and of every local header it includes
    (recursively, in include order), so that a change to a shared header also
    marks the stored counter figures as stale."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "joint_attention_dit_amd", "csrc")
    h = hashlib.sha256()
    seen = set()

    def add(name):
        path = os.path.join(csrc, name)
        if name in seen or not os.path.exists(path):
            return
        seen.add(name)
        with open(path, "rb") as f:
            data = f.read()
        h.update(name.encode() + b"\0" + data)
        for inc in re.findall(rb'^#include "([^"]+)"', data, re.M):
            add(inc.decode())

    add(KERNEL_SOURCES[stage])
    return h.hexdigest()[:16]


def measured_traffic(stage: str):
    """HBM bytes per launch of `stage` from the committed counter summary, or None
    when the summary is missing or the kernel's source changed since it was taken."""
    try:
        text = open(TRAFFIC_FILE).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)["kernels"][stage]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_digest(stage):
        return None
    return rec["hbm_bytes"]


def traffic_run(cfg):
    """One plain 1 GiB device copy, then one block forward: the command that the
    two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE) profile."""
    import torch
    from joint_attention_dit_amd import binding as B
    from joint_attention_dit_amd.inputs import make_inputs

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    inp = make_inputs(cfg, seed=0)
    blk = B.Block(cfg, inp, device="cuda:0")
    del inp
    blk.forward(torch.cuda.current_stream())
    torch.cuda.synchronize()
    print("traffic run done", flush=True)


def summarize_traffic(fetch_dir: str, write_dir: str, cfg) -> str:
    """Counter CSVs of the two traffic-run passes -> the profiles/ summary text."""
    import csv
    import glob

    def per_dispatch(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return rows

    out = {}
    scales = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(d, counter)
        copy = [r for r in rows if "copy" in r[1].lower() or "elementwise" in r[1].lower()]
        # library dispatches in order; a GEMM's slice-sum kernel counts with that GEMM
        lib = _library_dispatches(rows)
        assert copy, counter
        copy_kib = max(r[2] for r in copy)
        scales[counter] = COPY_BYTES / (copy_kib * 1024.0)
        for stage, r in zip(KERNEL_ORDER, lib[-1]):
            out.setdefault(stage, {})[counter] = r[2]
    kernels = {}
    for stage, v in out.items():
        b = v["FETCH_SIZE"] * 1024 * scales["FETCH_SIZE"] + v["WRITE_SIZE"] * 1024 * scales["WRITE_SIZE"]
        kernels[stage] = {"fetch_kib": v["FETCH_SIZE"], "write_kib": v["WRITE_SIZE"],
                          "hbm_bytes": round(b), "source_sha256_16": source_digest(stage)}
    rec = {"workload": cfg.description, "copy_bytes": COPY_BYTES,
           "scale_fetch": round(scales["FETCH_SIZE"], 4), "scale_write": round(scales["WRITE_SIZE"], 4),
           "kernels": kernels}
    flops, nbytes = stage_work(cfg)
    lines = ["| Kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) | algorithmic bytes |",
             "|---|---|---|---|---|"]
    for stage in KERNEL_ORDER:
        k = kernels[stage]
        lines.append(f"| {stage} | {k['fetch_kib']:.0f} | {k['write_kib']:.0f} | "
                     f"{k['hbm_bytes'] / 1e6:.1f} MB | {nbytes[stage] / 1e6:.1f} MB |")
    return "\n".join(lines) + "\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n"


PERCENT_COUNTERS = ("MfmaUtil", "VALUBusy", "LdsUtil", "VALUUtilization", "GPU_UTIL")


def _library_dispatches(rows, add_second: bool = True):
    """(dispatch id, kernel name, value) rows of the library's kernels in
    dispatch order, a GEMM's slice-sum kernel merged into that GEMM and the
    attention's key-piece merge into the attention, grouped into block
    forwards of len(KERNEL_ORDER) kernels each."""
    lib = []
    for r in sorted(rows):
        if "h3dit" not in r[1]:
            continue
        if "gemm_fixup" in r[1] or "attention_merge" in r[1]:
            assert lib, "second kernel of a stage before its first"
            if add_second:  # (a percentage of the main kernel is kept as it is)
                lib[-1] = (lib[-1][0], lib[-1][1], lib[-1][2] + r[2])
        else:
            lib.append(r)
    n = len(KERNEL_ORDER)
    assert lib and len(lib) % n == 0, f"{len(lib)} library dispatches, not whole blocks of {n}"
    return [lib[i:i + n] for i in range(0, len(lib), n)]


def _kernel_label(name: str) -> str:
    """A profiler kernel name (mangled or not) -> 'h3dit::kernel<args>'."""
    import subprocess

    if name.startswith("_Z"):
        try:
            # GNU c++filt lacks the bf16 code DF16b: spell it as a vendor type
            name = subprocess.run(["c++filt", name.replace("DF16b", "u6__bf16")],
                                  capture_output=True, text=True,
                                  check=False).stdout.strip() or name
        except OSError:
            pass
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    if "_Accum" in name:  # a bf16 template argument the profiler could not demangle
        name = name.split("<")[0]
    depth = 0
    for i, ch in enumerate(name):  # cut the parameter list
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def summarize_trace(trace_dir: str, warmup: int, cfg, linears: str = "bf16") -> str:
    """Kernel-trace CSV of a `bench.py --extra=none` run under rocprofv3
    --kernel-trace -> per-kernel durations of the timed blocks only (the first
    `warmup` block forwards are dropped), as the profiles/ summary table. With
    MXFP8 linears the weight quantisations before the first block are left
    out and the GEMMs are priced against the fp8 peak."""
    import csv
    import glob
    import statistics

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # us
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], dur))
    rows.sort()
    while rows and ("mxfp8_quantize" in rows[0][1] or "h3dit" not in rows[0][1]):
        rows.pop(0)  # the weights' quantisation (once, before the timed blocks)
    blocks = _library_dispatches(rows)[warmup:]
    flops, nbytes = stage_work(cfg)
    lines = [f"Timed block forwards: {len(blocks)} (the first {warmup} dropped as warm-up).", "",
             "| Kernel (stage) | Calls | Average (us) | Median (us) | Min (us) | Max (us) | "
             "Achieved | Of peak |", "|---|---|---|---|---|---|---|---|"]
    rec = {}
    for i, stage in enumerate(KERNEL_ORDER):
        d = [b[i][2] for b in blocks]
        avg = sum(d) / len(d)
        if stage in flops and stage != "modulation":
            peak = (PEAK_FP8_TFLOPS if linears == "mxfp8" and stage in GEMM_STAGES
                    else PEAK_BF16_TFLOPS)
            ach = f"{flops[stage] / (avg * 1e-6) / 1e12:.1f} TFLOP/s"
            frac = flops[stage] / (avg * 1e-6) / 1e12 / peak
        else:
            ach = f"{nbytes[stage] / (avg * 1e-6) / 1e9:.0f} GB/s"
            frac = nbytes[stage] / (avg * 1e-6) / 1e9 / PEAK_HBM_GBS
        rec[stage] = {"avg_us": round(avg, 2), "frac": round(frac, 4)}
        lines.append(f"| `{_kernel_label(blocks[0][i][1])}` ({stage}) | {len(d)} | {avg:.1f} | "
                     f"{statistics.median(d):.1f} | {min(d):.1f} | {max(d):.1f} | {ach} | "
                     f"{100 * frac:.1f} % |")
    total = sum(sum(x[2] for x in b) for b in blocks) / len(blocks)
    lines.append("")
    lines.append(f"Sum of the kernels' averages: {total:.1f} us per block "
                 f"({100 * block_flops(cfg) / (total * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of dense "
                 f"bf16 peak on kernel time alone).")
    return "\n".join(lines) + "\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n"


def summarize_counters(dirs, warmup: int, cfg=None) -> str:
    """Counter CSVs of `bench.py --extra=none` runs under rocprofv3 --pmc (one
    directory per pass) -> per-kernel averages over the timed block forwards
    (the first `warmup` dropped). A GEMM's slice-sum kernel adds into the GEMM.
    With `cfg`, a table of the matrix-core kernels comes first: the clock they
    ran at (GRBM_GUI_ACTIVE over the 8 XCDs and the dispatches' own durations in
    the pass that counted it) and their rate against the peak at that clock."""
    import csv
    import glob

    per = {}
    dur = {}  # stage -> average duration (ns) in the pass that counted GRBM_GUI_ACTIVE
    for d in dirs:
        trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
        counted = set()
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            counted |= {r["Counter_Name"] for r in csv.DictReader(open(f))}
        if trace and "GRBM_GUI_ACTIVE" in counted and not dur:
            rows = []
            for f in trace:
                for r in csv.DictReader(open(f)):
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))))
            blocks = _library_dispatches(rows)[warmup:]
            for i, stage in enumerate(KERNEL_ORDER):
                dur[stage] = sum(b[i][2] for b in blocks) / len(blocks)
        by_counter = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                by_counter.setdefault(r["Counter_Name"], []).append(
                    (int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        for counter, rows in by_counter.items():
            blocks = _library_dispatches(rows, counter not in PERCENT_COUNTERS)[warmup:]
            for i, stage in enumerate(KERNEL_ORDER):
                per.setdefault(stage, {})[counter] = sum(b[i][2] for b in blocks) / len(blocks)
    counters = sorted({c for v in per.values() for c in v})
    lines = []
    need = ("MfmaUtil", "VALUBusy", "LdsUtil", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS",
            "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    if cfg is not None and dur and all(c in counters for c in need):
        flops, _ = stage_work(cfg)
        lines += ["| Kernel | MfmaUtil (%) | VALUBusy (%) | LdsUtil (%) | LDS bank-conflict cycles "
                  "/ LDS instr. | MFMA-VALU co-issue cycles / MFMA busy cycles | clock under load "
                  "(GHz) | duration in the pass (us) | TFLOP/s | of the peak at that clock |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for stage in KERNEL_ORDER:
            c = per[stage]
            if stage not in GEMM_STAGES and stage != "attention":
                continue
            ghz = c["GRBM_GUI_ACTIVE"] / 8 / dur[stage]
            tf = flops[stage] / (dur[stage] * 1e-9) / 1e12
            at_clock = PEAK_BF16_TFLOPS * ghz / 2.4
            lines.append(f"| {stage} | {c['MfmaUtil']:.1f} | {c['VALUBusy']:.1f} | {c['LdsUtil']:.1f} | "
                         f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_INSTS_LDS'], 1):.3f} | "
                         f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(c['SQ_VALU_MFMA_BUSY_CYCLES'], 1):.3f} | "
                         f"{ghz:.2f} | {dur[stage] * 1e-3:.1f} | {tf:.0f} | {100 * tf / at_clock:.1f} % |")
        lines.append("")
    lines += ["| Kernel | " + " | ".join(counters) + " |", "|---|" + "---|" * len(counters)]
    for stage in KERNEL_ORDER:
        lines.append(f"| {stage} | " + " | ".join(f"{per[stage].get(c, float('nan')):.4g}"
                                                  for c in counters) + " |")
    return "\n".join(lines) + "\n\n```json\n" + json.dumps(per, indent=1) + "\n```\n"


def measure_stack(scfg, images: int, warmup: int, mod_table: bool = True, linears: str = "bf16"):
    """Seconds per image of DiT compute: `scfg.steps` evaluations of the whole
    stack (patch embedding, n_blocks blocks, final layer) with an Euler update
    after each, on seeded random-init weights resident in HBM. With mod_table,
    every block's and the final layer's modulation for all steps is computed
    first in one pass over each AdaLN weight (inside the timed region). With
    linears="mxfp8" the blocks' linear weights are quantised once before the
    timed region (as an online MXFP8 load would) and every block runs MXFP8."""
    import torch
    from joint_attention_dit_amd import binding as B
    from joint_attention_dit_amd.inputs import make_stack_inputs

    inp = make_stack_inputs(scfg, seed=0, device="cuda")
    cfg = B.config_from(scfg.block)
    gh, gw = scfg.grid
    st = B.StackConfig(scfg.n_blocks, scfg.channels, scfg.patch, gh, gw, scfg.block.text_tokens)
    mx = linears == "mxfp8"
    qblocks = None
    if mx:
        qblocks = B.quantize_blocks(inp["blocks"])
        for b in inp["blocks"]:  # only w_ada stays in use
            for k in B.MX_LINEARS:
                b[k] = None
        torch.cuda.empty_cache()
        nbytes = B.h3dit_stack_workspace_size_mxfp8(cfg, st)
    else:
        nbytes = B.h3dit_stack_workspace_size(cfg, st)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    latent0 = inp["latent"].clone()
    latent = latent0.clone()
    v = torch.empty_like(latent)
    stream = torch.cuda.current_stream()

    conds = torch.stack(list(inp["conds"])).contiguous()
    table = torch.empty(scfg.steps, scfg.n_blocks + 1, 6 * scfg.block.hidden, dtype=torch.float64,
                        device="cuda")

    def image():
        latent.copy_(latent0)
        if mod_table:
            B.h3dit_dit_modulation_table(cfg, st, inp["w_ada_final"], inp["blocks"], conds, table,
                                         stream)
        for k, cond in enumerate(inp["conds"]):
            if mx and mod_table:
                B.h3dit_dit_forward_mod_mxfp8(cfg, st, inp["w_patch"], inp["w_final"],
                                              inp["blocks"], qblocks, latent, inp["text"],
                                              table[k], inp["positions"], v, ws, stream)
            elif mx:
                B.h3dit_dit_forward_mxfp8(cfg, st, inp["w_patch"], inp["w_ada_final"],
                                          inp["w_final"], inp["blocks"], qblocks, latent,
                                          inp["text"], cond, inp["positions"], v, ws, stream)
            elif mod_table:
                B.h3dit_dit_forward_mod(cfg, st, inp["w_patch"], inp["w_final"], inp["blocks"],
                                        latent, inp["text"], table[k], inp["positions"], v, ws,
                                        stream)
            else:
                B.h3dit_dit_forward(cfg, st, inp["w_patch"], inp["w_ada_final"], inp["w_final"],
                                    inp["blocks"], latent, inp["text"], cond, inp["positions"], v,
                                    ws, stream)
            B.h3dit_latent_step(latent, v, 1.0 / scfg.steps, stream)

    for _ in range(warmup):
        image()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(images):
        image()
    t1.record(stream)
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) / 1e3 / images
    ok = bool(torch.isfinite(latent).all().item())
    return sec, ok


def attention_inputs(T: int, H: int, rising: bool, seed: int = 0):
    """Synthetic q (pre-scaled) and k, v in the attention kernel's layouts:
    base-2 scores of standard deviation 12 (about that of the full-width
    blocks), or with `rising` the keys' norms growing along the sequence
    (x 0.2 .. 40), so that every row's largest score lies far past its first
    key tile's and every workgroup takes the second pass of the kernel."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(T, H * 128, device="cuda", generator=g) * (12.0 / 128 ** 0.5)
    k = torch.randn(T, H * 128, device="cuda", generator=g)
    if rising:
        k *= (0.2 + 40.0 * torch.arange(T, device="cuda", dtype=torch.float32) / T).reshape(T, 1)
    qk = torch.cat([q, k], dim=1).to(torch.bfloat16).contiguous()
    vt = torch.randn(H, 128, T + (-T) % 64, device="cuda", generator=g).to(torch.bfloat16)
    return qk, vt


def measure_attention_cliff(cfg, steps: int, warmup: int):
    """Time of h3dit_attention at the block's shape on ordinary scores and on
    rising ones (every workgroup runs the key loop twice, after a scores-only
    pass for its rows' maxima): the factor between the two bounds the cost of
    the kernel's second pass."""
    import torch
    from joint_attention_dit_amd import binding as B

    T, H = cfg.n_tokens, cfg.heads
    c = B.make_config(cfg.hidden, H, cfg.ffn, T)
    o = torch.empty(T, H * 128, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name, rising in (("ordinary", False), ("rising", True)):
        qk, vt = attention_inputs(T, H, rising)
        for _ in range(warmup):
            B.h3dit_attention(c, qk, vt, o, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            B.h3dit_attention(c, qk, vt, o, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
        del qk, vt
    return res


def measure_gemm_reference(cfg, steps: int, warmup: int):
    """Context only: the QKV-shaped product (T x 3A x D of the workload) through
    this library's GEMM (h3dit_linear_f32, fp32 output) and through torch's
    F.linear (hipBLASLt, bf16 output) on the same bf16 operands."""
    import torch
    import torch.nn.functional as F
    from joint_attention_dit_amd import binding as B

    M, N, K = cfg.n_tokens, 3 * cfg.attn_width, cfg.hidden
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    res = {}
    for name, fn in (("h3dit_linear_f32", lambda: B.h3dit_linear_f32(x, w, y)),
                     ("torch_linear_hipblaslt", lambda: F.linear(x, w))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms": round(ms, 4), "tflops": round(2.0 * M * N * K / ms / 1e9, 1)}
    return {"shape": [M, N, K], **res}


def measure_ulysses(cfg, G: int, steps: int, warmup: int):
    """One GPU's share of a block under G-way Ulysses sequence parallelism: the
    per-token kernels on T/G tokens (a block of T/G tokens with the same widths),
    attention on H/G heads over all T tokens. The two all-to-alls (q, k, v from
    tokens to heads before attention, o back after it) are not run: one GPU is
    available, so the bytes each GPU would send are reported instead."""
    import dataclasses
    import torch
    from joint_attention_dit_amd import binding as B

    from joint_attention_dit_amd.inputs import CONFIGS

    T, H, A = cfg.n_tokens, cfg.heads, cfg.attn_width
    assert T % G == 0 and H % G == 0, (T, H, G)
    Ts, Hs = T // G, H // G
    if cfg.name == "4096" and f"share{G}" in CONFIGS:
        share = CONFIGS[f"share{G}"]   # the shapes the parity tests check
    else:
        text = cfg.text_tokens // G
        cols = 64
        assert (Ts - text) % cols == 0, (Ts, text)
        rows = (Ts - text) // cols
        share = dataclasses.replace(cfg, name=f"{cfg.name}_share{G}", text_tokens=text,
                                    images=((rows, cols, 0),),
                                    description=f"{cfg.name} share of {G}: {text} text + {rows}x{cols} image tokens")
    assert share.n_tokens == Ts, (share.n_tokens, Ts)
    ms, stage_ms, ok, _ = measure(share, steps, warmup)

    # attention of the share: Hs heads over all T tokens
    acfg = B.make_config(cfg.hidden, Hs, cfg.ffn, T)
    Tp = B.h3dit_padded_tokens(T)
    g = torch.Generator(device="cuda").manual_seed(0)
    qk = torch.randn(T, 2 * Hs * 128, device="cuda", generator=g)
    qk[:, :Hs * 128] *= 12.0 / 128 ** 0.5  # base-2 score spread like the block's (std ~ 12)
    qk = qk.to(torch.bfloat16)
    vt = torch.randn(Hs, 128, Tp, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty(T, Hs * 128, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        B.h3dit_attention(acfg, qk, vt, o, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        B.h3dit_attention(acfg, qk, vt, o, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    att_ms = e0.elapsed_time(e1) / steps
    ok = ok and bool(torch.isfinite(o).all().item())

    kernels = dict(stage_ms)
    kernels["attention"] = att_ms
    total = sum(kernels.values())
    flops = 2.0 * Ts * (3 * A * cfg.hidden + A * cfg.hidden + 2 * cfg.hidden * cfg.ffn) \
        + 4.0 * T * T * Hs * 128 + 2.0 * 6 * cfg.hidden * cfg.hidden
    qkv_bytes = Ts * 3 * A * 2            # this GPU's q, k, v before the first all-to-all
    o_bytes = T * Hs * 128 * 2            # this GPU's attention output before the second
    return {
        "gpus": G, "tokens_per_gpu": Ts, "heads_per_gpu": Hs, "share_workload": share.description,
        "ms_per_block_compute": round(total, 4),
        "tflops_per_gpu": round(flops / (total * 1e-3) / 1e12, 1),
        "pct_bf16_mfma_peak": round(100 * flops / (total * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {k: round(v, 4) for k, v in kernels.items()},
        "alltoall_bytes_sent_per_gpu": {"qkv": qkv_bytes * (G - 1) // G, "o": o_bytes * (G - 1) // G},
        "output_finite": ok,
    }


def stack_flops(scfg) -> float:
    b = scfg.block
    per_eval = scfg.n_blocks * block_flops(b) + 2.0 * 2 * b.image_tokens * b.hidden * scfg.patch_features \
        + 2.0 * 2 * b.hidden * b.hidden
    return per_eval * scfg.steps


def cpu_baseline(cfg, rows: int):
    """Time the float64 oracle on the same block at 1 and at `rows` sampled query rows.

    Keys and values always cover every token, so the cost splits into a part
    shared by all rows (modulation, RMSNorm1, K and V projections) and a part
    per query row; the two timings give both and extrapolate to a whole block.
    """
    from threadpoolctl import threadpool_info

    import oracle as O
    from joint_attention_dit_amd.inputs import make_inputs, sample_rows, to_numpy_f64

    inp = make_inputs(cfg, seed=0)
    w = {k: to_numpy_f64(inp[k]) for k in ("w_ada", "w_qkv", "w_o", "w_up", "w_down")}
    x, cond, pos = to_numpy_f64(inp["x"]), to_numpy_f64(inp["cond"]), inp["positions"].numpy()
    del inp
    times = {}
    for r in (1, rows):
        sel = sample_rows(cfg.n_tokens, r, seed=1)
        t0 = time.perf_counter()
        O.block_forward(x, cond, w, pos, heads=cfg.heads, eps=cfg.eps, rope_base=cfg.rope_base,
                        mode="contract", rows=sel)
        times[r] = time.perf_counter() - t0
    per_row = max(times[rows] - times[1], 0.0) / (rows - 1)
    shared = max(times[1] - per_row, 0.0)
    t_block = shared + per_row * cfg.n_tokens
    threads = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max(threads) if threads else len(os.sched_getaffinity(0))
    return {
        "value": round(cfg.n_tokens / t_block, 2), "unit": "block-tokens/s", "cores": cores,
        "kind": "oracle",
        "sample": (f"float64 oracle (contract mode) on the {cfg.n_tokens}-token block, run with 1 "
                   f"and with {rows} sampled query rows ({times[1]:.2f} s, {times[rows]:.2f} s); "
                   f"all-token part {shared:.2f} s + {per_row * 1e3:.2f} ms per query row, "
                   f"extrapolated to {t_block:.1f} s per whole block"),
        "seconds_measured": round(times[1] + times[rows], 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="4096", choices=["2048", "4096", "edit", "nonsquare", "tiny"])
    ap.add_argument("--extra", default="2048", help="second workload reported under 'extra' ('none' to skip)")
    ap.add_argument("--linears", default="bf16", choices=["bf16", "mxfp8"],
                    help="the block's four linears in bf16 (default) or MXFP8 (OCP MX, E4M3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=384, help="query rows of the oracle sample")
    ap.add_argument("--stack", action="store_true",
                    help="time the full DiT stack (50 blocks, 6 steps at 2048x2048) instead")
    ap.add_argument("--no-mod-table", action="store_true",
                    help="with --stack: compute each block's modulation per step instead of a table")
    ap.add_argument("--ulysses", type=int, default=0, metavar="G",
                    help="time one GPU's share of G-way Ulysses sequence parallelism instead")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="time the QKV-shaped GEMM here and through torch/hipBLASLt (context)")
    ap.add_argument("--attention-cliff", action="store_true",
                    help="time attention on ordinary vs rising scores (the kernel's second pass)")
    ap.add_argument("--traffic-run", action="store_true",
                    help="one 1 GiB copy + one block (the command the HBM counter passes profile)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="per-kernel times of a profiled --extra=none run, warm-ups dropped (host only)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="per-kernel counter averages of profiled --extra=none runs (host only)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two counter passes into the profiles/ summary table (host only)")
    args = ap.parse_args()

    if args.summarize_trace:
        from joint_attention_dit_amd.inputs import CONFIGS
        print(summarize_trace(args.summarize_trace, args.warmup, CONFIGS[args.workload],
                              args.linears))
        return
    if args.summarize_counters:
        from joint_attention_dit_amd.inputs import CONFIGS
        print(summarize_counters(args.summarize_counters, args.warmup, CONFIGS[args.workload]))
        return
    if args.summarize_traffic:
        from joint_attention_dit_amd.inputs import CONFIGS
        print(summarize_traffic(*args.summarize_traffic, CONFIGS[args.workload]))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the block runs on a single MI355X; there is no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from joint_attention_dit_amd.inputs import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = CONFIGS[args.workload]
    if args.traffic_run:
        traffic_run(cfg)
        return
    if args.gemm_reference:
        r = measure_gemm_reference(cfg, args.steps, max(args.warmup, 1))
        print(json.dumps({"metric": "QKV-shaped GEMM time, this library vs hipBLASLt (context)",
                          "config": {"workload": cfg.description}, **r}), flush=True)
        return
    if args.attention_cliff:
        r = measure_attention_cliff(cfg, max(args.steps // 2, 1), max(args.warmup // 2, 1))
        print(json.dumps({
            "metric": "attention time, ordinary scores vs scores rising along the sequence",
            "value": round(r["rising"] / r["ordinary"], 3), "unit": "x (rising / ordinary)",
            "n_gpus": 1, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": cfg.description},
            "ms": {k: round(v, 4) for k, v in r.items()}}), flush=True)
        return
    if args.ulysses:
        G = args.ulysses
        u = measure_ulysses(cfg, G, max(args.steps // 2, 1), max(args.warmup // 2, 1))
        print(json.dumps({
            "metric": f"one GPU's share of a {G}-way Ulysses-parallel block (compute only)",
            "value": round(cfg.n_tokens / (u["ms_per_block_compute"] * 1e-3), 1),
            "unit": "block-tokens/s of the whole job if the all-to-alls are hidden",
            "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": cfg.description}, "ulysses": u}), flush=True)
        return
    if args.stack:
        from joint_attention_dit_amd.inputs import STACK_CONFIGS
        scfg = STACK_CONFIGS["dit_2048"]
        sec, ok = measure_stack(scfg, images=max(args.steps // 10, 1), warmup=1 if args.warmup else 0,
                                mod_table=not args.no_mod_table, linears=args.linears)
        fl = stack_flops(scfg)
        print(json.dumps({
            "metric": "DiT compute images/s (50 blocks x 6 denoising steps, 2048x2048)",
            "modulation": "per-step table" if not args.no_mod_table else "per block call",
            "value": round(1.0 / sec, 4), "unit": "images/s", "n_gpus": 1,
            "ms_per_image": round(sec * 1e3, 2),
            "ms_per_block": round(sec * 1e3 / (scfg.n_blocks * scfg.steps), 4),
            "higher_is_better": True,
            "dtype": "bf16" if args.linears == "bf16" else "mxfp8 linears (e4m3 + e8m0/32), bf16 attention",
            "data": "synthetic (seeded, drawn on the GPU)",
            "config": {"workload": scfg.description, "n_blocks": scfg.n_blocks, "steps": scfg.steps,
                       "n_tokens": scfg.block.n_tokens, "latent": list(scfg.latent_shape)},
            "tflops": round(fl / sec / 1e12, 1),
            "pct_bf16_mfma_peak": round(100 * fl / sec / 1e12 / PEAK_BF16_TFLOPS, 2),
            "output_finite": ok}), flush=True)
        return
    ms, stage_ms, ok, spread = measure(cfg, args.steps, args.warmup, args.linears)
    tflops, kernels, roof = summarize(cfg, ms, stage_ms, args.linears)
    sclk = spread.pop("sclk")

    rec = {
        "metric": METRIC,
        "value": round(cfg.n_tokens / (ms * 1e-3), 1),
        "unit": "block-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "per_step": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.linears == "bf16" else "mxfp8 linears (e4m3 + e8m0/32), bf16 attention",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights)",
        "config": {"workload": cfg.description, "n_tokens": cfg.n_tokens,
                   "image_tokens": cfg.image_tokens, "text_tokens": cfg.text_tokens,
                   "hidden": cfg.hidden, "heads": cfg.heads, "head_dim": cfg.head_dim,
                   "ffn": cfg.ffn},
        "tflops": round(tflops, 1),
        "pct_bf16_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        # the shader clock the chip held during the timed forwards, and the same
        # rate against the dense peak at that clock (the chip lowers its clock
        # under sustained matrix-core load)
        "sclk": sclk,
        "pct_bf16_mfma_peak_at_sclk": (round(100 * tflops / (PEAK_BF16_TFLOPS * sclk["mean_mhz"] / 2400.0), 2)
                                       if sclk else None),
        "image_tokens_per_s": round(cfg.image_tokens / (ms * 1e-3), 1),
        "output_finite": ok,
        "kernels": kernels,
        "roofline": roof,
    }
    if args.extra not in ("", "none") and args.extra != args.workload:
        ecfg = CONFIGS[args.extra]
        ems, est, eok, espread = measure(ecfg, max(args.steps // 2, 1), args.warmup,
                                args.linears)
        etf, ekern, eroof = summarize(ecfg, ems, est, args.linears)
        rec["extra"] = {"workload": ecfg.description, "n_tokens": ecfg.n_tokens,
                        "ms_per_step": round(ems, 4), "per_step": espread, "sclk": espread.pop("sclk"), "value": round(ecfg.n_tokens / (ems * 1e-3), 1),
                        "unit": "block-tokens/s", "tflops": round(etf, 1),
                        "pct_bf16_mfma_peak": round(100 * etf / PEAK_BF16_TFLOPS, 2),
                        "kernels": ekern}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
