"""Host-side checks of bench.py's accounting (no GPU): the FLOP and byte counts
the roofline is priced with, the trace parser, the digest that ties stored
counter figures to the kernel sources, the clock sampler and the one-GPU guard."""
import csv
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from joint_attention_dit_amd.inputs import CONFIGS  # noqa: E402


@pytest.mark.parametrize("name, tflop", [("2048", 3.227), ("4096", 18.603), ("edit", 26.518)])
def test_block_flops(name, tflop):
    # linears 2 T (3 A D + A D + 2 D F), attention 4 T^2 A (two T x T x A products),
    # modulation 2 (6 D) D; D = 5376, A = 56 x 128, F = 14336
    cfg = CONFIGS[name]
    T, D, A, F = cfg.n_tokens, cfg.hidden, cfg.attn_width, cfg.ffn
    assert (D, A, F) == (5376, 7168, 14336)
    total = bench.block_flops(cfg)
    assert abs(total / 1e12 - tflop) < 5e-4 * tflop
    flops, _ = bench.stage_work(cfg)
    assert sum(flops.values()) == pytest.approx(total, rel=1e-12)
    assert flops["attention"] == 4.0 * T * T * A


def test_memory_bound_stage_bytes():
    cfg = CONFIGS["4096"]
    T, D = cfg.n_tokens, cfg.hidden
    _, nbytes = bench.stage_work(cfg)
    assert nbytes["rmsnorm1"] == 4.0 * T * D            # bf16 row in, bf16 row out
    assert nbytes["rmsnorm2"] == 6.0 * T * D            # fp32 row in, bf16 row out
    assert nbytes["modulation"] == 2.0 * 6 * D * D + 4 * D + 8 * 6 * D
    assert round(nbytes["rmsnorm1"] / 1e6, 1) == 363.3
    assert round(nbytes["modulation"] / 1e6, 1) == 347.1


def _write_trace(path, blocks, with_split=True):
    """A kernel-trace CSV of `blocks` block forwards: stage i of block b lasts
    (i + 1) * 1000 + b ns; the QKV GEMM and the attention each add a second
    kernel of 100 ns (K-slice fixup, key-piece merge)."""
    names = {
        "modulation": "h3dit::modulation_lds_kernel", "rope_table": "h3dit::rope_table_kernel",
        "rmsnorm1": "h3dit::rmsnorm_modulate_lds_kernel", "qkv_rope_gemm": "h3dit::gemm_kernel<0>",
        "attention": "h3dit::attention_kernel<false>", "out_proj_gemm": "h3dit::gemm_kernel<1>",
        "rmsnorm2": "h3dit::rmsnorm_modulate_lds_kernel", "mlp_up_gelu_gemm": "h3dit::gemm_kernel<3>",
        "mlp_down_gemm": "h3dit::gemm_kernel<2>",
    }
    rows, did, t = [], 1, 0
    for b in range(blocks):
        for i, stage in enumerate(bench.KERNEL_ORDER):
            d = (i + 1) * 1000 + b
            rows.append((did, names[stage], t, t + d))
            did += 1
            t += d + 10
            if with_split and stage in ("qkv_rope_gemm", "attention"):
                second = "h3dit::gemm_fixup_kernel<0, 8>" if stage == "qkv_rope_gemm" else \
                    "h3dit::attention_merge_kernel"
                rows.append((did, second, t, t + 100))
                did += 1
                t += 110
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)


def test_trace_summary_merges_second_kernels(tmp_path):
    _write_trace(tmp_path / "x_kernel_trace.csv", blocks=5)
    out = bench.summarize_trace(str(tmp_path), 2, CONFIGS["4096"])
    rec = bench.json.loads(out.split("```json", 1)[1].split("```", 1)[0])
    # blocks 2, 3, 4 are kept: stage i averages (i + 1) * 1000 + 3 ns, plus 100 ns
    # for the QKV GEMM's fixup and the attention's merge
    for i, stage in enumerate(bench.KERNEL_ORDER):
        extra = 100 if stage in ("qkv_rope_gemm", "attention") else 0
        assert rec[stage]["avg_us"] == pytest.approx(((i + 1) * 1000 + 3 + extra) * 1e-3, abs=1e-2)
    assert "Timed block forwards: 3" in out


def test_trace_summary_rejects_partial_blocks(tmp_path):
    _write_trace(tmp_path / "x_kernel_trace.csv", blocks=2)
    with open(tmp_path / "x_kernel_trace.csv") as f:
        lines = f.readlines()
    with open(tmp_path / "x_kernel_trace.csv", "w") as f:
        f.writelines(lines[:-1])  # the last block loses its last kernel
    with pytest.raises(AssertionError):
        bench.summarize_trace(str(tmp_path), 0, CONFIGS["4096"])


def test_source_digest_follows_included_headers(tmp_path, monkeypatch):
    csrc = os.path.join(ROOT, "joint_attention_dit_amd", "csrc")
    dst = tmp_path / "joint_attention_dit_amd" / "csrc"
    shutil.copytree(csrc, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {s: bench.source_digest(s) for s in ("attention", "qkv_rope_gemm", "modulation")}
    assert before == {s: bench.source_digest(s) for s in before}
    with open(dst / "gemm_common.h", "a") as f:  # included by the GEMM only
        f.write("\n// changed\n")
    after = {s: bench.source_digest(s) for s in before}
    assert after["qkv_rope_gemm"] != before["qkv_rope_gemm"]
    assert after["attention"] == before["attention"]
    with open(dst / "common.h", "a") as f:  # included by every kernel
        f.write("\n// changed\n")
    assert all(bench.source_digest(s) != after[s] for s in before)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_clock_sampler_reads_the_marked_level(tmp_path):
    dev = tmp_path / "card0" / "device"
    (dev / "hwmon" / "hwmon3").mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1821Mhz *\n2: 2400Mhz\n")
    (dev / "hwmon" / "hwmon3" / "power1_input").write_text("1161800000\n")
    c = bench.ClockSampler(period_s=0.001, root=str(tmp_path))
    c._read()
    c._read()
    out = c.summary()
    assert out["mean_mhz"] == 1821 and out["min_mhz"] == 1821 and out["samples"] == 2
    assert out["mean_board_power_w"] == pytest.approx(1161.8)
    assert bench.ClockSampler(root=str(tmp_path / "none")).summary() is None
