"""bench.py's host-only paths: the rocprofv3 counter summary and the refusal
of more than one GPU (no GPU needed)."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _write_counters(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_takes_the_last_dispatch_and_derives_ratios(tmp_path):
    import bench
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    # dispatch 1 is an earlier launch of the same kernel; dispatch 2 is the one summarised;
    # values of one counter over several units are summed
    _write_counters(a, [
        dict(Dispatch_Id=1, Kernel_Name="k_attn_fwd", Counter_Name="SQ_INSTS_MFMA", Counter_Value=1),
        dict(Dispatch_Id=2, Kernel_Name="k_attn_fwd", Counter_Name="SQ_INSTS_MFMA", Counter_Value=60),
        dict(Dispatch_Id=2, Kernel_Name="k_attn_fwd", Counter_Name="SQ_INSTS_MFMA", Counter_Value=40),
        dict(Dispatch_Id=2, Kernel_Name="k_attn_fwd", Counter_Name="SQ_INSTS_VALU", Counter_Value=300),
        dict(Dispatch_Id=2, Kernel_Name="other", Counter_Name="SQ_INSTS_VALU", Counter_Value=7),
        dict(Dispatch_Id=2, Kernel_Name="k_attn_fwd", Counter_Name="SQ_WAVE_CYCLES", Counter_Value=1000),
        dict(Dispatch_Id=2, Kernel_Name="k_attn_fwd", Counter_Name="SQ_WAIT_ANY", Counter_Value=250),
    ])
    _write_counters(b, [
        dict(Dispatch_Id=5, Kernel_Name="k_attn_fwd", Counter_Name="TCC_HIT_sum", Counter_Value=75),
        dict(Dispatch_Id=5, Kernel_Name="k_attn_fwd", Counter_Name="TCC_MISS_sum", Counter_Value=25),
    ])
    out = str(tmp_path / "s.md")
    bench.summarize_counters([a, b], "attn_fwd", out, ["cmd one", "cmd two"])
    text = open(out).read()
    assert "| `SQ_INSTS_MFMA` | 100 |" in text
    assert "| `SQ_INSTS_VALU` | 300 |" in text
    assert "| SQ_INSTS_VALU per MFMA | 3 |" in text
    assert "| waves waiting on a memory counter | 0.25 |" in text
    assert "| L2 hit rate | 0.75 |" in text
    assert "    cmd one" in text and "    cmd two" in text


def test_counter_clock_from_grbm_cycles_and_the_code_hash(tmp_path, monkeypatch):
    """The shader clock of a dispatch is GRBM_GUI_ACTIVE per XCD over its
    duration; bench takes it for the at-clock fraction only from a summary of
    the same kernel code."""
    import bench
    a = str(tmp_path / "a")
    # 8 XCDs x 1.8e6 cycles in 1 ms: 1800 MHz
    _write_counters(a, [dict(Dispatch_Id=3, Kernel_Name="attn_fwd_kernel<LatentCfg, 0>", Counter_Name="GRBM_GUI_ACTIVE",
                             Counter_Value=1.8e6, Start_Timestamp=1000, End_Timestamp=1000 + 1000000)] * 8)
    out = str(tmp_path / "c.md")
    bench.summarize_counters([a], "LatentCfg, 0", out, ["cmd"])
    text = open(out).read()
    assert "| shader clock over the dispatch (MHz) | 1800 |" in text
    assert f"Kernel code hash: `{bench.kernel_hash()}`" in text
    assert bench.counter_clock(out) == 1800.0
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.counter_clock(out) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_clock_sampler_reads_the_marked_level(tmp_path, monkeypatch):
    """The engine clock is the level pp_dpm_sclk marks with '*'; samples
    below 1 GHz (idle gaps) are left out of the summary."""
    import time
    import bench
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1834Mhz *\n2: 2400Mhz\n")
    monkeypatch.setattr(bench, "SCLK_FILES", (str(f),))
    with bench.ClockSampler(period_s=0.001) as clk:
        time.sleep(0.02)
        f.write_text("0: 500Mhz\n1: 189Mhz *\n2: 2400Mhz\n")
        time.sleep(0.02)
    s = clk.summary()
    assert s["median_mhz"] == 1834 and s["min_mhz"] == 1834 and s["samples"] >= 2
    assert 189 in clk.mhz
    monkeypatch.setattr(bench, "SCLK_FILES", (str(tmp_path / "missing"),))
    with bench.ClockSampler() as clk:
        pass
    assert clk.summary() is None
