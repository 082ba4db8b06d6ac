"""Host-side summaries of rocprofv3 output (profiling.py) on small synthetic CSVs."""

import csv
import os

import pytest

from ring_attention_blockwise_ra_amd import profiling as P


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_counts_copy_time_under_attention(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    rows = [
        dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=100, End_Timestamp=200),
        dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=300, End_Timestamp=400),
        # side-queue copies: fully under the first launch, half under the second, outside
        dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=2, Start_Timestamp=120, End_Timestamp=160),
        dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=2, Start_Timestamp=380, End_Timestamp=420),
        dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=2, Start_Timestamp=500, End_Timestamp=510),
        # a copy on the attention queue is not a staging copy
        dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=1, Start_Timestamp=210, End_Timestamp=290),
    ]
    _write(str(tmp_path / "t.csv"), rows)
    _write(str(tmp_path / "s.csv"), [dict(Name=attn, Calls=2, AverageNs=100.0, TotalDurationNs=200.0,
                                          Percentage=50.0)])
    s = P.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "s.csv"))
    assert s["staging_copies"] == 3
    assert s["staging_copy_ms"] == pytest.approx(90e-6)
    assert s["staging_copy_hidden_ms"] == pytest.approx(60e-6)
    assert s["staging_copy_hidden_frac"] == pytest.approx(60 / 90)
    (st,) = s["kernels"].values()
    assert st["calls"] == 2 and st["avg_ms"] == pytest.approx(1e-4)


def test_traffic_scales_by_calibration_copy(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    for counter, d, calib_kib, per in (("FETCH_SIZE", "f", 2 * 1024 * 1024, [300.0, 500.0]),
                                       ("WRITE_SIZE", "w", 1024 * 1024, [100.0, 100.0])):
        rows = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=counter,
                     Counter_Value=calib_kib),
                dict(Dispatch_Id=2, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=counter,
                     Counter_Value=10.0)]
        # the second attention dispatch reports two instances that are summed
        rows += [dict(Dispatch_Id=3, Kernel_Name=attn, Counter_Name=counter, Counter_Value=per[0]),
                 dict(Dispatch_Id=4, Kernel_Name=attn, Counter_Name=counter, Counter_Value=per[1] / 2),
                 dict(Dispatch_Id=4, Kernel_Name=attn, Counter_Name=counter, Counter_Value=per[1] / 2),
                 dict(Dispatch_Id=5, Kernel_Name="ra::merge_partials_kernel(long)", Counter_Name=counter,
                      Counter_Value=64.0)]
        _write(str(tmp_path / d / "x_counter_collection.csv"), rows)
    t = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), 1 << 30)
    # FETCH reads 2 GiB for the 1 GiB copy: factor 1/2
    assert t["FETCH_SIZE"]["factor"] == pytest.approx(0.5)
    assert t["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(400.0 * 1024 * 0.5)
    assert t["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(100.0 * 1024)
    assert t["hbm_bytes_per_launch"] == pytest.approx(400.0 * 512 + 100.0 * 1024)
    assert t["merge"]["FETCH_SIZE"]["launches"] == 1
    assert t["merge"]["hbm_bytes_per_launch"] == pytest.approx(64.0 * 512 + 64.0 * 1024)


def test_sq_summary_busy_fraction_and_clock(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    # two dispatches of 1 ms each; 8 XCDs at 2 GHz -> 2e6 cycles per XCD each
    rows = []
    for did, (s, e) in ((1, (0, 1_000_000)), (2, (2_000_000, 3_000_000))):
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 2e6), ("SQ_INSTS_MFMA", 1000.0),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 2e6 * 1024), ("SQ_INSTS_VALU", 6000.0),
                          ("SQ_INSTS_LDS", 1500.0)):
            rows.append(dict(Dispatch_Id=did, Kernel_Name=attn, Counter_Name=name, Counter_Value=val,
                             Start_Timestamp=s, End_Timestamp=e))
    rows.append(dict(Dispatch_Id=3, Kernel_Name="other", Counter_Name="SQ_INSTS_MFMA", Counter_Value=9e9,
                     Start_Timestamp=0, End_Timestamp=1))
    _write(str(tmp_path / "r" / "x_counter_collection.csv"), rows)
    _write(str(tmp_path / "r" / "x_agent_info.csv"),
           [dict(Name="cpu", Simd_Count=0, Num_Xcc=0), dict(Name="gfx950", Simd_Count=1024, Num_Xcc=8)])
    s = P.sq_summary(str(tmp_path / "r"))
    assert s["dispatches"] == 2
    assert s["engine_clock_ghz"] == pytest.approx(2.0)
    assert s["mfma_busy_frac"] == pytest.approx(0.5)
    assert s["mfma_executed_flops"] == 2000 * 32 * 32 * 16 * 2
    assert s["sq_insts_valu_per_mfma"] == pytest.approx(6.0)
    assert s["sq_insts_lds_per_mfma"] == pytest.approx(1.5)


def test_trace_summary_checks_launches_fit_the_step(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    rows = [dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=0, End_Timestamp=2_000_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=3_000_000, End_Timestamp=7_000_000)]
    _write(str(tmp_path / "t.csv"), rows)
    _write(str(tmp_path / "s.csv"), [dict(Name=attn, Calls=2, AverageNs=3e6, TotalDurationNs=6e6,
                                          Percentage=100.0)])
    s = P.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "s.csv"), 6.5, 2)
    assert s["attention_avg_ms"] == pytest.approx(3.0)
    assert s["attention_ms_per_step"] == pytest.approx(6.0)
    with pytest.raises(ValueError):
        P.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "s.csv"), 5.9, 2)


def test_overlap_summary_splits_staged_and_nocopy_runs(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    rows = []
    t = 0
    for run, dur in enumerate([10, 11, 10, 10, 12, 10]):  # staged, nocopy, staged, ...
        for _ in range(2):
            rows.append(dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=t * 1000,
                             End_Timestamp=(t + dur) * 1000))
            if run % 2 == 0:
                rows.append(dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=2,
                                 Start_Timestamp=(t + 1) * 1000, End_Timestamp=(t + 3) * 1000))
            t += dur + 1
    _write(str(tmp_path / "t.csv"), rows)
    o = P.overlap_summary(str(tmp_path / "t.csv"), 2)
    assert o["runs"] == {"staged": 3, "nocopy": 3}
    assert o["mean_attention_ms"]["staged"] == pytest.approx(2 * (10 + 10 + 12) / 3 / 1000)
    assert o["mean_attention_ms"]["nocopy"] == pytest.approx(2 * (11 + 10 + 10) / 3 / 1000)
    assert o["staged_minus_nocopy_ms"] == pytest.approx(2 * (32 - 31) / 3 / 1000)
    assert o["staging_copies"] == 6
    # interleaved pairs (staged run, then its no-copy run): 2 x (10-11, 10-10, 12-10) us
    pr = o["paired"]
    assert pr["pairs"] == 3
    assert pr["attention_diff_ms"] == pytest.approx([-2e-3, 0.0, 4e-3])
    assert pr["attention_diff_ms_median"] == pytest.approx(0.0)
    assert pr["attention_diff_ms_range"] == pytest.approx([-2e-3, 4e-3])
    assert pr["copy_ms_per_staged_run"] == pytest.approx(4e-3)   # two 2-us copies per run
    assert pr["efficiency"] == pytest.approx(1.0)


def test_overlap_summary_queue_idle(tmp_path):
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    merge = "ra::merge_partials_kernel(long)"
    # staged run: attn 0-10, gap 2, merge 12-13, gap 1, attn 14-24; copy on queue 2
    # no-copy run: attn 30-40, merge 40-41, attn 41-51 (no gaps)
    rows = [dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=0, End_Timestamp=10_000),
            dict(Kernel_Name=merge, Queue_Id=1, Start_Timestamp=12_000, End_Timestamp=13_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=14_000, End_Timestamp=24_000),
            dict(Kernel_Name="__amd_rocclr_copyBuffer", Queue_Id=2, Start_Timestamp=1_000,
                 End_Timestamp=3_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=30_000, End_Timestamp=40_000),
            dict(Kernel_Name=merge, Queue_Id=1, Start_Timestamp=40_000, End_Timestamp=41_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=41_000, End_Timestamp=51_000)]
    _write(str(tmp_path / "t.csv"), rows)
    o = P.overlap_summary(str(tmp_path / "t.csv"), 2)
    assert o["runs"] == {"staged": 1, "nocopy": 1}
    assert o["mean_queue_idle_ms"]["staged"] == pytest.approx(3e-3)
    assert o["mean_queue_idle_ms"]["nocopy"] == pytest.approx(0.0)
    assert o["queue_idle_staged_minus_nocopy_ms"] == pytest.approx(3e-3)
    pr = o["paired"]
    assert pr["pairs"] == 1 and pr["queue_idle_diff_ms_median"] == pytest.approx(3e-3)
    # attention time equal (20 us each); the 3 us of idle cost against 2 us of copies
    assert pr["cost_ms"] == pytest.approx(3e-3) and pr["efficiency"] == pytest.approx(-0.5)


def test_staging_copy_kernel_counts_as_a_copy(tmp_path):
    """The ring stages K and V with its own copy kernel; the summaries count it
    as a staging copy like the runtime's copy."""
    attn = "void ra::attn_bf16_mfma<128, 8>(ra::AttnParams)"
    stage = "ra::copy2_kernel(long, unsigned int __vector(4) const*, ...)"
    rows = [dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=0, End_Timestamp=10_000),
            dict(Kernel_Name=stage, Queue_Id=2, Start_Timestamp=1_000, End_Timestamp=3_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=10_000, End_Timestamp=20_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=30_000, End_Timestamp=40_000),
            dict(Kernel_Name=attn, Queue_Id=1, Start_Timestamp=40_000, End_Timestamp=50_000)]
    _write(str(tmp_path / "t.csv"), rows)
    o = P.overlap_summary(str(tmp_path / "t.csv"), 2)
    assert o["runs"] == {"staged": 1, "nocopy": 1}
    assert o["staging_copies"] == 1 and o["staging_copy_ms"] == pytest.approx(2e-3)
