"""Host-side checks of the profile-summary helpers that feed bench.py's roofline.traffic."""
import json
import os
import sys

from selective_recompute_cf_amd import profiles

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_short_names():
    assert profiles.short_name("void cf::gemm_bf16_dtl<cf::DtlCfg<128, 256, 2, 4, 3, 1> >(cf::GemmArgs)") == \
        "cf::gemm_bf16_dtl<cf::DtlCfg<128, 256, 2, 4, 3, 1> >"
    assert profiles.short_name("_ZN2cf15qkv_post_kernelIDF16bEEvNS_7QkvPostE") == "cf::qkv_post_kernel<__bf16>"


def test_counter_parsing_and_copy_factor(tmp_path):
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name,"
           "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name,"
           "Counter_Value,Start_Timestamp,End_Timestamp\n")
    p = tmp_path / "c.csv"
    rows = [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0), (1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0),
            (2, "void cf::gemm_bf16_dtl<X>(cf::GemmArgs)", "FETCH_SIZE", 100.0)]
    p.write_text(hdr + "".join(f'{d},{d},"Agent 1",1,1,1,1,1,"{n}",256,0,0,8,0,16,"{c}",{v},0,1\n'
                               for d, n, c, v in rows))
    # two counter rows of one dispatch add up (per-XCD instances); 1 MiB copy -> 1024 KiB counted
    assert profiles.counter_per_dispatch(str(p), "FETCH_SIZE", "gemm") == [("cf::gemm_bf16_dtl<X>", 100.0)]
    assert abs(profiles.copy_factor(str(p), "FETCH_SIZE", 1 << 20) - 1.0) < 1e-12


def test_committed_traffic_summary_is_well_formed():
    path = os.path.join(ROOT, "profiles", "gemm_bf16_dtl_llama3-8b_hbm_traffic.json")
    with open(path) as f:
        t = json.load(f)
    for key in ("source_sha256", "fetch_bytes_per_launch", "write_bytes_per_launch", "traffic_bytes_per_launch",
                "fetch_factor", "write_factor", "command"):
        assert key in t
    assert t["traffic_bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert len(profiles.sources_sha256()) == 64


def test_copy_overlap_summary(tmp_path, monkeypatch):
    """Hand-worked traces: kernels busy on [0, 100) and [150, 300) ns; copies on [50, 170)
    (70 of 120 covered) and [320, 340) (none); one side kernel on [90, 160) (20 of 70 covered,
    and not part of the busy union itself); nothing before the start kernel counts."""
    kt = tmp_path / "k.csv"
    cp = tmp_path / "c.csv"
    kt.write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n"
                  "early,-50,-10\nembed_kernel,0,40\ngemm,30,100\ngemm,150,300\nreposition_kernel,90,160\n")
    cp.write_text("Direction,Start_Timestamp,End_Timestamp\n"
                  "MEMORY_COPY_HOST_TO_DEVICE,-40,-20\nMEMORY_COPY_HOST_TO_DEVICE,50,170\n"
                  "MEMORY_COPY_DEVICE_TO_HOST,0,500\nMEMORY_COPY_HOST_TO_DEVICE,320,340\n")
    out = tmp_path / "o.md"
    monkeypatch.setattr(sys, "argv", ["profiles", "overlap", str(kt), str(cp), str(out), "--start", "embed_kernel",
                                      "--side", "reposition", "--command", "x"])
    profiles.main()
    text = out.read_text()
    assert "Host-to-device copies: 2, 0.00 ms in total" in text
    assert "(50.0%)" in text  # (70 + 0) / (120 + 20)
    assert "(28.6%)" in text  # (10 + 10) / 70
    assert profiles._covered(profiles._union([(0, 100), (150, 300), (30, 60)]), 50, 170) == 70


def test_counter_shares(tmp_path, monkeypatch):
    """Derived shares on hand-made passes: one 10 us dispatch with 12 288 000 MFMA-busy SIMD cycles
    (= half of 10 us x 2.4 GHz x 1024 SIMDs), 300 of 1000 wave cycles waiting, 25 of 100 LDS cycles
    in bank conflicts, 8 VALU instructions per 2 MFMA."""
    head = "Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    p1 = tmp_path / "p1.csv"
    p2 = tmp_path / "p2.csv"
    p1.write_text(head + "".join(f"attn_dtl_kernel,{c},{v},0,10000\n" for c, v in
                                 [("SQ_VALU_MFMA_BUSY_CYCLES", 12288000), ("SQ_WAVE_CYCLES", 1000),
                                  ("SQ_WAIT_INST_ANY", 300), ("SQ_INSTS_MFMA", 2)]) + "other,SQ_WAVE_CYCLES,5,0,1\n")
    p2.write_text(head + "".join(f"attn_dtl_kernel,{c},{v},0,10000\n" for c, v in
                                 [("SQ_LDS_IDX_ACTIVE", 100), ("SQ_LDS_BANK_CONFLICT", 25), ("SQ_INSTS_VALU", 8)]))
    out = tmp_path / "c.md"
    monkeypatch.setattr(sys, "argv", ["profiles", "counters", str(p1), str(p2), "--out", str(out), "--group",
                                      "attention=attn_dtl", "--command", "x"])
    profiles.main()
    assert "| attention | 1 | 50.0% | 30.0% | 25.0% | 4.00 |" in out.read_text()


def test_stats_group_and_tail_window(tmp_path, monkeypatch):
    """Kernel statistics with a group total, and the group's last dispatches in the trace (the event-timed
    steps run last): two GEMM launches of 10 and 30 us in the statistics average 20 us; in the trace the
    last two of three GEMM dispatches (by start time, not file order) last 40 and 20 us, average 30 us."""
    stats = tmp_path / "s.csv"
    stats.write_text("Name,Calls,TotalDurationNs,AverageNs,Percentage\n"
                     "void cf::gemm_bf16_dtl<X>(cf::GemmArgs),2,40000,20000,80\n"
                     "cf::attn_dtl_kernel(cf::AttnArgs),1,10000,10000,20\n")
    trace = tmp_path / "t.csv"
    trace.write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n"
                     "void cf::gemm_bf16_dtl<X>(cf::GemmArgs),500,20500\n"
                     "void cf::gemm_bf16_dtl<X>(cf::GemmArgs),0,10000\n"
                     "cf::attn_dtl_kernel(cf::AttnArgs),100000,900000\n"
                     "void cf::gemm_bf16_dtl<X>(cf::GemmArgs),100,40100\n")
    out = tmp_path / "o.md"
    monkeypatch.setattr(sys, "argv", ["profiles", "stats", str(stats), str(out), "--group", "gemm_bf16_dtl",
                                      "--tail-trace", str(trace), "--tail", "2", "--command", "x"])
    profiles.main()
    text = out.read_text()
    assert "together: 2 calls, 0.040 ms, average 20.00 us per launch." in text
    assert "The last 2 of them in the kernel trace" in text and "average 30.00 us per launch." in text
