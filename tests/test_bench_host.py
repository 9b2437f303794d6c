"""Host-side checks of the benchmark's bookkeeping (no GPU): the MFMA peak each kernel is
measured against, and the HBM-traffic records kept under profiles/ (each names its kernel
and the hash of the sources it was measured with)."""
import glob
import json
import os

import bench
from decoder_only_transformer_05_amd import profsum


def test_peaks_follow_the_kernels_arithmetic():
    assert bench.mfma_peak("gemm_kernel<1,1,0>") == bench.PEAK_TFLOPS_FP32_MFMA
    assert bench.mfma_peak("attn_bwd_dkdv_kernel") == bench.PEAK_TFLOPS_FP32_MFMA
    # split-operand fp32 kernels: the published fp32 peak for their fp32 results, plus the
    # bf16 MFMA products they execute (six per fp32 product) against the bf16 peak
    for name in ("gemm_x6_kernel<256,1,1,0>", "gemm_x6_kernel<192,0,0,2>",
                 "attn_fwd_x6_kernel", "attn_bwd_dq_x6_kernel"):
        assert bench.mfma_peak(name) == bench.PEAK_TFLOPS_FP32_MFMA
        ex = bench.executed_mfma(name, 200.0)
        assert ex["achieved"] == 1200.0 and ex["peak"] == bench.PEAK_TFLOPS_BF16_MFMA
    assert bench.executed_mfma("gemm_kernel<1,1,0>", 100.0) is None
    assert bench.mfma_peak("gemm_bf16_kernel<TileCfg<256,256,64,2,4,2,1,8>,1,1,1,0>") == \
        bench.PEAK_TFLOPS_BF16_MFMA
    assert bench.mfma_peak("attn_fwd_bf16mma_kernel") == bench.PEAK_TFLOPS_BF16_MFMA
    assert bench.mfma_peak("layernorm_fwd_kernel") is None
    assert bench.mfma_peak("attn_bwd_rowdot_kernel") is None
    r = bench.roofline_of("gemm_x6_kernel<256,1,1,0>",
                          {"flop": 2e12, "ms": 10.0, "bytes": 1e9, "launches": 10})
    assert r["peak"] == 157.3 and abs(r["achieved"] - 200.0) < 1e-9
    assert abs(r["mfma_executed"]["frac"] - 1200.0 / 2516.6) < 1e-4


def test_host_info_and_clock_parsing():
    h = bench.host_info()
    assert h["nproc"] and h["ram_gib"]
    reply = {"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": 2400, "unit": "MHz"}},
                                               "mem_0": {"clk": {"value": 1900}}}}]}
    f = bench._clock_fields(reply)
    assert f == {"gpu_data.0.clock.gfx_0.clk.value": 2400.0}


def test_traffic_records_are_current():
    """Every traffic record matches the sources it covers, so the benchmark reports it."""
    paths = glob.glob(os.path.join(bench.ROOT, "profiles", "*_hbm_traffic.json"))
    assert paths
    for p in paths:
        with open(p) as f:
            rec = json.load(f)
        assert rec["source_sha256"] == profsum.source_hash(rec["kernel"]), p
        assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + \
            rec["write_bytes_per_launch"]
        workload = os.path.basename(p).split("_hbm_traffic")[0]
        workload = workload[len("".join(c if c.isalnum() else "_"
                                        for c in rec["kernel"]).strip("_")) + 1:]
        assert bench.measured_traffic(rec["kernel"], workload) == rec["bytes_per_launch"]


def _counter_csv(path, counter, rows):
    """A rocprofv3 counter_collection.csv with the columns profsum reads."""
    with open(path, "w") as fh:
        fh.write('"Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        for name, value, t0, t1 in rows:
            fh.write(f'"{name}","{counter}",{value},{t0},{t1}\n')


def test_profsum_tables(tmp_path):
    # mangled _Float16 instances are named as the profiler names the others
    assert profsum.short_name(
        "_ZN4gpt212_GLOBAL__N_117xent_fused_kernelIDF16_Li13ELi0EEEvPfS2_PT_PKS3_PKifPKfiiPi"
    ) == "xent_fused_kernel<_Float16,13,0>"
    assert profsum.short_name(
        "void gpt2::(anonymous namespace)::gemm_x6_kernel<256, true, true, 0>(gpt2::Args)"
    ) == "gemm_x6_kernel<256,1,1,0>"
    # traffic: counters in KiB per dispatch, scaled by the copy calibration (fetch reads half),
    # joined with the launch profile's algorithmic bytes (by name, else without template args)
    k = "void gpt2::(anonymous namespace)::adamw_kernel<unsigned short>(float*)"
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(k, 1000.0, 0, 1), (k, 1000.0, 2, 3)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(k, 1500.0, 0, 1), (k, 1500.0, 2, 3)])
    _counter_csv(tmp_path / "cf.csv", "FETCH_SIZE", [("copy", 512.0, 0, 1)])
    _counter_csv(tmp_path / "cw.csv", "WRITE_SIZE", [("copy", 1024.0, 0, 1)])
    with open(tmp_path / "kt.json", "w") as fh:
        json.dump({"kernels": {"adamw_kernel": {"bytes": 2 * 2.5e6, "launches": 2}}}, fh)
    out = tmp_path / "t.md"
    profsum.traffic_md(str(out), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                       str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1048576.0, "cmd",
                       str(tmp_path / "kt.json"))
    row = [l for l in out.read_text().splitlines() if l.startswith("| adamw_kernel")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "2.05" and cells[3] == "1.54"  # MB per launch
    assert cells[4] == "2.50" and cells[5] == "1.43"
    # MFMA busy: GRBM_GUI_ACTIVE summed over 8 XCDs; busy cycles over cycles x 1024 SIMDs
    g = "void gpt2::(anonymous namespace)::gemm_x6_kernel<256, true, true, 0>(gpt2::Args)"
    with open(tmp_path / "m.csv", "w") as fh:
        fh.write('"Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        fh.write(f'"{g}","GRBM_GUI_ACTIVE",{8 * 1000},0,500\n')
        fh.write(f'"{g}","SQ_VALU_MFMA_BUSY_CYCLES",{1024 * 600},0,500\n')
        fh.write(f'"{g}","SQ_INSTS_VALU_MFMA_MOPS_BF16",{1024 * 1024 * 600 / 512},0,500\n')
    profsum.mfma_md(str(tmp_path / "m.md"), str(tmp_path / "m.csv"), "cmd")
    row = [l for l in (tmp_path / "m.md").read_text().splitlines() if l.startswith("| gemm")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "60.0" and cells[3] == "60.0" and cells[8] == "2.00"
