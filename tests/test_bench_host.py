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
