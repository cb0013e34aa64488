"""The benchmark's work accounting (no GPU): the algorithmic bytes and flops
its rooflines divide by the measured launch times.

Bytes are checked against an independent list of the tensors each call must
touch once, flops against the MFMA operation counts the hardware reported for
these kernels at the Qwen3-30B-A3B shape (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512,
recorded with the GEMMs' profiles), and the roofline's bound against the
ridge point of the stated peaks.
"""
import json
import os

import bench
import moe_inputs

QWEN = moe_inputs.WORKLOADS["qwen3_30b_a3b_n4096_h2048_e128_k8"]
BF16, I32, F32 = 2, 4, 4

# hardware-counted bf16 MFMA operations per launch at the Qwen shape
MFMA_FC1 = 402_653_184 * 512
MFMA_FC2 = 201_326_592 * 512


def _tensor_bytes(*shapes_and_sizes):
    total = 0
    for size, *dims in shapes_and_sizes:
        n = size
        for d in dims:
            n *= d
        total += n
    return total


def test_forward_bytes_enumerate_the_tensors():
    w, C = QWEN, 256
    Cp = C
    R = w.E * Cp
    kept = 31_000
    got = bench.algorithmic_bytes(w, C, Cp, kept)
    fc1 = _tensor_bytes((BF16, w.E, 2 * w.I, w.H),      # W1
                        (BF16, w.N, w.H),               # x, each token row once
                        (I32, R), (F32, R),             # route list and slot probabilities
                        (BF16, R, w.I))                 # act written
    fc2 = _tensor_bytes((BF16, w.E, w.H, w.I),          # W2
                        (BF16, R, w.I),                 # act read
                        (BF16, R, w.H))                 # route_out written
    combine = _tensor_bytes((BF16, kept, w.H),          # each kept route's row once
                            (I32, w.N, w.K),            # token_routes
                            (BF16, w.N, w.H))           # y written
    assert got["fc1"] == fc1 == 872_677_376
    assert got["fc2"] == fc2 == 587_202_560
    assert got["combine"] == combine


def test_gemm_flops_equal_the_counted_mfma_work():
    w, Cp = QWEN, 256
    work = bench.backward_work(w, Cp, kept=31_000)
    for name in ("fc1_save", "fc1_dgrad", "fc1_wgrad"):
        assert work[name][0] == MFMA_FC1, name
    for name in ("fc2", "fc2_dgrad", "fc2_wgrad"):
        assert work[name][0] == MFMA_FC2, name
    # the forward's own figures (bench main) use 2*E*Cp*2I*H and 2*E*Cp*H*I
    assert 2 * w.E * Cp * 2 * w.I * w.H == MFMA_FC1
    assert 2 * w.E * Cp * w.H * w.I == MFMA_FC2


def test_roofline_bound_follows_the_ridge():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)     # flop per byte
    assert 300 < ridge < 320
    # FC1 at the Qwen shape: AI 236 < ridge, HBM-bound
    r = bench.roofline("fc1", MFMA_FC1, 872_677_376, 180.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - 872_677_376 / 180e-6 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / bench.PEAK_HBM_GBS) < 1e-12
    assert r["arithmetic_intensity"] < ridge
    # an expert-parallel rank's FC1 (16 experts x 2048 rows): AI above the ridge
    rows, H, I, El = 16 * 2048, 2048, 768, 16
    flops = 2 * rows * 2 * I * H
    nbytes = El * 2 * I * H * 2 + rows * H * 2 + rows * I * 2
    r = bench.roofline("fc1 ep8", flops, nbytes, 176.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - flops / 176e-6 / 1e12 / bench.PEAK_BF16_TFLOPS) < 1e-12


def test_counter_traffic_only_for_its_workload():
    path = bench.PMC_SUMMARY
    assert os.path.exists(path)
    d = json.load(open(path))
    assert bench.pmc_traffic("deepseek_wide_n8192_h7168_e256_k8") is None
    t = bench.pmc_traffic(d["workload"])
    if d.get("kernel_source_sha") == bench.kernel_source_hash():
        # scaled FETCH + WRITE per launch: at least the algorithmic bytes
        assert t is not None and t >= 872_677_376
    else:
        assert t is None
