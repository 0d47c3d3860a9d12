"""Host checks of the figures bench.py reports (no GPU): the matrix-flop
counts behind ``mfma_frac``, the bound a roofline takes from its arithmetic
intensity, the fraction of the measured read ceiling, the per-step
algorithmic bytes, and the source hashes that decide whether a committed
counter summary still applies."""

import numpy as np

import bench
from workloads import get_workload


def test_step_flops_counts_both_products_per_query_head():
    w = get_workload("mla_bf16_bimodal")
    # QK^T over 576 dims and PV over 512 dims, 2 flops per multiply-add, 128 heads
    assert bench.step_flops(w, 1) == 2 * 128 * (576 + 512) == 278_528
    g = get_workload("gqa_fp8_binned")
    assert bench.step_flops(g, 10) == 10 * 2 * 64 * (128 + 128)


def test_verify_flops_matches_brute_force_over_query_tokens():
    w = get_workload("gqa_bf16_32k")
    rng = np.random.default_rng(3)
    for q_len in (1, 2, 4, 7):
        lens = rng.integers(q_len, 5000, size=9)
        seen = sum(int(L) - q_len + i + 1 for L in lens for i in range(q_len))
        assert bench.verify_flops(w, lens, q_len) == 2 * seen * w.num_q_heads * (w.head_dim_k + w.head_dim_v)
    # one query token: the decode count
    assert bench.verify_flops(w, [100, 7], 1) == bench.step_flops(w, 107)


def test_roofline_bound_follows_the_ridge():
    ridge = bench.BF16_MFMA_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)   # flop per byte
    assert abs(ridge - 312.5) < 1e-9
    kv, ms = 10 ** 9, 1.0
    below = bench.attn_roofline(kv, int(0.9 * ridge * kv), ms, None)
    above = bench.attn_roofline(kv, int(1.1 * ridge * kv), ms, None)
    assert below["bound"] == "hbm" and below["unit"] == "GB/s" and below["peak"] == bench.HBM_PEAK_GBS
    assert above["bound"] == "mfma" and above["unit"] == "TFLOP/s" and above["peak"] == bench.BF16_MFMA_PEAK_TFLOPS
    # 1 GB in 1 ms is 1000 GB/s; both fractions are always reported
    for r in (below, above):
        assert abs(r["hbm_gbs"] - 1000.0) < 1e-6 and abs(r["hbm_frac"] - 1000.0 / 8000.0) < 1e-6
    assert abs(above["achieved"] - above["mfma_tflops"]) < 0.1
    assert abs(above["frac"] - above["mfma_frac"]) < 1e-4
    assert abs(below["frac"] - below["hbm_frac"]) < 1e-6


def test_fraction_of_read_ceiling_uses_the_hbm_rate():
    r = bench.attn_roofline(7 * 10 ** 9, 10 ** 9, 1.0, None)        # 7000 GB/s, HBM-bound
    bench.with_ceiling(r, 7000.0)
    assert abs(r["frac_of_read_ceiling"] - 1.0) < 1e-9
    m = bench.attn_roofline(10 ** 9, 10 ** 12, 1.0, None)           # matrix-bound line: still its HBM rate
    bench.with_ceiling(m, 4000.0)
    assert abs(m["frac_of_read_ceiling"] - 0.25) < 1e-9


def test_step_bytes_terms():
    w = get_workload("gqa_fp8_binned")

    class Case:  # the two attributes step_bytes reads from a case
        batch = 3

        @staticmethod
        def kv_bytes():
            return 12345

    b = bench.step_bytes(w, Case, 2)
    D, B, Hq, Dk, Dv = w.dcp_size, 3, w.num_q_heads, w.head_dim_k, w.head_dim_v
    assert b["kv"] == 12345
    assert b["q_reads"] == D * B * Hq * Dk * 2                       # every rank reads the bf16 queries
    assert b["partials_write_read"] == 2 * D * B * Hq * (Dv + 1) * 4  # fp32 O and LSE, written and read
    assert b["final_out"] == B * Hq * (Dv * 2 + 4)
    assert b["total"] == b["kv"] + b["q_reads"] + b["partials_write_read"] + b["final_out"]


def test_source_hashes_cover_each_family():
    hashes = {f: bench.source_hash(f) for f in bench.KERNEL_SOURCES}
    assert all(len(h) == 16 for h in hashes.values())
    # the GQA and MLA families share the split header but not their kernels
    assert hashes["gqa"] != hashes["mla"]
