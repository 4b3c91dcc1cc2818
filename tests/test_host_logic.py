"""Host-side logic that needs no GPU: the bench contract and the parity tolerance helper."""
import math

import numpy as np
import pytest

import bench
from exact_tiled_attention_07_amd.inputs import WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f32
from parity import O_TOL, bf16_ulp, compare, passed


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
    assert bench.main(["--gpus", "8", "--steps", "1"]) == 2


def test_bench_traffic_record_matches_sources():
    # the committed counter summary is used only while the kernel sources are unchanged
    t = bench.recorded_traffic()
    text = open(bench.TRAFFIC_FILE).read() if __import__("os").path.exists(bench.TRAFFIC_FILE) else ""
    if bench.kernel_source_hash() in text:
        assert t is not None and t > 0
    else:
        assert t is None


def test_bench_backward_traffic_record_matches_sources():
    t = bench.recorded_traffic(bench.BWD_TRAFFIC_FILE, bench.BWD_SOURCES)
    os_ = __import__("os")
    text = open(bench.BWD_TRAFFIC_FILE).read() if os_.path.exists(bench.BWD_TRAFFIC_FILE) else ""
    if bench.kernel_source_hash(bench.BWD_SOURCES) in text:
        assert t is not None and t > 0
    else:
        assert t is None


@pytest.mark.parametrize("path,sources,key", [
    (bench.FP8_TRAFFIC_FILE, bench.FP8_SOURCES, "hbm_bytes_per_launch"),
    (bench.SPLITKV_TRAFFIC_FILE, bench.SPLITKV_SOURCES, "hbm_bytes_per_call[B4 H12 T1 Tk16384 d64 causal]"),
    (bench.SPLITKV_TRAFFIC_FILE, bench.SPLITKV_SOURCES, "hbm_bytes_per_call[B4 H12 T16 Tk16384 d64 causal]"),
    (bench.SPLITKV_TRAFFIC_FILE, bench.SPLITKV_SOURCES, "hbm_bytes_per_merge[c5a_causal_B4_H12_T16384_d64 x4]"),
])
def test_bench_other_traffic_records_match_sources(path, sources, key):
    os_ = __import__("os")
    text = open(path).read() if os_.path.exists(path) else ""
    t = bench.recorded_traffic(path, sources, key)
    if bench.kernel_source_hash(sources) in text and key in text:
        assert t is not None and t > 0
    else:
        assert t is None
    assert bench.recorded_traffic(path, sources, key + "x") is None  # an unknown key reads nothing


def test_bench_clock_record_matches_sources():
    c = bench.recorded_clock_mhz()
    text = open(bench.COUNTERS_FILE).read() if __import__("os").path.exists(bench.COUNTERS_FILE) else ""
    if bench.kernel_source_hash() in text:
        assert c is not None and 1000 < c < 2500
    else:
        assert c is None
    assert bench.MFMA_FLOP_PER_CLK * 2.4e9 / 1e12 == pytest.approx(bench.PEAK_BF16_TFLOPS, rel=1e-4)


def test_bench_cpu_baseline_small():
    r, (o_ref, lse_ref), n_heads = bench.cpu_baseline(WORKLOADS["c1"], budget_s=1.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert r["value"] > 0 and "heads of c1" in r["sample"]
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert n_heads == 2 and o_ref.shape == (1, 2, 256, 64) and lse_ref.shape == (1, 2, 256)


def test_bench_compulsory_bytes():
    # q, k, v read and o written once (bf16), lse written once (fp32): 101.4 MB at B4 H12 T4096 d64
    assert bench.compulsory_bytes(WORKLOADS["c4"]) == 48 * (4 * 4096 * 64 * 2 + 4 * 4096) == 101449728
    assert bench.compulsory_bytes(WORKLOADS["c5b"]) == 64 * (4 * 8192 * 128 * 2 + 4 * 8192)


def test_bench_parity_check_uses_the_oracle_output_and_catches_errors():
    import torch

    wl = WORKLOADS["c1"]
    _, ref, n_heads = bench.cpu_baseline(wl, budget_s=1.0)
    o = torch.from_numpy(ref[0].reshape(wl.B, wl.H, wl.T, wl.d)).to(torch.bfloat16)
    lse = torch.from_numpy(ref[1].reshape(wl.B, wl.H, wl.T)).float()
    p = bench.parity_check(wl, o, lse, ref, n_heads)
    assert p["pass"] and p["n_fail"] == 0 and p["rows"] == wl.B * wl.H * wl.T
    assert p["max_err_o"] <= 2.0 ** -7  # only the bf16 rounding of the oracle's own output (|O| < 4)
    # that one rounding: relative RMS about 2^-7 / sqrt(24)
    assert 0.5 * 2.0 ** -7 / 24 ** 0.5 < p["rms_rel_err_o"] < 1.5 * 2.0 ** -7 / 24 ** 0.5
    o[0, 1, 17, 5] += 0.05  # one element off by more than the tolerance
    lse[0, 0, 3] += 2e-3
    p = bench.parity_check(wl, o, lse, ref, n_heads)
    assert not p["pass"] and p["n_fail"] == 2


def test_bench_warm_up_runs_at_least_the_given_steps_and_time():
    calls = []
    bench.warm_up(lambda: calls.append(1), 7, lambda: None, min_s=0.05)
    assert len(calls) >= 7


def test_bench_cpu_baseline_per_config_lists_every_workload():
    assert bench.PER_CONFIG == ("c1", "c2", "c3", "c4", "c5a", "c5b")
    r = bench.cpu_baseline_per_config(names=("c1", "c5b"), budget_heads_s=0.0)
    assert set(r) == {"c1", "c1_1thread", "c5b"}
    assert "1 of 64 heads" in r["c5b"]["sample"]
    assert r["c1_1thread"]["cores"] == 1
    for v in r.values():
        assert v["kind"] == "oracle" and v["value"] > 0


def test_bf16_ulp_is_the_spacing_of_bf16():
    x = np.array([1.0, 1.5, 2.0, 3.99, 4.0, 7.5, 8.0, 0.75, -5.0])
    ulp = bf16_ulp(x)
    # the next bf16 value above |x| (for x on the bf16 grid) is |x| + ulp
    for xi, ui in zip(np.abs(x), ulp):
        b = bf16_bits_from_f32(np.float32(xi))
        nxt = bf16_bits_to_f32(np.uint16(int(np.asarray(b).reshape(-1)[0]) + 1))
        if bf16_bits_to_f32(b) == np.float32(xi):
            assert nxt - xi == pytest.approx(ui)
    assert ulp[0] == 2.0 ** -7 and ulp[4] == 2.0 ** -5 and ulp[6] == 2.0 ** -4


def test_tolerance_reading():
    ref = np.array([0.5, 3.0, 5.0, 5.0, 1.0])
    gpu = np.array([0.5 + 0.014, 3.0 + 0.0155, 5.0 + 0.031, 5.0 + 0.032, 1.0 - 0.016])
    s = compare(gpu, np.zeros(1), ref, np.zeros(1))
    # 0.014 literal; 0.0155 <= ulp(3)=2^-6; 0.031 <= ulp(5)=2^-5; 0.032 > 2^-5 fails; 0.016 at |1| fails
    assert s["n_ulp_clause"] == 2 and s["n_fail_o"] == 2
    assert math.isclose(O_TOL, 1.5e-2)
    # LSE: the literal 1e-3, in both directions; a non-finite output fails and is counted
    lse_ref = np.array([2.0, -3.0, 10.0])
    s = compare(np.ones(3), lse_ref + np.array([9.9e-4, -9.9e-4, 0.0]), np.ones(3), lse_ref)
    assert s["n_fail_lse"] == 0 and passed(s)
    s = compare(np.ones(3), lse_ref + np.array([1.01e-3, 0.0, -1.01e-3]), np.ones(3), lse_ref)
    assert s["n_fail_lse"] == 2 and not passed(s)
    s = compare(np.array([1.0, np.nan, np.inf]), lse_ref, np.ones(3), lse_ref)
    assert s["n_nonfinite"] == 2 and s["n_fail_o"] == 2 and not passed(s)


def test_page_claims_are_context_only():
    assert bench.PAGE_CLAIMS and all({"claim", "hardware", "source"} <= set(c) for c in bench.PAGE_CLAIMS)
    assert not any("MI355X" == c["hardware"] for c in bench.PAGE_CLAIMS)


def test_rms_check_matches_two_bf16_roundings():
    # the relative RMS allowance of the forward tests is twice the expected error of the kernel's two
    # bf16 roundings (P before P.V, O at the end) for i.i.d. zero-mean V: 2^-7 / sqrt(12). Simulate
    # exactly those roundings in float64 on causal rows of random scores and check the expectation
    from parity import RMS_O_REL

    rng = np.random.default_rng(12)
    T, d = 512, 64
    s = rng.standard_normal((T, T)) * 2.0
    s[np.triu_indices(T, 1)] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    v = bf16_bits_to_f32(bf16_bits_from_f32(rng.standard_normal((T, d)).astype(np.float32))).astype(np.float64)
    o = (p @ v) / l
    p16 = bf16_bits_to_f32(bf16_bits_from_f32(p.astype(np.float32))).astype(np.float64)
    o16 = bf16_bits_to_f32(bf16_bits_from_f32(((p16 @ v) / l).astype(np.float32))).astype(np.float64)
    rel = np.sqrt(np.mean((o16 - o) ** 2) / np.mean(o ** 2))
    o_only = np.sqrt(np.mean((bf16_bits_to_f32(bf16_bits_from_f32(o.astype(np.float32))) - o) ** 2)
                     / np.mean(o ** 2))
    assert o_only == pytest.approx(2.0 ** -7 / 24 ** 0.5, rel=0.05)  # the rounding of O alone
    assert o_only < rel <= 1.02 * 2.0 ** -7 / 12 ** 0.5                 # P's adds at most as much
    assert rel <= RMS_O_REL / 1.9
