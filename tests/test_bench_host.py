"""Host-side logic of bench.py (no GPU): exact allowed-pair counts."""
import json
import os

import numpy as np
import pytest

import bench
import oracle
from synth import WORKLOADS


@pytest.mark.parametrize("Lq,Lkv,causal,window", [(7, 7, False, 0), (9, 9, True, 0), (12, 12, True, 4),
                                                  (10, 6, True, 3), (6, 10, False, 2), (5, 9, True, 0),
                                                  (30, 30, False, 7)])
def test_allowed_pairs_matches_mask(Lq, Lkv, causal, window):
    want = int(oracle.mask_matrix(np.arange(Lq), Lkv, causal, window).sum())
    assert bench.allowed_pairs(Lq, Lkv, causal, window) == want


def test_workload_pair_counts():
    # closed forms: causal L(L+1)/2; causal + window W(W+1)/2 + (L-W)W
    assert bench.allowed_pairs(2048, 2048, True, 0) == 2048 * 2049 // 2 == 2098176
    assert bench.allowed_pairs(8192, 8192, True, 1024) == 1024 * 1025 // 2 + (8192 - 1024) * 1024 == 7864832
    assert bench.allowed_pairs(32768, 32768, True, 0) == 536887296
    f = bench.workload_flops(WORKLOADS[2])
    assert abs(f["total"] - 4.813e11) / 4.813e11 < 1e-3


def test_gpus_other_than_one_exit(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().out


def test_traffic_is_reported_only_for_the_kernels_it_was_measured_on(monkeypatch):
    import bench

    rec_path = os.path.join(bench.PROFILES, "hbm_traffic_bf16_causal_gqa4_L2048_D128.json")
    if not os.path.exists(rec_path):
        pytest.skip("no committed counter summary")
    with open(rec_path) as fh:
        rec = json.load(fh)
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: rec["source_sha256"])
    t = bench.measured_traffic("bf16_causal_gqa4_L2048_D128", "fa_bwd_dkv")
    assert t == float(rec["kernels"]["fa_bwd_dkv"]["bytes_per_launch"]) and t > 0
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic("bf16_causal_gqa4_L2048_D128", "fa_bwd_dkv") is None
    assert bench.measured_traffic("no_such_workload", "fa_bwd_dkv") is None


def test_roofline_bound_follows_the_machine_balance():
    # the 2048-token forward: ~815 FLOP per algorithmic byte, above the bf16
    # balance of 2500 TFLOP/s / 8 TB/s = 312.5 -> matrix-core bound
    w = WORKLOADS[2]
    f, by = bench.workload_flops(w), bench.workload_bytes(w)
    r = bench.roofline("fa_fwd", f["fwd"], by["fwd"], 0.2, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - f["fwd"] / 0.2e-3 / 1e12) < 1e-9 and abs(r["frac"] - r["achieved"] / 2500) < 1e-12
    # 8 query rows against 4096 keys: ~32 FLOP per byte -> HBM bound, GB/s
    w = next(x for x in WORKLOADS if x.name == "bf16_gqa4_q8_kv4096_D128")
    f, by = bench.workload_flops(w), bench.workload_bytes(w)
    assert f["fwd"] / by["fwd"] < 100
    r = bench.roofline("fa_fwd", f["fwd"], by["fwd"], 0.01, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - by["fwd"] / 0.01e-3 / 1e9) < 1e-6


def test_cpu_baseline_on_a_small_workload():
    # the oracle timed on whole slices of the 256-token workload, threads reported
    r = bench.cpu_baseline(WORKLOADS[1], budget_s=1.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert 1 <= r["cores"] <= min(16, len(os.sched_getaffinity(0)))
    assert "slices" in r["sample"]


def test_cpu_baseline_cuts_a_large_slice_to_a_prefix(monkeypatch):
    # the 8192-token windowed workload: a slice is cut to its first rows and keys,
    # at least twice the window
    import oracle as orc

    seen = {}

    def fake_backward(q, k, v, do, scale, causal, window):
        seen["shape"] = (q.shape, k.shape, causal, window)

    monkeypatch.setattr(orc, "backward", fake_backward)
    r = bench.cpu_baseline(WORKLOADS[3], budget_s=0.5)
    (qs, ks, causal, window) = seen["shape"]
    assert qs[2] == ks[2] == 2048 and causal and window == 1024
    assert r["sample"].startswith("first 2048 query rows and 2048 keys")
