"""Host logic of bench.py (no GPU): the one-GPU guard, the work charged to each launch,
the HBM-counter bookkeeping (copy calibration, the source-hash gate) and the oracle
baselines on small samples."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic as S  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_work_per_launch():
    """The figures the roofline is computed from, at B4 H16 N8192 d128: forward
    4*B*H*N^2*d = 2199.0 GFLOP over Q, K, V, O (bf16) and the fp32 LSE; the dK/dV kernel
    four of the five backward products, dQ one (and three executed)."""
    kt = {k["name"]: k for k in bench.kernel_table(S.HEADLINE)}
    assert kt["fwd_mfma_kernel"]["work"] == 4 * 64 * 8192 ** 2 * 128 == 2199023255552
    assert kt["fwd_mfma_kernel"]["bytes"] == 4 * 64 * 8192 * 128 * 2 + 64 * 8192 * 4
    assert kt["bwd_dkdv_kernel"]["work"] == pytest.approx(8 * 64 * 8192 ** 2 * 128)
    assert kt["bwd_dq_kernel"]["work"] == pytest.approx(2 * 64 * 8192 ** 2 * 128)
    assert kt["bwd_dq_kernel"]["executed_work"] == pytest.approx(6 * 64 * 8192 ** 2 * 128)
    # Preprocess: O and dO read (d bf16 each), LSE read, D and LSE*log2(e) written.
    assert kt["bwd_preprocess_kernel"]["work"] == 64 * 8192 * (2 * 128 * 2 + 12)


def test_causal_work_is_halved():
    w = S.WORKLOADS["fp16_causal"]
    assert w.causal
    assert w.fwd_flop() == 4 * w.B * w.H * w.N ** 2 * w.d / 2
    assert w.bwd_flop() == pytest.approx(2.5 * w.fwd_flop())


def test_row_bytes():
    w = S.ROWS["xent_bf16_T8192_V128256"]
    fb, bb = bench.row_bytes(w)
    el = 8192 * 128256 * 2
    assert fb == el + 8192 * 12  # logits; int32 target, fp32 loss and lse per row
    assert bb == 2 * el + 8192 * 12  # logits read, dlogits written; target, lse, dloss
    w = S.ROWS["softmax_bf16_R65536_C8192"]
    assert bench.row_bytes(w) == (2 * 65536 * 8192 * 2, 3 * 65536 * 8192 * 2)


def test_stats():
    st = bench.stats([5.0, 1.0, 3.0, 2.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert st["mean"] == 5.5 and st["min"] == 1.0 and st["median"] == 5.5 and st["p90"] == 9.0
    assert bench.stats([3.0, 1.0, 2.0])["median"] == 2.0


def _counter_folder(path, counter, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, vs in values.items():
            for v in vs:
                wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
    return str(path)


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    """Counters per dispatch are averaged over dispatches and scaled so that the copy of
    COPY_BYTES reads and writes exactly its size; the record carries the source hash and
    traffic_of serves it only while the kernel's sources are unchanged."""
    out = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy_kib = bench.COPY_BYTES / 1024
    names = {"fwd": "_ZN6osattn15fwd_mfma_kernelIDF16b", "pre": "bwd_preprocess_kernel<bf16>",
             "dkdv": "bwd_dkdv_kernel<bf16>", "dq": "bwd_dq_kernel<bf16>"}
    fetch = {names["fwd"]: [100.0, 300.0], names["pre"]: [10.0], names["dkdv"]: [20.0],
             names["dq"]: [30.0], "__amd_rocclr_copyBuffer": [copy_kib / 2]}
    write = {names["fwd"]: [50.0], names["pre"]: [1.0], names["dkdv"]: [2.0], names["dq"]: [3.0],
             "__amd_rocclr_copyBuffer": [copy_kib]}
    f = _counter_folder(tmp_path / "f", "FETCH_SIZE", fetch)
    w = _counter_folder(tmp_path / "w", "WRITE_SIZE", write)
    bench.write_traffic([f, w, f, w], None)
    rec = json.loads(out.read_text())
    assert rec["copy_calibration"]["fetch_scale"] == 2.0
    assert rec["copy_calibration"]["write_scale"] == 1.0
    ent = rec["kernels"]["fwd_mfma_kernel"]
    hw = ent["workloads"][S.HEADLINE.name]
    assert hw["hbm_bytes_per_launch"] == int(200.0 * 1024 * 2 + 50.0 * 1024)
    kt = bench.kernel_table(S.HEADLINE)[0]
    assert bench.traffic_of(rec, kt, S.HEADLINE.name) == hw["hbm_bytes_per_launch"]
    stale = dict(rec, kernels={"fwd_mfma_kernel": dict(ent, source_sha="0" * 16)})
    assert bench.traffic_of(stale, kt, S.HEADLINE.name) is None
    assert bench.traffic_of(rec, kt, "some_other_workload") is None


def test_attention_cpu_baseline_on_the_single_head_workload():
    """The whole fp32 single-head workload is the sample (one head); fed the oracle's
    own output as the 'GPU' result, the recorded errors vanish."""
    import oracle.attention as A
    w = S.WORKLOADS["fp32_single_head"]
    inp = S.make_inputs(w, with_grad=True)
    ref = A.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.causal)
    o = torch.from_numpy(np.ascontiguousarray(ref["o"]))
    dq = torch.from_numpy(np.ascontiguousarray(ref["dq"]))
    cb = bench.cpu_baseline(w, inp, (o, dq))
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] >= 1
    assert "1 of 1 heads" in cb["sample"]
    # (the 'GPU' side is taken through float32, as the device output would be)
    assert cb["gpu_vs_oracle_on_sample"]["o_max_abs"] < 1e-6
    assert cb["gpu_vs_oracle_on_sample"]["dq_rel"] < 1e-6


def test_cpu_baseline_sample_scales_with_length():
    """16 heads at N = 8192, a quarter of that at N = 16384, whole KV groups."""
    cases = {"sweep_bf16_B4_H16_N8192_d128": [(0, g) for g in range(16)],
             "bf16_gqa_causal": [(0, 0)],                 # 4 query heads share kv head 0
             "fp32_single_head": [(0, 0)],
             "sweep_bf16_B4_H16_N2048_d128": [(0, g) for g in range(16)]}  # capped at 16
    for name, groups in cases.items():
        assert bench.baseline_groups(S.WORKLOADS[name]) == groups, name


def test_row_cpu_baseline_covers_rows_in_order():
    w = S.RowWorkload("tiny_log_softmax", "log_softmax", "fp32", 64, 1000, 777)
    inp = S.row_inputs(w)
    cb = bench.row_cpu_baseline(w, inp, budget_s=5.0)
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert "rows 0-63 of 64" in cb["sample"]


def test_decode_cpu_baseline_covers_batch_in_order():
    """Fed the oracle's own output as the 'GPU' result, the recorded error vanishes; the
    whole batch is the sample when the budget allows."""
    import oracle.attention as A
    w = S.custom("bf16", 2, 4, 2, 3, 64, True, seed_base=123, Nk=200)
    inp = S.make_inputs(w, with_grad=False)
    ref_o, _ = A.attention_forward(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    cb = bench.decode_cpu_baseline(w, inp, torch.from_numpy(ref_o), 1000, budget_s=5.0)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0
    assert "batch entries 0-1 of 2" in cb["sample"]
    assert cb["gpu_vs_oracle_o_max_abs"] < 1e-6


def test_masked_cpu_baseline_walks_groups():
    import oracle.attention as A
    w = S.custom("bf16", 2, 4, 2, 40, 64, False, seed_base=321, Nk=50)
    inp = S.make_inputs(w, with_grad=True)
    lo, hi = S.mask_intervals("sliding", w.B, w.N, w.nk, left=7, right=3, causal=False)
    ref = A.attention_backward_intervals(inp["q"], inp["k"], inp["v"], inp["do"], w.scale,
                                         lo.numpy(), hi.numpy())
    o, dq = torch.from_numpy(ref["o"]), torch.from_numpy(ref["dq"])
    cb = bench.masked_cpu_baseline(w, inp, lo, hi, o, dq, budget_s=5.0)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert "4 of 8 heads" in cb["sample"] and "kv groups 0-1" in cb["sample"]
    assert cb["gpu_vs_oracle_on_sample"]["o_max_abs"] < 1e-6
    assert cb["gpu_vs_oracle_on_sample"]["dq_rel"] < 1e-6


def test_sclk_reading(tmp_path):
    """The current core clock is the starred level of pp_dpm_sclk; the peak scales
    linearly from the 2.4 GHz spec clock."""
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\n1: 2105Mhz *\n2: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) == 2105.0
    p.write_text("0: 500Mhz\n1: 157Mhz\n2: 2400Mhz *\n")
    assert bench.read_sclk_mhz(str(p)) == 2400.0
    p.write_text("garbage\n")
    assert bench.read_sclk_mhz(str(p)) is None
    assert bench.read_sclk_mhz(str(tmp_path / "missing")) is None
    assert bench.peak_at_clock(2516.6, 2.1) == pytest.approx(2516.6 * 2.1 / 2.4)
    assert bench.peak_at_clock(2516.6, None) is None


def test_clock_sampler_without_sysfs(monkeypatch):
    monkeypatch.setattr(bench, "sclk_path", lambda: None)
    c = bench.ClockSampler()
    c.start()
    c.stop()
    rec = c.record()
    assert rec["source"] == "unavailable" and rec["during_mhz"] is None
    assert not c.median_ghz()


def test_clock_sampler_uses_settled_samples(monkeypatch):
    """The clock is the median of the samples inside the timed region that were taken
    at least settle_s after the load began; with none, no clock is claimed."""
    monkeypatch.setattr(bench, "sclk_path", lambda: None)
    c = bench.ClockSampler(settle_s=0.3)
    c.samples = [(0.0, 900.0), (0.1, 1200.0), (0.2, 1500.0), (0.35, 2100.0), (0.4, 2200.0),
                 (0.45, 2000.0)]
    c.t_timed = 0.15
    assert c.timed_samples() == [1500.0, 2100.0, 2200.0, 2000.0]
    assert c.settled_samples() == [2100.0, 2200.0, 2000.0]
    assert c.median_ghz() == pytest.approx(2.1)
    rec = c.record()
    assert rec["settled_mhz"]["n"] == 3 and rec["during_mhz"]["n"] == 4
    c.t_timed = 0.5  # timed region after every sample
    assert c.median_ghz() is None and c.record()["settled_mhz"] is None
    c.t_timed, c.samples = 0.0, [(0.0, 900.0), (0.29, 1200.0)]  # a run shorter than settle_s
    assert c.median_ghz() is None
