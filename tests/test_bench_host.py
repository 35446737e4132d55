"""Host logic of bench.py that needs no GPU: the digest that ties the committed
HBM-traffic counters to the FFN kernel code they were taken with."""
import json
import os
import shutil

import bench


def _copy_sources(tmp_path):
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), dst)


def _digest_at(monkeypatch, root):
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_source_digest()


def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    base = _digest_at(monkeypatch, tmp_path)
    f = tmp_path / bench.KERNEL_SOURCES[0]
    text = f.read_text()
    f.write_text("// a new line comment\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 3) + "\n   \n")
    assert _digest_at(monkeypatch, tmp_path) == base


def test_digest_changes_with_the_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    base = _digest_at(monkeypatch, tmp_path)
    f = tmp_path / bench.KERNEL_SOURCES[1]
    f.write_text(f.read_text() + "\nstatic const int unused_constant = 1;\n")
    assert _digest_at(monkeypatch, tmp_path) != base


def test_traffic_is_reported_only_for_the_code_it_was_taken_with(tmp_path, monkeypatch):
    traffic = {"kernel_source_sha256": bench.kernel_source_digest(), "fetch_factor": 2.0, "write_factor": 1.0,
               "kernels": {"decode/ffn_up": {"fetch_kib": 100.0, "write_kib": 10.0}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(traffic))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("decode", "ffn_up") == int((100.0 * 2.0 + 10.0 * 1.0) * 1024)
    assert bench.measured_traffic("decode", "ffn_down") is None
    traffic["kernel_source_sha256"] = "0" * 64
    path.write_text(json.dumps(traffic))
    assert bench.measured_traffic("decode", "ffn_up") is None


def test_algorithmic_bytes_count_weights_and_x_only():
    import synth
    w = bench.algorithmic_work(synth.FULL, 64, 212)
    per_up = 2 * 2048 * 7168 + 2 * 16 * 56 * 4          # w1 + w3 and their block scales
    per_dn = 2048 * 7168 + 56 * 16 * 4
    assert w["ffn_up"]["bytes"] == 213 * per_up + 64 * (7168 + 56 * 4)
    assert w["ffn_down"]["bytes"] == 213 * per_dn
    assert w["h_bytes"] == 64 * 9 * (2048 + 16 * 4) and w["o_bytes"] == 64 * 9 * 7168 * 2
    assert w["ffn_up"]["flops"] == 2 * 64 * 9 * 7168 * 4096 and w["ffn_down"]["flops"] == 2 * 64 * 9 * 2048 * 7168
    assert w["layer_flops"] == 64 * 9 * 6 * 7168 * 2048


def test_roofline_position_names_the_binding_peak():
    hbm = bench.roofline_position(8e9, 1e12, 1.0)        # 8 GB/s -> 1e-3 of HBM; 1 TFLOP/s -> 4e-4 of bf16
    assert hbm["bound"] == "hbm" and hbm["frac"] == 0.001
    mf = bench.roofline_position(1e9, 1.25e15, 1.0)
    assert mf["bound"] == "mfma" and mf["bf16_mfma_frac"] == 0.5 and mf["fp8_mfma_frac"] == 0.25


def test_cpu_baseline_one_call_and_parity_on_host_tensors():
    # the baseline leg on host tensors of the tiny workload: one oracle call over the
    # sample; handed the oracle's own rounded output, it reports identical routing and
    # at most the final bf16 rounding (max |d| / rms below 2^-8 of the largest element)
    import numpy as np
    import torch

    import oracle
    import synth
    data = synth.make_workload("tiny", device="cpu")
    p, x, dims = data["blocks"][0], data["x"], data["dims"]
    ref = oracle.moe_forward(x.double().numpy(), {k: v.numpy() for k, v in p.items()}, dims)
    delta = torch.from_numpy(ref["delta"]).to(torch.bfloat16)
    tok = np.arange(0, 64, 3)
    base, parity = bench.cpu_baseline(x, p, dims, 2, tok, gpu_delta=delta, gpu_idx=ref["idx"])
    assert base["kind"] == "oracle" and base["cores"] == 2 and base["value"] > 0
    assert f"{tok.size} of 64 tokens in one oracle call" in base["sample"]
    assert parity["tokens"] == tok.size and parity["routing_identical"] == tok.size
    assert parity["routed_differently_not_near_tie"] == 0
    assert parity["max_abs_over_rms"] < 1e-2 and parity["mean_rel"] < 2e-3
