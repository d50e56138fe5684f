"""Host-side logic of bench.py, on the CPU: the algorithmic bytes it prices
the kernels with, its rocprofv3 counter summaries (on synthetic counter
files) and its refusal of more than one GPU."""
import csv
import os

import pytest

import bench
from fixed_cost_drafter_amd import workload as WLM


def test_algorithmic_bytes_are_the_shapes_closed_forms():
    """At the 128K workload every per-call figure is the sum of the arrays the
    step must touch, written out from the shapes."""
    wl = WLM.WORKLOADS["q3_8b_128k"]
    tau = 3.0
    a = bench.algorithmic(wl, tau, wl.L0)
    C, Hq, Hkv, d, W, S, B, V = wl.C, wl.Hq, wl.Hkv, wl.d, wl.W, wl.S, wl.B, wl.V
    units = C * Hkv
    # logits once, the drafts, and the target tokens + tau words
    assert a["verify"] == C * (B + 1) * V * 2 + C * B * 4 + C * (B + 2) * 4
    # fp32 (m, l, n) read and written, bf16 slots written, tau rows read and
    # written to the ring, the slot queries read once
    state = units * S * (2 * d + 2) * 4
    slots = units * S * d * 2 * 2
    rows = C * tau * Hkv * d * 2 * 2
    assert a["append"] == pytest.approx(2 * state + slots + 2 * rows + Hkv * S * d * 2)
    # every key and value of the three views, the queries and the output, the
    # window positions
    assert a["draft"] == units * (W + S + B) * d * 2 * 2 + 2 * C * B * Hq * d * 2 + C * W * 4
    assert a["draft"] == 80_805_888
    # one launch: the merged slots are not read back
    assert a["update_draft"] == pytest.approx(a["append"] + a["draft"] - slots)
    assert a["round"] == pytest.approx(a["verify"] + a["update_draft"])
    assert a["draft_flop"] == units * 4 * B * (Hq // Hkv) * (W + S + B) * d
    assert a["init"] == units * wl.L0 * d * 2 * 2
    assert a["init_flop"] == units * wl.L0 * 6 * S * d


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow(dict(Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value))


def test_traffic_summary_scales_by_the_calibration_copies(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled so the 512 MiB copy
    reads and writes 512 MiB; the 64 MiB copies give the second point; an
    entry point's bytes are the sum over its kernels."""
    neg = "void at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel_cuda(...)"
    # this part's FETCH_SIZE counts half of a copy's reads; WRITE_SIZE all
    fetch = [(neg, "FETCH_SIZE", 256 * 1024)] + [(neg, "FETCH_SIZE", 32 * 1024)] * 3
    write = [(neg, "WRITE_SIZE", 512 * 1024)] + [(neg, "WRITE_SIZE", 64 * 1024)] * 3
    for k, f_kib, w_kib in (("void ls::(anonymous namespace)::verify_partial<ls::BF16>(...)", 40000, 100),
                            ("void ls::(anonymous namespace)::update_draft<4>(...)", 48000, 27000)):
        fetch += [(k, "FETCH_SIZE", f_kib)] * 2
        write += [(k, "WRITE_SIZE", w_kib)] * 2
    _counter_csv(tmp_path / "f", fetch)
    _counter_csv(tmp_path / "w", write)
    t = bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd")
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_scale_64MiB"] == pytest.approx(2.0)
    assert t["write_scale_64MiB"] == pytest.approx(1.0)
    assert t["fetch_calibration_64MiB_dispatches"] == 3
    ud = t["entry_points"]["update_draft"]
    assert ud["fetch_bytes"] == round(48000 * 1024 * 2.0)
    assert ud["write_bytes"] == round(27000 * 1024)
    rd = t["entry_points"]["round"]  # verify_partial + update_draft
    assert rd["fetch_bytes"] == round((40000 + 48000) * 1024 * 2.0)
    assert rd["write_bytes"] == round((100 + 27000) * 1024)
    assert sorted(rd["kernels"]) == ["ls::update_draft<4>", "ls::verify_partial<ls::BF16>"]
    assert rd["source_hash"] == bench.source_hash(bench.KERNEL_SOURCES["round"])


def test_traffic_summary_needs_the_calibration_copy(tmp_path):
    _counter_csv(tmp_path / "f", [("void ls::x(...)", "FETCH_SIZE", 1)])
    _counter_csv(tmp_path / "w", [("void ls::x(...)", "WRITE_SIZE", 1)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd")


def test_counter_summary_means_per_dispatch(tmp_path):
    k = "void ls::(anonymous namespace)::update_draft<4>(...)"
    _counter_csv(tmp_path / "a", [(k, "MfmaUtil", 6.0), (k, "MfmaUtil", 8.0), (k, "GRBM_GUI_ACTIVE", 100.0),
                                  (k, "GRBM_GUI_ACTIVE", 300.0)])
    _counter_csv(tmp_path / "b", [(k, "SQ_WAVES", 2048.0), (k, "SQ_WAVES", 2048.0)])
    c = bench.summarize_counters([str(tmp_path / "a"), str(tmp_path / "b")], "cmd")
    ent = c["entry_points"]["update_draft"]
    assert ent["kernel"] == "ls::update_draft<4>"
    assert ent["MfmaUtil"] == pytest.approx(7.0)
    assert ent["GRBM_GUI_ACTIVE"] == pytest.approx(200.0)
    assert ent["SQ_WAVES"] == pytest.approx(2048.0)
    assert c["kernels"]["ls::update_draft<4>"]["dispatches"] == 2


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_hash_follows_code_not_comments():
    """A profile stays valid across comment and layout edits of its kernel's
    sources, and goes stale with any change of the code itself."""
    code = "__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n"
    commented = "/* a kernel */\n__global__ void k(int* p) {\n    p[0] = 1;  // the one store\n}\n"
    changed = "__global__ void k(int* p) {\n  p[0] = 2;  // store\n}\n"
    assert bench._code_only(code) == bench._code_only(commented)
    assert bench._code_only(code) != bench._code_only(changed)
    assert len(bench.source_hash(bench.KERNEL_SOURCES["round"])) == 16


def _synthetic_measurements():
    """A run_gpu-shaped result with round-number timings (seconds)."""
    main = dict(wall_s=20 * 41e-6, gpu_s=20 * 40e-6, issue_s=20 * 10e-6,
                passes_wall_s=[20 * 41e-6] * 5, passes_gpu_s=[20 * 40e-6] * 5)
    kern = dict(verify_s=17e-6, append_s=12e-6, draft_s=16e-6, update_draft_s=26e-6,
                draft_cold_s=28e-6, draft_warm_single_s=18.5e-6, update_draft_event_s=28.5e-6,
                verify_keys_s=14e-6, round_split_s=40e-6, verify_append_s=24e-6)
    return dict(main=main, kern=kern, init_s=2.5e-3, sweep={}, state_bytes_per_seq=5_779_464,
                stream_reference=dict(copy_64MiB_gb_per_s=6800.0, copy_512MiB_gb_per_s=6250.0),
                mfma_reference=dict(gemm="8192x8192x8192 bf16 torch.mm", tflop_per_s=1100.0,
                                    frac_of_peak=0.44))


def test_result_line_keeps_the_contract():
    """The JSON line's required fields and its arithmetic, from synthetic
    measurements: whole-job rounds/s, the roofline of the longest kernel
    (algorithmic bytes / its time against the 8 TB/s peak) and the oracle's
    CPU rate, all JSON-serialisable."""
    import argparse
    import json
    wl = WLM.WORKLOADS["q3_8b_128k"]
    args = argparse.Namespace(steps=20, warmup=5, passes=5, heat=400, next=False)
    cpu = dict(value=50.0, unit="rounds/s", cores=16, kind="oracle", sample="synthetic")
    line = bench.result_line(args, wl, _synthetic_measurements(), cpu)
    json.loads(json.dumps(line))
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 5
    assert line["unit"] == "rounds/s" and line["higher_is_better"] is True
    assert line["vs_baseline"] is None and line["data"] == "synthetic"
    assert line["config"]["workload"] == "q3_8b_128k"
    assert line["value"] == pytest.approx(1 / 41e-6, rel=1e-3)
    assert line["ms_per_step"] == pytest.approx(0.041, rel=1e-3)
    roof = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    alg = bench.algorithmic(wl, WLM.expected_tau(wl), wl.L0)
    assert roof["kernel"] == "update_draft" and roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["peak"] == 8000.0
    assert roof["achieved"] == pytest.approx(alg["update_draft"] / 26e-6 / 1e9, abs=0.1)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0, abs=1e-4)
    assert roof["frac_of_stream_reference"] == pytest.approx(roof["achieved"] / 6800.0, abs=1e-4)
    assert line["cpu_baseline"] == cpu
    init = line["kernels"]["init"]
    assert init["mfma_frac"] == pytest.approx(alg["init_flop"] / 2.5e-3 / 1e12 / 2500.0, abs=1e-4)
    ex = bench.executed_flop("init")  # from the committed counters, when they are current
    if ex is None:
        assert init["frac_of_mfma_reference"] is None and init["executed_tflop_per_s"] is None
    else:
        assert init["frac_of_mfma_reference"] == pytest.approx(ex / 2.5e-3 / 1e12 / 1100.0, abs=1e-4)
        # at a 128K prefix the far splits pool half the slots on all but the newest ~12K rows
        assert 0.5 * alg["init_flop"] < ex < 0.6 * alg["init_flop"]
