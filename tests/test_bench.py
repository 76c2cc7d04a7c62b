"""bench.py's command-line contract: one JSON line with the fields a reader of the results relies on.

The GPU test runs a short benchmark of the tiny workload and of the mixed step (bench.main() in the
test's own process) and checks the line's fields and their consistency: roofline fraction =
achieved / peak, percentiles in order, the CPU baseline's sample stated. The CPU test checks that
more than one GPU is refused before anything touches a device.
"""
import json
import sys

import pytest

import bench

REQUIRED = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


def run_bench(monkeypatch, *args):
    """bench.main() in this process (no child process: the GPU may already be initialised)."""
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    bench.main()


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    with pytest.raises(SystemExit) as e:
        run_bench(monkeypatch, "--gpus", "2")
    assert e.value.code == 2
    out = capsys.readouterr()
    assert "one GPU" in out.err and out.out.strip() == ""


@pytest.mark.gpu
@pytest.mark.parametrize("workload,cpu", [("tiny_decode", True), ("chunked_prefill_mixed", True),
                                          ("prefix_sharing_2040", False),
                                          ("llama2_7b_decode", False)])
def test_bench_prints_one_complete_json_line(workload, cpu, monkeypatch, capsys):
    args = ["--workload", workload, "--steps", "3", "--warmup", "1", "--cpu-seconds", "2"]
    if not cpu:
        args.append("--no-cpu-baseline")
    print(f"[bench contract] {workload}", file=sys.stderr, flush=True)
    run_bench(monkeypatch, *args)
    stdout = capsys.readouterr().out
    lines = [l for l in stdout.splitlines() if l.strip()]
    assert len(lines) == 1, stdout
    d = json.loads(lines[0])
    for k in REQUIRED:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == workload
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    p10, p50, p90 = d["decode_ms_p10_p50_p90"]
    assert 0 < p10 <= p50 <= p90
    nd = d["config"]["num_seqs"]
    assert d["step_tokens"] == nd + d["config"]["prefill_rows"]
    # ms_per_step and decode_ms are printed rounded to 1e-5 ms: compare relatively
    rate = d["step_tokens"] / (d["ms_per_step"] * 1e-3)
    assert abs(d["step_tokens_per_s"] - rate) <= 1e-3 * rate
    assert abs(d["decode_us_per_call"] - 1e3 * d["decode_ms"]) < 0.02
    if cpu:
        c = d["cpu_baseline"]
        assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
        assert c["single_thread"]["value"] > 0
    else:
        assert "cpu_baseline" not in d
    st = d.get("stages", {})
    assert ("reshape_and_cache" in st) == (d["config"]["scatter_tokens"] > 0)
    assert ("copy_blocks" in st) == (d["config"]["copy_pairs"] > 0)
    for name, x in st.items():
        assert x["us_per_call"] > 0 and x["algorithmic_bytes"] > 0 and x["unit"] == "GB/s"
        assert abs(x["achieved"] - x["algorithmic_bytes"] / x["us_per_call"] / 1e3) \
            <= 1e-2 * x["achieved"] + 0.01
        assert abs(x["frac"] - x["achieved"] / 8000.0) < 1e-3
    if d["config"]["prefill_rows"]:
        assert d["step_tokens"] == 2048            # the mixed step's token budget
        assert d["prefill_ms"] > 0 and 0 < d["prefill_mfma_frac"] < 1
        rp = d["roofline_prefill"]
        assert rp["bound"] == "mfma" and rp["peak"] == 2500.0 and rp["frac"] == d["prefill_mfma_frac"]
        if cpu:
            cp = d["cpu_baseline_prefill"]
            assert cp["kind"] == "oracle" and cp["unit"] == "GFLOP/s" and cp["value"] > 0
    else:
        assert "roofline_prefill" not in d and "cpu_baseline_prefill" not in d


@pytest.mark.gpu
def test_bench_line_of_a_speculative_step(monkeypatch, capsys):
    """A step of drafted rows only (llama2_7b_spec4): its rows go through pa_decode_multi, whose
    HBM roofline and CPU baseline become the line's."""
    print("[bench contract] llama2_7b_spec4", file=sys.stderr, flush=True)
    run_bench(monkeypatch, "--workload", "llama2_7b_spec4", "--steps", "3", "--warmup", "1",
              "--cpu-seconds", "2")
    lines = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in REQUIRED:
        assert k in d, k
    assert d["config"]["num_seqs"] == 0 and d["config"]["prefill_rows"] == 256
    rf, rp = d["roofline"], d["roofline_prefill"]
    assert rf["kernel"].startswith("pa_decode_multi") and rf == rp
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert d["multi_token_rows_per_s"] > 0 and d["prefill_ms"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GB/s" and c["value"] > 0 and c["sample"]
