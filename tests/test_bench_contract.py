"""The JSON line bench.py prints: its keys, units and internal consistency
(tokens/s against ms per step, the roofline fraction against its parts), on
a short run of the 480p layer.  The argument check for more than one GPU runs
on the CPU."""
import json

import pytest

import bench
from tests.gpu_util import have_gpu


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.gpu
@pytest.mark.skipif(not have_gpu(), reason="needs a GPU")
def test_bench_line_480p(capsys):
    rc = bench.main(["--steps", "4", "--warmup", "2", "--workload", "480p_81f", "--no-cpu-baseline",
                     "--no-block-step", "--no-gated"])
    assert rc == 0
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 4 and r["warmup"] == 2
    assert r["unit"] == "tokens/s" and r["higher_is_better"] is True and r["dtype"] == "bf16"
    assert r["vs_baseline"] is None and r["data"] == "synthetic"
    cfg = r["config"]
    assert cfg["workload"] == "480p_81f" and cfg["N"] == 21 * 30 * 52 and cfg["H"] == 24
    assert r["value"] == pytest.approx(cfg["B"] * cfg["N"] / (r["ms_per_step"] * 1e-3), rel=1e-9)
    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert 0.0 < roof["frac"] < 1.0
    assert roof["kernel"] in ("apply_mfma_kernel", "state_mfma_kernel")
    ref = r["same_bytes_reference"]
    assert ref["bytes_per_call"] == roof["algorithmic_bytes_per_launch"] or roof["kernel"] != "apply_mfma_kernel"
    assert 0.0 < ref["frac"] < 1.0
    # the per-stage durations of the dominant kernel fit inside a step
    assert all(v is None or 0.0 < v < r["ms_per_step"] for v in r["stages_ms"].values())
    for leg in ("backward", "token_causal"):
        assert r[leg]["ms_per_call"] > 0 and 0 < r[leg]["roofline"]["frac"] < 1
