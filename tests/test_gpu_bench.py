"""bench.py's output contract on the GPU: one JSON line with the metric, the
roofline object of the dominant kernel and, on bf16 workloads, the sustained
MFMA rates and the dense library reference (a short run on the 60-expert
layer; the CPU baseline is skipped to keep it short)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_common import announce, device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    device()
    announce("bench.py --workload qwen2_moe_bf16 --steps 2 --warmup 1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "qwen2_moe_bf16", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "qwen2_moe_bf16"
    roof = d["roofline"]
    assert set(("bound", "achieved", "peak", "unit", "frac", "traffic")) <= set(roof)
    assert roof["bound"] == "mfma" and roof["peak"] == 2500.0 and roof["unit"] == "TFLOP/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    ceil = d["mfma_ceiling"]
    assert "error" not in ceil, ceil
    for mode in ("mfma_zero", "mfma_only", "operand_movement"):
        assert 0 < ceil[mode + "_tflops"] <= 2600, ceil
    for mode in ("fp8_mfma_only", "fp8_operand_movement"):
        assert 0 < ceil[mode + "_tflops"] <= 5200, ceil
    dense = d["dense_reference"]
    assert dense["shape_mkn"][1:] == [2048, 2 * 1408] and dense["tflops"] > 0
