"""bench.py's command-line contract on the host: more than one GPU is refused
with a message and exit status 2 before anything touches a device, and the
traffic record is looked up by the GEMM source digest."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_follows_the_gemm_source(tmp_path, monkeypatch):
    import bench
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // a comment\n")
    d0 = bench.kernel_source_digest([str(src)])
    src.write_text("int f() {\n  return 1;  // another comment\n}\n")
    assert bench.kernel_source_digest([str(src)]) == d0  # comments and spacing only
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_digest([str(src)]) != d0  # a code change
    # a record taken on other source is not used
    monkeypatch.setattr(bench, "GEMM_SRC", [str(src)])
    assert bench.gemm_traffic("redundant_slots_zipf") is None


def test_mfma_ceiling_reads_program_output(tmp_path, monkeypatch):
    """bench.py takes the ceiling program's two JSON lines as rates, and
    reports a reason instead when the program is missing or fails."""
    import bench
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.mfma_ceiling() == {"error": "program not built"}
    prog = tmp_path / "moe_expert_dispatch_amd" / "probe" / "mfma_ceiling"
    prog.parent.mkdir(parents=True)
    prog.write_text("#!/bin/sh\n"
                    "echo '{\"mode\": \"mfma_only\", \"tflops\": 1800.5}'\n"
                    "echo '{\"mode\": \"operand_movement\", \"tflops\": 1400.0}'\n")
    prog.chmod(0o755)
    got = bench.mfma_ceiling()
    assert got["mfma_only_tflops"] == 1800.5 and got["operand_movement_tflops"] == 1400.0
    prog.write_text("#!/bin/sh\necho no device >&2\nexit 1\n")
    assert bench.mfma_ceiling()["error"].startswith("exit status 1")


def test_ceiling_fraction_uses_the_gemm_precision():
    import bench
    c = {"operand_movement_tflops": 1400.0, "fp8_operand_movement_tflops": 2800.0}
    assert bench.ceiling_with_frac(c, 700.0, False)["gate_up_frac_of_operand_movement"] == 0.5
    assert bench.ceiling_with_frac(c, 700.0, True)["gate_up_frac_of_operand_movement"] == 0.25
    assert bench.ceiling_with_frac({"error": "x"}, 700.0, True) == {"error": "x"}
    assert bench.ceiling_with_frac(None, 700.0, False) is None
