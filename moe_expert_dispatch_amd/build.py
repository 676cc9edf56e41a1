"""Builds libmoe_hip.so (gfx950) in-tree from csrc/*.hip with hipcc.

    python -m moe_expert_dispatch_amd.build [--verbose]

Every call recompiles all sources (one hipcc process per file, in parallel)
and links the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as _fut
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmoe_hip.so")
# Stand-alone measurement program (not part of the library): the chip's
# sustained bf16 MFMA rate alone and with the GEMM's operand movement.
PROBE_SRC = os.path.join(HERE, "probe", "mfma_ceiling.hip")
PROBE_BIN = os.path.join(HERE, "probe", "mfma_ceiling")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # loop heads start on 64-byte instruction-fetch boundaries: the GEMM's
    # K-loop time otherwise depends on where the linker happens to place it
    "-falign-loops=64",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# The direct-to-LDS GEMM counts its own outstanding vector-memory operations
# (s_waitcnt vmcnt with fixed counts), so no compiler-generated memory access
# may appear in it: register spills to scratch would shift every count. The
# build asks for the resource-usage remarks and rejects such a kernel (file ->
# kernel-name fragment) if it uses scratch.
NO_SCRATCH = {"gemm_mfma.hip": "grouped_gemm_dma_kernel"}
_REMARK = "kernel-resource-usage"


_SCRATCH = re.compile(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)")


def _check_no_scratch(src, out):
    frag = NO_SCRATCH[os.path.basename(src)]
    name = None
    for line in out.splitlines():
        if _REMARK not in line:
            continue
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and name and frag in name and int(m.group(2)) != 0:
            raise RuntimeError(f"{os.path.basename(src)}: kernel {name} reports "
                               f"{m.group(1)} {m.group(2)}; its hand-counted memory waits "
                               "need a kernel without scratch accesses")


def _run(cmd, verbose, check_src=None):
    if check_src:
        cmd = [*cmd, f"-Rpass-analysis={_REMARK}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if check_src:
        _check_no_scratch(check_src, out)
        if not verbose:
            out = ""
    if verbose and out.strip():
        print(out, flush=True)


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the
# validation and planning code (each flag applies to the host compilation
# only; GPU code is not instrumented). Used by a CPU test, never shipped.
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined"]


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Builds out_dir/libmoe_hip.so with host-side ASan and UBSan."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with _fut.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1, 16)) as ex:
        futs = [ex.submit(_run, [cc, *COMPILE_FLAGS, *SANITIZE_FLAGS, "-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    lib = os.path.join(out_dir, "libmoe_hip.so")
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-shared-libsan",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-o", lib, *objs], verbose)
    return lib


def build(verbose: bool = False, jobs: int = 0) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources in {CSRC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    probe_tmp = PROBE_BIN + ".tmp"
    with _fut.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [cc, *COMPILE_FLAGS, "-c", s, "-o", o], verbose,
                          s if os.path.basename(s) in NO_SCRATCH else None)
                for s, o in zip(srcs, objs)]
        futs.append(ex.submit(_run, [cc, *COMPILE_FLAGS, PROBE_SRC, "-o", probe_tmp], verbose))
        for f in futs:
            f.result()
    os.replace(probe_tmp, PROBE_BIN)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
