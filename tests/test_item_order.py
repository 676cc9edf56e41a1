"""The grouped GEMM's work-item order (csrc/item_order.h) on the host.

Every launch hands out items 0 .. RT*CT-1 to its blocks; each must name a
distinct (row tile, column tile) pair inside the RT x CT grid, and together
they must cover it, for every group shape the kernels use (GN = min(CT, 4),
GM = 32 / GN) and the others the mapping allows. Built with the host C++
compiler, so no GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "moe_expert_dispatch_amd", "csrc", "item_order.h")

DRIVER = r"""
#define __host__
#define __device__
#define __forceinline__ inline
#include <cstdio>
#include <vector>
#include "item_order.h"
int main() {
  long bad = 0, cases = 0;
  for (int RT = 1; RT <= 260; ++RT)
    for (int CT = 1; CT <= 36; ++CT)
      for (int GN0 : {1, 2, 3, 4, 8}) {
        const int GN = CT < GN0 ? CT : GN0;
        const int GM = 32 / GN;
        std::vector<int> seen(RT * CT, 0);
        for (int w = 0; w < RT * CT; ++w) {
          int rt = -1, ct = -1;
          moe::item_tile(w, RT, CT, GM, GN, &rt, &ct);
          if (rt < 0 || rt >= RT || ct < 0 || ct >= CT) { ++bad; continue; }
          ++seen[rt * CT + ct];
        }
        for (int v : seen) bad += v != 1;
        ++cases;
      }
  std::printf("%ld %ld\n", cases, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_item_order_is_a_bijection(tmp_path):
    src = tmp_path / "item_order_check.cpp"
    exe = tmp_path / "item_order_check"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HEADER), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    cases, bad = map(int, out.stdout.split())
    assert cases == 260 * 36 * 5
    assert bad == 0 and out.returncode == 0
