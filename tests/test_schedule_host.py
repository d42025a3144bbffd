"""The persistent grids' tile schedule (StaticSchedule in csrc/common.h), run on the host.

The causal forward and dK/dV kernels launch one workgroup per resident slot and walk this
schedule instead of taking one tile each.  A tile that no workgroup takes would be left
unwritten, and one that two take would be written twice; the parity tests see only the
grids their shapes produce.  Here the schedule itself is compiled for the host and
checked over many (tiles, workgroups) pairs: every tile exactly once, each workgroup
within its XCD's block, and, for tiles whose lengths fall linearly within each head
(the causal order), workgroups of one XCD within a few percent of each other's work.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_attn_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "common.h"
int main() {
  // total tiles, grid sizes: small and large, multiples of 8 and not
  const int totals[] = {1, 2, 7, 8, 9, 31, 64, 100, 255, 256, 257, 1000, 1024, 2048, 4095, 8192};
  const int grids[] = {1, 3, 7, 8, 9, 32, 100, 255, 256, 512};
  for (int total : totals)
    for (int grid0 : grids) {
      const int grid = grid0 < total ? grid0 : total;
      std::vector<int> seen(total, 0);
      for (int bid = 0; bid < grid; ++bid) {
        osattn::StaticSchedule s(total, bid, grid);
        const int k = grid < 8 ? grid : 8;
        for (int L = s.next(); L >= 0; L = s.next()) {
          if (L >= total) { printf("FAIL range %d %d %d\n", total, grid, L); return 1; }
          const int per = (total + k - 1) / k;
          if (L / per != bid % k) { printf("FAIL block %d %d %d\n", total, grid, L); return 1; }
          seen[L]++;
        }
      }
      for (int L = 0; L < total; ++L)
        if (seen[L] != 1) { printf("FAIL count %d %d %d %d\n", total, grid, L, seen[L]); return 1; }
    }
  // balance: heads of n tiles with lengths n, n-1, ..., 1 (longest first), 8 XCDs x 32
  for (int n : {32, 64, 128}) {
    const int heads = 64, total = heads * n, grid = 256;
    double lo = 1e30, hi = 0;
    for (int bid = 0; bid < grid; ++bid) {
      osattn::StaticSchedule s(total, bid, grid);
      double work = 0;
      for (int L = s.next(); L >= 0; L = s.next()) work += n - L % n;
      lo = work < lo ? work : lo;
      hi = work > hi ? work : hi;
    }
    printf("balance %d %.4f\n", n, hi / lo);
  }
  printf("OK\n");
  return 0;
}
"""


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def test_static_schedule_covers_every_tile_once(tmp_path):
    hipcc = _hipcc()
    if not hipcc:
        pytest.skip("hipcc not found")
    src = tmp_path / "sched.hip"
    exe = tmp_path / "sched"
    src.write_text(PROGRAM)
    build = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC,
                            str(src), "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and "OK" in run.stdout, run.stdout + run.stderr
    for line in run.stdout.splitlines():
        if line.startswith("balance"):
            _, n, ratio = line.split()
            assert float(ratio) <= 1.05, line  # max / min work of one XCD's workgroups
