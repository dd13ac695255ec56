"""Launch planning (moe_plan.h) checked on the host with g++.

The kernels size their register arrays and LDS from compile-time bounds; the
planner must never pick a schedule that exceeds them.  A small C++ driver
walks a grid of shapes and asserts, for every plan:
  * fused: at most kFusedMaxRows rows, tile rows <= kMaxTileRows;
  * coarse: coarse tiles are whole tiles, at most kMaxCoarseTiles of them,
    histogram entries <= kCoarseMaxHist, rows before a tile inside its coarse
    tile <= kCoarseMaxRowsPerTile, LDS of the scatter kernel <= 64 KiB;
  * the workspace query bounds the requirement of every smaller call and is
    monotone in the token count.
"""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_token_amd", "csrc")

DRIVER = r'''
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include "moe_plan.h"
using namespace moe;
static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { ++fails; std::printf("FAIL %s: ", #c); std::printf(__VA_ARGS__); std::printf("\n"); } } while (0)
int main() {
  const int Ks[] = {1, 2, 3, 8, 16, 64, 512, 1024};
  const int Es[] = {1, 8, 37, 128, 256, 1000, 1024};
  const long long Ns[] = {1, 7, 100, 2047, 2048, 2049, 4096, 8192, 8193, 16384, 30000, 65536, 140000, 1000000};
  for (int K : Ks) for (int E : Es) {
    if (K > E) continue;
    size_t prev = 0;
    for (long long N : Ns) {
      if (N * K >= (1LL << 31)) continue;
      const PermutePlan p = plan_permute(N, K, E);
      const size_t bound = workspace_bound(N, K, E);
      CHECK(bound >= p.ws_bytes, "N=%lld K=%d E=%d bound %zu < need %zu", N, K, E, bound, p.ws_bytes);
      CHECK(bound >= prev, "N=%lld K=%d E=%d bound not monotone", N, K, E);
      prev = bound;
      for (long long n2 : {N / 2, N - 1, N / 3 + 1}) {
        if (n2 < 1) continue;
        const PermutePlan q = plan_permute(n2, K, E);
        CHECK(q.ws_bytes <= bound, "N=%lld smaller %lld K=%d E=%d needs %zu > %zu", N, n2, K, E, q.ws_bytes, bound);
      }
      CHECK(p.tile_rows == p.tokens_per_tile * K, "tile rows");
      CHECK(p.tile_rows <= kMaxTileRows, "N=%lld K=%d tile rows %d", N, K, p.tile_rows);
      if (p.fused) {
        CHECK(p.rows <= kFusedMaxRows, "fused rows");
        CHECK(fused_lds_bytes(E, p.tile_rows) <= 4 * kMaxLdsInts, "fused lds");
      } else if (p.coarse) {
        CHECK(p.coarse_rows % p.tile_rows == 0, "coarse rows %d not whole tiles of %d", p.coarse_rows, p.tile_rows);
        CHECK(p.num_coarse >= 1 && p.num_coarse <= kMaxCoarseTiles, "num coarse %d", p.num_coarse);
        CHECK((long long)p.num_coarse * p.coarse_rows >= p.rows, "coarse tiles cover the rows");
        CHECK((long long)(p.num_coarse - 1) * p.coarse_rows < p.rows, "no empty coarse tile");
        CHECK(p.num_coarse * (E + 1) <= kCoarseMaxHist, "hist entries %d", p.num_coarse * (E + 1));
        CHECK(p.coarse_rows - p.tile_rows <= kCoarseMaxRowsPerTile, "rows before a tile %d", p.coarse_rows - p.tile_rows);
        CHECK(coarse_scatter_lds_bytes(E, p.tile_rows, p.num_coarse) <= 4 * (size_t)kMaxLdsInts, "coarse lds");
        CHECK(p.ws_bytes >= sizeof(int) * (size_t)p.num_coarse * (E + 1), "coarse workspace");
      } else {
        CHECK(p.ws_bytes >= staged_workspace_bytes(p.rows, p.num_tiles, E), "staged workspace");
        CHECK(rank_lds_bytes(E, p.tile_rows) <= 4 * (size_t)kMaxLdsInts, "rank lds");
      }
    }
  }
  // the named workloads take the schedules the design notes describe
  CHECK(plan_permute(4096, 2, 8).fused, "mixtral fused");
  CHECK(plan_permute(8192, 8, 128).coarse, "qwen3 coarse");
  CHECK(plan_permute(16384, 8, 256).coarse, "dsv3 coarse");
  CHECK(plan_permute(256, 8, 256).fused, "decode fused");
  CHECK(!plan_permute(140000, 2, 16).coarse && !plan_permute(140000, 2, 16).fused, "large staged");
  std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
'''


def test_plans_respect_kernel_bounds(tmp_path):
    src = tmp_path / "plan_driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "plan_driver"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, "-o", str(exe), str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout[-3000:]
