"""Launch planning (moe_plan.h) checked on the host with g++.

The kernels size their register arrays and LDS from compile-time bounds; the
planner must never pick a schedule that exceeds them.  A small C++ driver
walks a grid of shapes and asserts, for every plan:
  * fused: at most kFusedMaxRows rows, tile rows <= kMaxTileRows;
  * coarse: coarse tiles are whole tiles, at most kMaxCoarseTiles of them,
    histogram entries <= kCoarseMaxHist, rows before a tile inside its coarse
    tile <= kCoarseMaxRowsPerTile, LDS of the scatter kernel <= 64 KiB;
  * staged: each grid dimension of the rank and scatter kernels within 32-bit
    work-item counts, up to the largest accepted row count;
  * wave: exactly the calls of at most kWaveMaxRows rows without a map, no
    workspace, LDS within bounds;
  * the workspace query bounds the requirement of every smaller call and is
    monotone in the token count.
The grid covers the plain sort over E experts and the local-expert sort over
B buckets with an E-entry map held in LDS, each with and without a row copy.
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
// Every grid dimension of the staged kernels stays within 32-bit work-item
// counts, and the grid covers every tile.
static void check_staged_grid(const PermutePlan& p) {
  unsigned gx = 0, gy = 0;
  staged_grid(p.num_tiles, gx, gy);
  const unsigned long long lim = 0xFFFFFFFFull;
  CHECK((unsigned long long)gx * kRankThreads <= lim && (unsigned long long)gx * kScatterThreads <= lim, "grid x %u", gx);
  CHECK((unsigned long long)gy <= lim && gy <= 65535u, "grid y %u", gy);
  CHECK((long long)gx * gy >= p.num_tiles, "grid %u x %u covers %lld tiles", gx, gy, (long long)p.num_tiles);
  CHECK((long long)gx * (gy - 1) < p.num_tiles || p.num_tiles == 0, "no all-empty grid row");
}
int main() {
  // the largest accepted row counts (N * topk < 2^31): tiles below 128 rows for topk 3 and 5
  for (int K : {1, 2, 3, 5, 7, 8}) {
    const long long N = ((1LL << 31) - 1) / K;
    const PermutePlan p = plan_permute(N, K, 64, 0);
    CHECK(!p.fused && !p.coarse, "K=%d N=%lld staged", K, N);
    check_staged_grid(p);
  }
  // without the 2-D grid topk 3 (126-row tiles) would need more than 2^32 work-items in one dimension
  CHECK((long long)plan_permute(((1LL << 31) - 1) / 3, 3, 64, 0).num_tiles * kScatterThreads > 0xFFFFFFFFLL,
        "the limit case is the one the 2-D grid exists for");
  const int Ks[] = {1, 2, 3, 8, 16, 64, 512, 1024};
  const int Es[] = {1, 8, 37, 128, 256, 1000, 1024};
  const long long Ns[] = {1, 7, 100, 2047, 2048, 2049, 4096, 8192, 8193, 16384, 30000, 65536, 140000, 1000000};
  for (int K : Ks) for (int E : Es) for (int mode = 0; mode < 6; ++mode) {
    if (K > E) continue;
    const bool index_only = mode >= 3;  // no row copy: fewer, larger fused tiles
    const int B = mode % 3 == 0 ? E : (mode % 3 == 1 ? (E / 8 > 0 ? E / 8 : 1) : E);  // buckets
    const int M = mode % 3 == 0 ? 0 : E;                                             // map entries
    size_t prev = 0;
    for (long long N : Ns) {
      if (N * K >= (1LL << 31)) continue;
      const PermutePlan p = plan_permute(N, K, B, M, index_only);
      const size_t bound = workspace_bound(N, K, B, M);
      CHECK(bound >= p.ws_bytes, "N=%lld K=%d B=%d M=%d bound %zu < need %zu", N, K, B, M, bound, p.ws_bytes);
      CHECK(bound >= prev, "N=%lld K=%d B=%d M=%d bound not monotone", N, K, B, M);
      prev = bound;
      for (long long n2 : {N / 2, N - 1, N / 3 + 1}) {
        if (n2 < 1) continue;
        const PermutePlan q = plan_permute(n2, K, B, M, index_only);
        CHECK(q.ws_bytes <= bound, "N=%lld smaller %lld K=%d B=%d needs %zu > %zu", N, n2, K, B, q.ws_bytes, bound);
      }
      CHECK(p.nbits >= 0 && (1 << p.nbits) >= B, "key bits");
      CHECK(p.tile_rows == p.tokens_per_tile * K, "tile rows");
      CHECK(p.tile_rows <= kMaxTileRows, "N=%lld K=%d tile rows %d", N, K, p.tile_rows);
      CHECK(p.wave == (N * K <= kWaveMaxRows && M == 0), "N=%lld K=%d M=%d wave schedule", N, K, M);
      if (p.wave) {
        CHECK(p.rows <= 2 * kWaveSize && p.ws_bytes == 0 && !p.fused && !p.coarse, "wave plan");
        CHECK(wave_lds_bytes(E, (int)p.rows) <= 4 * (size_t)kMaxLdsInts, "wave lds");
      } else if (p.fused) {
        CHECK(p.rows <= kFusedMaxRows, "fused rows");
        CHECK(fused_lds_bytes(B, p.tile_rows, M) <= 4 * kMaxLdsInts, "fused lds");
      } else if (p.coarse) {
        CHECK(p.coarse_rows % p.tile_rows == 0, "coarse rows %d not whole tiles of %d", p.coarse_rows, p.tile_rows);
        CHECK(p.num_coarse >= 1 && p.num_coarse <= kMaxCoarseTiles, "num coarse %d", p.num_coarse);
        CHECK((long long)p.num_coarse * p.coarse_rows >= p.rows, "coarse tiles cover the rows");
        CHECK((long long)(p.num_coarse - 1) * p.coarse_rows < p.rows, "no empty coarse tile");
        CHECK(p.num_coarse * (B + 1) <= kCoarseMaxHist, "hist entries %d", p.num_coarse * (B + 1));
        CHECK(p.coarse_rows - p.tile_rows <= kCoarseMaxRowsPerTile, "rows before a tile %d", p.coarse_rows - p.tile_rows);
        CHECK(coarse_scatter_lds_bytes(B, p.tile_rows, p.num_coarse, M) <= 4 * (size_t)kMaxLdsInts, "coarse lds");
        CHECK(coarse_hist_lds_bytes(B, M) <= 4 * (size_t)kMaxLdsInts, "coarse hist lds");
        CHECK(p.ws_bytes >= sizeof(int) * (size_t)p.num_coarse * (B + 1), "coarse workspace");
      } else {
        CHECK(p.ws_bytes >= staged_workspace_bytes(p.rows, p.num_tiles, B), "staged workspace");
        CHECK(rank_lds_bytes(B, p.tile_rows, M) <= 4 * (size_t)kMaxLdsInts, "rank lds");
        CHECK(scatter_lds_bytes(B, p.tile_rows, M) <= 4 * (size_t)kMaxLdsInts, "scatter lds");
        check_staged_grid(p);
      }
    }
  }
  // the named workloads take the schedules the design notes describe
  CHECK(plan_permute(4096, 2, 8, 0).fused, "mixtral fused");
  CHECK(plan_permute(8192, 8, 128, 0).coarse, "qwen3 coarse");
  CHECK(plan_permute(8192, 8, 128, 0).tile_rows == 64, "qwen3 coarse copy tiles of 64 rows");
  CHECK(plan_permute(16384, 8, 256, 0).tile_rows == 64, "dsv3 coarse copy tiles of 64 rows");
  CHECK(plan_permute(8192, 8, 128, 0, true).tile_rows == 512, "qwen3 index-only tiles of 512 rows");
  CHECK(plan_permute(16384, 8, 32, 256).tile_rows == 128, "expert map: staged-size tiles");
  CHECK(plan_permute(16384, 8, 256, 0).coarse, "dsv3 coarse");
  CHECK(plan_permute(256, 8, 256, 0).fused, "decode N=256 fused");
  CHECK(plan_permute(16, 8, 256, 0).wave && plan_permute(1, 8, 256, 0).wave, "decode N<=16 wave");
  CHECK(plan_permute(17, 8, 256, 0).fused && plan_permute(64, 8, 256, 0).fused, "decode N>16 fused");
  CHECK(plan_permute(16, 8, 256, 256).fused, "decode with an expert map: fused");
  CHECK(!plan_permute(140000, 2, 16, 0).coarse && !plan_permute(140000, 2, 16, 0).fused, "large staged");
  CHECK(plan_permute(16384, 8, 32, 256).coarse, "dsv3 one of eight expert ranks: coarse");
  CHECK(split_copy_applies(16384, 8, 7168 * 2, 0), "dsv3 bf16 rows: split copy");
  CHECK(split_copy_applies(16384, 8, 7168 * 2, 256), "dsv3 with an expert map: split copy");
  CHECK(!split_copy_applies(8192, 8, 2048 * 2, 128), "qwen3 with an expert map: no split copy");
  CHECK(!split_copy_applies(16384, 2, 4096 * 2, 8), "topk 2 with an expert map: no split copy");
  CHECK(!split_copy_applies(8192, 8, 2048 * 2, 0), "qwen3: no split copy");
  CHECK(!split_copy_applies(4096, 2, 4096 * 2, 0), "mixtral: no split copy");
  CHECK(!split_copy_applies(1 << 20, 8, 0, 0), "index only: no split copy");
  CHECK(split_copy_applies(1, 1, kSplitCopyMinBytes, 0) && !split_copy_applies(1, 1, kSplitCopyMinBytes - 16, 0),
        "split copy from kSplitCopyMinBytes on");
  std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
'''


def test_plans_respect_kernel_bounds(tmp_path):
    src = tmp_path / "plan_driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "plan_driver"
    extra = os.environ.get("MOE_TEST_SANITIZE_FLAGS", "").split()  # set by the sanitizer test
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", *extra, "-I", CSRC, "-o", str(exe), str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout[-3000:]
