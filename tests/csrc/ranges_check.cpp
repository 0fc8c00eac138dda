// CPU check of the bounds arithmetic the grouped kernels use
// (block_scaled_fp8_quant_amd/csrc/ranges.h, compiled here unchanged with a
// plain C++ compiler). Offsets arrays that break the grouped GEMM's
// contract (negative, decreasing, past the row count, extreme int32 values)
// must never yield a row outside [0, total) or a negative tile.
//
// A host model of the grouped GEMM's launch (tile search over per-expert
// tile counts, then expert_tile) runs over random offsets, valid and
// broken: every row a workgroup may touch lies in [0, total), and with
// valid offsets every row of every expert is covered by exactly one tile.
//
// Prints "ok" and exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "ranges.h"

using namespace fp8blk;

static long failures = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      if (failures++ < 20) fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c); \
    }                                                             \
  } while (0)

static void check_clamp_len() {
  CHECK(clamp_len(-(int64_t(1) << 40)) == 0u);
  CHECK(clamp_len(-1) == 0u);
  CHECK(clamp_len(0) == 0u);
  CHECK(clamp_len(1) == 1u);
  CHECK(clamp_len(0xFFFFFFFEll) == 0xFFFFFFFEu);
  CHECK(clamp_len(0xFFFFFFFFll) == 0xFFFFFFFFu);
  CHECK(clamp_len(int64_t(1) << 32) == 0xFFFFFFFFu);
  CHECK(clamp_len(int64_t(1) << 40) == 0xFFFFFFFFu);
}

static void check_rows_and_counts() {
  const int32_t extremes[] = {INT32_MIN, INT32_MIN + 1, -1000, -129, -128, -1, 0, 1, 5, 127, 128, 129,
                              1000, INT32_MAX - 1, INT32_MAX};
  std::vector<int32_t> vals;
  for (int v = -20; v <= 40; ++v) vals.push_back(v);
  for (int32_t v : extremes) vals.push_back(v);
  const int64_t totals[] = {0, 1, 7, 20, 128, 1000, INT32_MAX};
  const int bms[] = {64, 128, 256};
  for (int32_t a : vals)
    for (int32_t b : vals) {
      for (int bm : bms) {
        const int c = tile_count(a, b, bm);
        const int64_t d = (int64_t)b - a;
        CHECK(c >= 0 && c <= kMaxTileCount);
        if (d <= 0) CHECK(c == 0);
        if (d > 0 && (d + bm - 1) / bm <= kMaxTileCount) CHECK(c == (d + bm - 1) / bm);
      }
      for (int64_t total : totals) {
        const RowRange r = clamp_rows(a, b, total);
        CHECK(0 <= r.lo && r.lo <= r.hi && r.hi <= total);
        if (0 <= a && a <= b && b <= total) CHECK(r.lo == a && r.hi == b);
        for (int bm : bms) {
          const int64_t tiles[] = {-1, 0, 1, 2, 3, 7, 1000, kMaxTileCount - 1, kMaxTileCount, INT32_MAX};
          for (int64_t tile : tiles) {
            int64_t row0 = -7, rows = -7, m0 = -7;
            const bool live = expert_tile(a, b, total, tile, bm, row0, rows, m0);
            CHECK(row0 >= 0 && rows >= 0 && row0 + rows <= total);
            if (live) {
              CHECK(m0 >= 0 && m0 < rows);
              // every row the tile may read or write: row0 + m0 + r, m0 + r < rows
              const int64_t last = row0 + (m0 + bm < rows ? m0 + bm : rows) - 1;
              CHECK(row0 + m0 >= 0 && last < total);
            }
            if (0 <= a && a <= b && b <= total && tile >= 0 && tile < kMaxTileCount)
              CHECK(live == (tile < tile_count(a, b, bm)));
          }
        }
      }
    }
  // the tile search sums up to 64 capped counts in 32 bits
  CHECK((int64_t)64 * kMaxTileCount <= INT32_MAX);
}

// Host model of one grouped launch: grid of (total / bm + E) row tiles; the
// tile search (sequential here) over tile_count; expert_tile. Returns the
// number of rows covered; with `cover` given, counts coverage per row.
static void model_launch(const std::vector<int32_t>& off, int64_t total, int bm, std::vector<int>* cover) {
  const int E = (int)off.size() - 1;
  const int64_t grid = total / bm + E;
  for (int64_t t = 0; t < grid; ++t) {
    int64_t base = 0;
    int expert = -1;
    int64_t tile = -1;
    for (int e = 0; e < E; ++e) {
      const int c = tile_count(off[e], off[e + 1], bm);
      if (t < base + c) {
        expert = e;
        tile = t - base;
        break;
      }
      base += c;
    }
    if (expert < 0) continue;
    CHECK(expert < E && tile >= 0);
    int64_t row0, rows, m0;
    if (!expert_tile(off[expert], off[expert + 1], total, tile, bm, row0, rows, m0)) continue;
    for (int64_t r = 0; r < bm && m0 + r < rows; ++r) {
      const int64_t row = row0 + m0 + r;
      CHECK(row >= 0 && row < total);
      if (cover && row >= 0 && row < total) (*cover)[row]++;
    }
  }
}

static void check_launch_model() {
  std::mt19937_64 rng(12345);
  const int bms[] = {64, 128, 256};
  for (int trial = 0; trial < 3000; ++trial) {
    const int E = 1 + (int)(rng() % 40);
    const int64_t total = (int64_t)(rng() % 3000);
    // valid offsets: sorted cut points in [0, total]
    std::vector<int32_t> off(E + 1);
    off[0] = 0;
    off[E] = (int32_t)total;
    std::vector<int32_t> cuts;
    for (int e = 1; e < E; ++e) cuts.push_back((int32_t)(total ? rng() % (total + 1) : 0));
    std::sort(cuts.begin(), cuts.end());
    for (int e = 1; e < E; ++e) off[e] = cuts[e - 1];
    for (int bm : bms) {
      std::vector<int> cover(total, 0);
      model_launch(off, total, bm, &cover);
      for (int64_t r = 0; r < total; ++r) CHECK(cover[r] == 1);
    }
    // broken offsets: random perturbations, extreme values, decreasing runs
    std::vector<int32_t> bad = off;
    const int kinds = 1 + (int)(rng() % 4);
    for (int k = 0; k < kinds; ++k) {
      const int e = (int)(rng() % (E + 1));
      switch (rng() % 6) {
        case 0: bad[e] = -(int32_t)(rng() % 5000); break;
        case 1: bad[e] = (int32_t)(total + rng() % 5000); break;
        case 2: bad[e] = INT32_MAX; break;
        case 3: bad[e] = INT32_MIN; break;
        case 4: bad[e] = (int32_t)(rng() % (total + 1)); break;  // out of order
        default: {  // one more than the next offset (a decreasing step)
          const int32_t nx = bad[(e + 1) % (E + 1)];
          bad[e] = nx < INT32_MAX ? nx + 1 : nx;
          break;
        }
      }
    }
    for (int bm : bms) model_launch(bad, total, bm, nullptr);
  }
}

int main() {
  check_clamp_len();
  check_rows_and_counts();
  check_launch_model();
  if (failures) {
    printf("failures=%ld\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
