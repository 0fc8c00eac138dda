// Index arithmetic behind the kernels' bounds: buffer-resource lengths and
// the row ranges of experts read from device offsets. Free of HIP, so that
// the CPU tests compile exactly this code with a plain C++ compiler.
//
// The grouped kernels take each expert's rows from offsets[E+1] on the
// device. The documented contract (offsets[0] = 0, nondecreasing,
// offsets[E] = total rows) is not checked: with offsets that break it the
// results are wrong, but these helpers keep every access inside the
// buffers sized from the host-side row count.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8BLK_HD __host__ __device__ __forceinline__
#else
#define FP8BLK_HD inline
#endif

namespace fp8blk {

// Bytes a buffer resource may cover: negative lengths (a tile or an expert
// range past the operand's end) become 0, so every load through the
// resource reads zeros; 4 GB or more is clamped to the largest 32-bit value.
FP8BLK_HD uint32_t clamp_len(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes < 0xFFFFFFFFll ? (uint32_t)bytes : 0xFFFFFFFFu);
}

// Row range [lo, hi) of one expert, from offsets a = offsets[e] and
// b = offsets[e+1], clamped so that 0 <= lo <= hi <= total.
struct RowRange {
  int64_t lo, hi;
};
FP8BLK_HD RowRange clamp_rows(int64_t a, int64_t b, int64_t total) {
  const int64_t lo = a < 0 ? 0 : (a > total ? total : a);
  const int64_t hi = b < lo ? lo : (b > total ? total : b);
  return RowRange{lo, hi};
}

// Largest tile count one expert reports to the tile search. A launch has
// fewer than 2^24 workgroups, so a larger count changes no search result,
// and with the cap the search's sums of up to 64 counts stay in 32 bits.
constexpr int kMaxTileCount = 1 << 24;

// Tiles of bm rows that cover offsets a .. b: ceil((b - a) / bm) computed in
// 64 bits, 0 for a negative length, capped at kMaxTileCount.
FP8BLK_HD int tile_count(int32_t a, int32_t b, int bm) {
  const int64_t d = (int64_t)b - (int64_t)a;
  if (d <= 0) return 0;
  const int64_t t = (d + bm - 1) / bm;
  return t < kMaxTileCount ? (int)t : kMaxTileCount;
}

// The rows an expert-grouped GEMM workgroup works on: tile `tile` (bm rows)
// of the expert whose offsets are a, b, in an operand of `total` rows.
// Returns false when the tile holds no row of the clamped range (the
// workgroup then does nothing); otherwise row0 = the expert's first row,
// rows = its row count and m0 = the tile's first row relative to row0, with
// 0 <= m0 < rows and row0 + rows <= total.
FP8BLK_HD bool expert_tile(int32_t a, int32_t b, int64_t total, int64_t tile, int bm, int64_t& row0,
                           int64_t& rows, int64_t& m0) {
  const RowRange r = clamp_rows(a, b, total);
  row0 = r.lo;
  rows = r.hi - r.lo;
  if (tile < 0 || tile >= kMaxTileCount) return false;
  m0 = tile * (int64_t)bm;
  return m0 < rows;
}

}  // namespace fp8blk
