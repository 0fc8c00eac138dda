// Shared helpers of libfp8blk.so: host-side argument checks and small
// device utilities (bf16 unpacking and packing, buffer resources).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8blk.h"
#include "ranges.h"

namespace fp8blk {

constexpr int kBlock = FP8BLK_BLOCK;     // 128: group width and block edge
constexpr float kE4M3Max = 448.0f;

// ------------------------------------------------------------------ host

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Map the result of a kernel launch to a status (no device synchronisation).
inline fp8blk_status launch_status() {
  return hipGetLastError() == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_HIP;
}

// ------------------------------------------------------------------ device

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Buffer resource over `bytes` bytes from `base` (raw, stride 0): loads at
// byte offsets past the end return zeros instead of faulting, which lets
// ragged edges be read without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// bf16 bits of an fp32 value, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes within each 16-lane row (DPP, lanes shifted in from outside the row
// read 0), then the totals of the earlier rows (readlane) added to each row.
// No LDS round trips, unlike lane shuffles.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Find which expert owns M-tile `t` (0 <= t < 2^24) of the concatenated
// per-expert tile lists (expert e has ceil(M_e / BM) tiles). Every lane of
// the wave computes the same answer: lanes take 64 experts at a time and a
// wave prefix sum turns per-expert tile counts into tile ranges. The
// results are passed through readfirstlane so the compiler knows they are
// uniform (they feed the scalar base addresses of buffer resources;
// otherwise each resource would be built in a loop over the lanes).
// Counts come from tile_count (negative lengths count 0, each count at most
// 2^24), so `base` stays below 2^24 + 2^30 and the returned expert is
// always in [0, E); offsets that break their contract give a wrong expert
// or tile, never an index outside the arrays.
template <int BM>
__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ off, int E, int t, int& expert,
                                            int& tile_in_expert) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int cnt = e < E ? tile_count(off[e], off[e + 1], BM) : 0;
    const int incl = wave_prefix_sum(cnt);
    const int total = __builtin_amdgcn_readlane(incl, 63);  // uniform: so is the branch
    if (t < base + total) {
      const bool mine = cnt > 0 && t >= base + incl - cnt && t < base + incl;
      const unsigned long long owners = (unsigned long long)__ballot(mine);
      if (owners == 0ull) return false;  // uniform; unreachable with consistent counts
      const int src = __builtin_amdgcn_readfirstlane(__ffsll(owners) - 1);
      expert = __builtin_amdgcn_readfirstlane(e0 + src);
      tile_in_expert = __builtin_amdgcn_readfirstlane(t - base - __builtin_amdgcn_readlane(incl - cnt, src));
      return true;
    }
    base += total;
  }
  return false;
}

// Sum over the experts before e of ceil(M_e' / BM): where expert e's tiles
// start in the concatenated per-expert tile lists (the same in every lane,
// returned as a uniform value; 64-bit, so broken offsets cannot wrap it).
template <int BM>
__device__ __forceinline__ int64_t tiles_before(const int32_t* __restrict__ off, int e) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int e0 = 0; e0 < e; e0 += 64) {
    const int i = e0 + lane;
    int cnt = i < e ? tile_count(off[i], off[i + 1], BM) : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) cnt += __shfl_xor(cnt, d);  // <= 64 * 2^24
    total += cnt;
  }
  return ((int64_t)__builtin_amdgcn_readfirstlane((int)(total >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)total);
}

}  // namespace fp8blk
