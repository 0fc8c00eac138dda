// Shared helpers of libfp8blk.so: host-side argument checks and small
// device utilities (bf16 unpacking, 16-lane DPP reductions, packing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8blk.h"

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

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15). Every lane
// of the row must be active. quad_perm swaps lanes 1<->0 and 2<->3, then
// pairs of lanes; row_half_mirror and row_mirror fold 8 and 16 lanes.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// bf16 bits of an fp32 value, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

}  // namespace fp8blk
