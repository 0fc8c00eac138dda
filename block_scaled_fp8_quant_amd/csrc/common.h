// Shared helpers of libfp8blk.so: host-side argument checks and small
// device utilities (bf16 unpacking and packing, buffer resources).
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

}  // namespace fp8blk
