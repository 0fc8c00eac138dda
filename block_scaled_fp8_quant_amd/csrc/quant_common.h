// Device helpers shared by the E4M3 quantization kernels (quant.hip,
// kv_cache.hip): the scale rule, the group maximum and the encoders.
//
// The quotient RN32(x/s) is formed with one IEEE division per lane (the
// reciprocal r = RN32(1/s)) and a corrected product per element:
//     q0 = |x| * r;  e = fma(s, q0, -|x|);  q = fma(-e, r, q0)
// This equals the IEEE quotient for every quotient >= 2**-12 whenever
// s >= 2**-90 (checked exhaustively on the CPU over every bf16 pair
// |x| <= amax in both scale modes); smaller quotients all give the code +-0
// either way. Groups with s < 2**-90 use a true division per element. The
// sign never passes through this arithmetic: magnitudes are encoded and the
// bf16 sign bits are OR-ed into the codes, which keeps -0 as 0x80.
#pragma once

#include "common.h"

namespace fp8blk {

constexpr float kFastMinScale = 0x1p-90f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (two dwords, byte i = element i) -> 8 fp16 values. Exact:
// every E4M3 value (subnormals included) is an fp16 value.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// RN32(amax / 448) without a division: q0 = amax * RN32(1/448), then one
// fma-corrected step. Equal to the IEEE quotient for every positive finite
// bf16 amax, subnormal results included (checked exhaustively on the CPU);
// amax is always a bf16 value here, the largest magnitude of its group.
constexpr float kInv448 = 0x1.24924ap-9f;  // RN32(1/448)

__device__ __forceinline__ float group_scale(float amax, int pow2) {
  if (amax == 0.0f) return 0.0f;
  if (!pow2) {
    const float q0 = amax * kInv448;
    return __builtin_fmaf(-__builtin_fmaf(kE4M3Max, q0, -amax), kInv448, q0);
  }
  // amax = m * 2**e with m in [0.5, 1); 448 * 2**k = 0.875 * 2**(k+9).
  // k = e-9 suffices iff m <= 0.875 (k = e-10 never does), else k = e-8.
  int e;
  const float m = frexpf(amax, &e);
  return ldexpf(1.0f, m <= 0.875f ? e - 9 : e - 8);
}

// Encode 8 bf16 values (packed two per word in w[0..3]) under scale s.
// Returns the 8 codes, element 0 in the lowest byte of the first word.
__device__ __forceinline__ u32x2 encode8(const uint32_t w[4], float s) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] = fabsf(bf16_lo(w[i]));
    a[2 * i + 1] = fabsf(bf16_hi(w[i]));
  }
  // v_cvt_pk_fp8_f32 rounds to nearest even and gives the NaN code only
  // above 464 (the midpoint between 448 and 480). With a normal scale every
  // quotient is at most RN32(amax / s) <= 448 (1 + 2^-23), so the fast path
  // needs no clamp; a subnormal scale can be rounded far below amax / 448,
  // so the division path clamps at 448.
  float q[8];
  if (s >= kFastMinScale) {
    const float r = 1.0f / s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q0 = a[j] * r;
      const float e = __builtin_fmaf(s, q0, -a[j]);
      q[j] = __builtin_fmaf(-e, r, q0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (s == 0.0f) ? 0.0f : fminf(a[j] / s, kE4M3Max);
  }

  uint32_t c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c0, true);
  uint32_t c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], c1, true);
  // bytes 1 and 3 of each bf16 pair hold the two sign bits (bit 7 of each)
  c0 |= __builtin_amdgcn_perm(w[1], w[0], 0x07050301u) & 0x80808080u;
  c1 |= __builtin_amdgcn_perm(w[3], w[2], 0x07050301u) & 0x80808080u;
  return u32x2{c0, c1};
}

// Largest magnitude of the 8 bf16 values in w[0..3], as fp32 bits. For
// finite non-negative floats the order of the bit patterns is the numeric
// order, so the maximum is taken on the packed 16-bit magnitudes (one
// v_pk_max_u16 per two values) and widened once.
__device__ __forceinline__ uint32_t amax8_bits(const uint32_t w[4]) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  const uint32_t p = __builtin_bit_cast(uint32_t, m);
  return max(p << 16, p & 0xFFFF0000u);
}

// Maximum of non-negative fp32 bit patterns over a 16-lane DPP row (lanes
// 16r .. 16r+15): quad_perm swaps lanes 1<->0 and 2<->3, then pairs of
// lanes; row_half_mirror and row_mirror fold 8 and 16 lanes. Every lane of
// the row must be active.
// No lane of these patterns reads outside its row, so the 0 supplied for
// out-of-row sources (bound_ctrl) never takes part; with it the compiler
// fuses each exchange into one v_max_u32_dpp.
__device__ __forceinline__ uint32_t row16_max_bits(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
  return v;
}

// Encode 8 bf16 values under a scale that does not come from their own
// maximum (a calibrated per-tensor scale): quotients may exceed 448 or the
// fp32 range and saturate to 448; s = 0 gives codes +-0. For
// 2^-90 <= s <= 2^126 (`fast`) the quotient is the corrected reciprocal
// product with r = RN32(1/s), saturating as soon as q0 = RN32(|x| r)
// reaches 448 (the IEEE quotient is then above 432, whose code is 448
// anyway); its codes equal those of the clamped IEEE quotient for every
// bf16 |x| (checked exhaustively on the CPU over thousands of scales). Other
// scales take an IEEE division per element (small scales: the correction's
// residual underflows; large: r is subnormal).
constexpr float kCalibratedMinScale = 0x1p-90f;
constexpr float kCalibratedMaxScale = 0x1p126f;

__device__ __forceinline__ u32x2 encode8_calibrated(const uint32_t w[4], float s, float r, bool fast) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = fabsf(bf16_lo(w[i]));
    q[2 * i + 1] = fabsf(bf16_hi(w[i]));
  }
  if (fast) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q0 = q[j] * r;
      const float qc = fminf(__builtin_fmaf(__builtin_fmaf(-s, q0, q[j]), r, q0), kE4M3Max);
      q[j] = q0 >= kE4M3Max ? kE4M3Max : qc;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (s == 0.0f) ? 0.0f : fminf(q[j] / s, kE4M3Max);
  }
  uint32_t c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c0, true);
  uint32_t c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], c1, true);
  c0 |= __builtin_amdgcn_perm(w[1], w[0], 0x07050301u) & 0x80808080u;
  c1 |= __builtin_amdgcn_perm(w[3], w[2], 0x07050301u) & 0x80808080u;
  return u32x2{c0, c1};
}

}  // namespace fp8blk
