// Block quantisation of bf16 to OCP E4M3 for gfx950.
//
// Method (greentreeone.com NeMo RL FP8 article, «Технический прорыв»): one
// scale per 1x128 activation group and per 128x128 weight block; power-of-two
// scales as an option (upppp.jp NeMo RL FP8 article, «設定方法»).
//
// Per group/block: amax = max|x|; s = RN32(amax/448), or the smallest power
// of two with 448*s >= amax; code = E4M3_RNE_saturating(RN32(x/s)); s = 0 and
// codes +-0 for an all-zero group.
//
// Both kernels are bound by HBM traffic (3 bytes in/out per element plus the
// scales), so the design is about coalescing and bytes in flight:
//   * activations: a 16-lane DPP row owns one 128-wide group; each lane
//     moves 16 bytes in (8 bf16) and 8 bytes out; a wave handles 16
//     consecutive groups (4 KB) with four independent 1 KB loads in flight;
//   * weights: a 256-thread workgroup owns one 128x128 block held entirely
//     in registers (64 values per thread), reduced through DPP and LDS.
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
#include "common.h"

namespace fp8blk {
namespace {

constexpr float kFastMinScale = 0x1p-90f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float group_scale(float amax, int pow2) {
  if (amax == 0.0f) return 0.0f;
  if (!pow2) return amax / kE4M3Max;  // correctly rounded fp32 division
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
    for (int j = 0; j < 8; ++j) q[j] = (s == 0.0f) ? 0.0f : a[j] / s;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = fminf(q[j], kE4M3Max);  // saturate

  uint32_t c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  c0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c0, true);
  uint32_t c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  c1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], c1, true);
  // bytes 1 and 3 of each bf16 pair hold the two sign bits (bit 7 of each)
  c0 |= __builtin_amdgcn_perm(w[1], w[0], 0x07050301u) & 0x80808080u;
  c1 |= __builtin_amdgcn_perm(w[3], w[2], 0x07050301u) & 0x80808080u;
  return u32x2{c0, c1};
}

// x, q viewed as 16-byte / 8-byte units: group g occupies units 16g .. 16g+15.
__global__ __launch_bounds__(256) void quant_act_kernel(const u32x4* __restrict__ x,
                                                        u32x2* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t groups, int pow2) {
  const int lane = threadIdx.x & 63;
  const int64_t g_wave = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t g = g_wave + u * 4 + (lane >> 4);
    v[u] = g < groups ? __builtin_nontemporal_load(&x[g * 16 + (lane & 15)]) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t g = g_wave + u * 4 + (lane >> 4);
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
    m = row16_max(m);  // all 64 lanes take part
    const float sc = group_scale(m, pow2);
    const u32x2 codes = encode8(w, sc);
    if (g < groups) {
      __builtin_nontemporal_store(codes, &q[g * 16 + (lane & 15)]);
      if ((lane & 15) == 0) s[g] = sc;
    }
  }
}

// One workgroup per 128x128 block. Thread t holds rows (t>>4) + 16i, i < 8,
// columns 8*(t&15) .. +7 of the block.
__global__ __launch_bounds__(256) void quant_weight_kernel(const u32x4* __restrict__ w,
                                                           u32x2* __restrict__ q,
                                                           float* __restrict__ s,
                                                           int64_t kblocks, int64_t K, int pow2) {
  __shared__ float red[16];
  const int t = threadIdx.x;
  const int64_t bi = blockIdx.x / kblocks;
  const int64_t bj = blockIdx.x % kblocks;
  const int64_t row_units = K / 8;  // 16-byte units per bf16 row
  const int64_t base = (bi * kBlock + (t >> 4)) * row_units + bj * 16 + (t & 15);

  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(&w[base + (int64_t)i * 16 * row_units]);

  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ww[j])), fabsf(bf16_hi(ww[j]))));
  }
  m = row16_max(m);
  if ((t & 15) == 0) red[t >> 4] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
  const float sc = group_scale(m, pow2);

  const int64_t qrow_units = K / 8;  // 8-byte units per code row
  const int64_t qbase = (bi * kBlock + (t >> 4)) * qrow_units + bj * 16 + (t & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    __builtin_nontemporal_store(encode8(ww, sc), &q[qbase + (int64_t)i * 16 * qrow_units]);
  }
  if (t == 0) s[blockIdx.x] = sc;
}

// ---------------------------------------------------------------------------
// Producers fused with the activation quantization (the pages name the
// quantization kernels as overhead and their fusion as the way past it:
// upppp.jp «重要度サンプリングで精度を保つ», greentreeone.com «Реальные
// прирост производительности»). Each computes the producer's output in fp32,
// rounds it once to bf16 (what the unfused producer would write), and
// quantizes those bf16 values exactly as quant_act_kernel does; the bf16
// values can also be written out (y != nullptr).

// Sum over the 16 lanes of a DPP row, then over the four rows: every lane
// gets the wave total. All 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
}

// Quantize one lane's 8 bf16 values w[0..3] as part of the 128-wide group
// formed by its 16-lane DPP row, and store codes, scale and (optionally)
// the bf16 values. `live` is uniform over the row; every lane of the wave
// must call this (DPP).
__device__ __forceinline__ void quant_store8(const uint32_t w[4], int pow2, bool live, u32x2* q_unit,
                                             float* s_group, bool first_lane, u32x4* y_unit) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  m = row16_max(m);
  const float sc = group_scale(m, pow2);
  const u32x2 codes = encode8(w, sc);
  if (live) {
    __builtin_nontemporal_store(codes, q_unit);
    if (first_lane) *s_group = sc;
    if (y_unit) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, y_unit);
  }
}

// RMSNorm + quantization: one wave per row of K (K % 128 == 0) elements.
// The row is walked in 512-element chunks (lane l holds elements 8l..8l+7
// of a chunk, so each 16-lane row holds one 128-wide group); the first
// kCachedChunks stay in registers between the two passes, later ones are
// read again (from L2).
constexpr int kCachedChunks = 8;  // K <= 4096 kept in registers

// Second pass over one chunk: y = bf16(x * r * gamma), then quantize. Every
// lane of the wave calls it (DPP inside); lanes past the row end store nothing.
__device__ __forceinline__ void rmsnorm_quant_chunk(u32x4 v, const u32x4* __restrict__ gamma, float r, int64_t u,
                                                    int64_t units, int64_t row, int64_t kb, int lane,
                                                    u32x2* __restrict__ q, float* __restrict__ s,
                                                    u32x4* __restrict__ y, int pow2) {
  const bool live = u < units;  // whole 16-lane rows (K % 128 == 0)
  const u32x4 gv = live ? gamma[u] : u32x4{0, 0, 0, 0};
  const uint32_t xw[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack_bf16(bf16_lo(xw[i]) * r * bf16_lo(gw[i]), bf16_hi(xw[i]) * r * bf16_hi(gw[i]));
  quant_store8(w, pow2, live, &q[row * units + u], &s[row * kb + u / 16], (lane & 15) == 0,
               y ? &y[row * units + u] : nullptr);
}

__global__ __launch_bounds__(256) void rmsnorm_quant_act_kernel(const u32x4* __restrict__ x,
                                                                const u32x4* __restrict__ gamma, float eps,
                                                                int64_t M, int64_t K, u32x2* __restrict__ q,
                                                                float* __restrict__ s, u32x4* __restrict__ y,
                                                                int pow2) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform over the wave
  const int64_t units = K / 8;                     // 16-byte units per row
  const int64_t chunks = (units + 63) / 64;
  const u32x4* xr = x + row * units;

  u32x4 cache[kCachedChunks];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kCachedChunks; ++c) {
    const int64_t u = (int64_t)c * 64 + lane;
    cache[c] = (c < chunks && u < units) ? __builtin_nontemporal_load(&xr[u]) : u32x4{0, 0, 0, 0};
    const uint32_t w[4] = {cache[c].x, cache[c].y, cache[c].z, cache[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  for (int64_t c = kCachedChunks; c < chunks; ++c) {
    const int64_t u = c * 64 + lane;
    const u32x4 v = u < units ? xr[u] : u32x4{0, 0, 0, 0};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  // r = 1 / sqrt(mean + eps): correctly rounded fp32 division and square root
  const float r = 1.0f / sqrtf(ss / (float)K + eps);

  const int64_t kb = K / kBlock;
#pragma unroll
  for (int c = 0; c < kCachedChunks; ++c)
    if (c < chunks)  // uniform
      rmsnorm_quant_chunk(cache[c], gamma, r, c * 64 + lane, units, row, kb, lane, q, s, y, pow2);
  for (int64_t c = kCachedChunks; c < chunks; ++c) {
    const int64_t u = c * 64 + lane;
    rmsnorm_quant_chunk(u < units ? xr[u] : u32x4{0, 0, 0, 0}, gamma, r, u, units, row, kb, lane, q, s, y, pow2);
  }
}

// SiLU(gate) * up + quantization. gu is [M][2F] = [gate | up] per row; the
// output groups are the M * F/128 groups of h = silu(g) * u, laid out like
// quant_act_kernel's (a 16-lane row per group, 16 groups per wave).
__global__ __launch_bounds__(256) void silu_mul_quant_act_kernel(const u32x4* __restrict__ gu,
                                                                 u32x2* __restrict__ q, float* __restrict__ s,
                                                                 u32x4* __restrict__ y, int64_t groups,
                                                                 int64_t fb, int pow2) {
  const int lane = threadIdx.x & 63;
  const int64_t g_wave = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
  u32x4 gv[4], uv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t gi = g_wave + k * 4 + (lane >> 4);
    const int64_t m = gi / fb, b = gi % fb;
    const int64_t src = m * (2 * fb * 16) + b * 16 + (lane & 15);  // 16-byte units; up starts fb*16 later
    gv[k] = gi < groups ? __builtin_nontemporal_load(&gu[src]) : u32x4{0, 0, 0, 0};
    uv[k] = gi < groups ? __builtin_nontemporal_load(&gu[src + fb * 16]) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t gi = g_wave + k * 4 + (lane >> 4);
    const uint32_t gw[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w}, uw[4] = {uv[k].x, uv[k].y, uv[k].z, uv[k].w};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = bf16_lo(gw[i]), g1 = bf16_hi(gw[i]);
      const float h0 = g0 / (1.0f + expf(-g0)) * bf16_lo(uw[i]);
      const float h1 = g1 / (1.0f + expf(-g1)) * bf16_hi(uw[i]);
      w[i] = pack_bf16(h0, h1);
    }
    const int64_t unit = gi * 16 + (lane & 15);
    quant_store8(w, pow2, gi < groups, &q[unit], &s[gi], (lane & 15) == 0, y ? &y[unit] : nullptr);
  }
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status fp8blk_quant_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                                          float* s, int pow2, hipStream_t stream) {
  if (M < 0 || K <= 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (K % kBlock) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !q || !s) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t groups = M * (K / kBlock);
  const int64_t blocks = (groups + 63) / 64;  // 4 waves x 16 groups
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(quant_act_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), s, groups, pow2);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                                             float* s, int pow2, hipStream_t stream) {
  if (N < 0 || K <= 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (N % kBlock || K % kBlock) return FP8BLK_ERR_SHAPE;
  if (N == 0) return FP8BLK_OK;
  if (!w || !q || !s) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t kblocks = K / kBlock;
  const int64_t blocks = (N / kBlock) * kblocks;
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(quant_weight_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(w), reinterpret_cast<u32x2*>(q), s, kblocks, K,
                     pow2);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_rmsnorm_quant_act(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                                  int64_t K, uint8_t* q, float* s, uint16_t* y, int pow2,
                                                  hipStream_t stream) {
  if (M < 0 || K <= 0 || (pow2 != 0 && pow2 != 1) || !(eps >= 0.0f) || !(eps < INFINITY))
    return FP8BLK_ERR_INVALID_ARG;
  if (K % kBlock) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !gamma || !q || !s) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(q, 16) || !aligned(s, 4) || (y && !aligned(y, 16)))
    return FP8BLK_ERR_ALIGNMENT;
  const int64_t blocks = (M + 3) / 4;  // one wave per row
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(rmsnorm_quant_act_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<const u32x4*>(gamma), eps, M, K,
                     reinterpret_cast<u32x2*>(q), s, reinterpret_cast<u32x4*>(y), pow2);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_silu_mul_quant_act(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s,
                                                   uint16_t* y, int pow2, hipStream_t stream) {
  if (M < 0 || F <= 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (F % kBlock) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!gu || !q || !s) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(gu, 16) || !aligned(q, 16) || !aligned(s, 4) || (y && !aligned(y, 16))) return FP8BLK_ERR_ALIGNMENT;
  const int64_t fb = F / kBlock;
  const int64_t groups = M * fb;
  const int64_t blocks = (groups + 63) / 64;  // 4 waves x 16 groups
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(silu_mul_quant_act_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(gu), reinterpret_cast<u32x2*>(q), s, reinterpret_cast<u32x4*>(y),
                     groups, fb, pow2);
  return launch_status();
}

extern "C" const char* fp8blk_status_string(fp8blk_status status) {
  switch (status) {
    case FP8BLK_OK: return "ok";
    case FP8BLK_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad flag)";
    case FP8BLK_ERR_SHAPE: return "unsupported shape (K and N must be multiples of 128, GEMM K <= 2^24, E >= 1)";
    case FP8BLK_ERR_ALIGNMENT: return "misaligned pointer (data 16 bytes, scales 4 bytes)";
    case FP8BLK_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}
