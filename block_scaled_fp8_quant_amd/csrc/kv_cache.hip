// FP8 KV cache on gfx950: per-step Q/K/V scale recalibration and the
// quantize-and-write of K and V into the cache.
//
// Method (upppp.jp NeMo RL FP8 article, «KVキャッシュとAttentionにも拡張»;
// greentreeone.com article, «Реальные прирост производительности»): the KV
// cache is stored in FP8; because the policy's weights change every training
// step, the Q, K and V scales are recomputed from BF16 activations at the end
// of each step and used by the next rollout.
//
// Granularity (not stated on the pages): one scale per tensor -- Q, K and V
// of one attention layer -- with the linear layers' rule s = RN32(amax/448)
// (or the power-of-two option). Recalibration is a max reduction over every
// chunk of the calibration batch (fp8blk_qkv_amax) followed by
// fp8blk_kv_scales; the cache write quantizes each token's K and V rows with
// those scales. Both are HBM-bound streams.
#include <algorithm>

#include "common.h"
#include "quant_common.h"

namespace fp8blk {
namespace {

// One 1024-thread workgroup per CU: eight 16-byte loads per thread keep
// 128 KB in flight per CU, and at most 3 x 256 atomics reach L2.
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxMaxWGs = 256;

__global__ void kv_amax_reset_kernel(float* __restrict__ amax) {
  if (threadIdx.x < 3) amax[threadIdx.x] = 0.0f;
}

// Largest |Q|, |K|, |V| of qkv [T][C] (C = (Hq + 2 Hkv) D, 16-byte units:
// row_units = C/8, of which the first q_units are Q and the next kv_units K).
// The matrix is streamed as one flat range of units: workgroup steps of
// kAmaxThreads x kAmaxUnroll units, eight independent loads per thread
// whatever the row boundaries. A unit's section follows from its column:
// one 64-bit modulo per step, then each load advances it by
// inc = kAmaxThreads mod row_units (so one conditional subtraction wraps it). Per-thread maxima are kept as fp32 bits (the
// order of the bit patterns of non-negative floats is their numeric order),
// reduced over the wave by DPP, over the workgroup through LDS, and folded
// into amax by an atomic max per tensor: max is exact and order-independent,
// so the result is the same whatever the order of the atomics. Atomics on one
// address serialize in L2, so a workgroup first reads the current maximum and
// skips the atomic when it would not raise it (a stale read only costs a
// redundant atomic).
constexpr int kAmaxUnroll = 8;

__global__ __launch_bounds__(kAmaxThreads) void qkv_amax_kernel(const u32x4* __restrict__ qkv, int64_t total,
                                                                int64_t row_units, int64_t inc, int64_t q_units,
                                                                int64_t kv_units, uint32_t* __restrict__ amax_bits) {
  constexpr int kWaves = kAmaxThreads / 64;
  __shared__ uint32_t red[kWaves][3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int64_t kStep = (int64_t)kAmaxThreads * kAmaxUnroll;
  uint32_t m[3] = {0, 0, 0};
  for (int64_t base = (int64_t)blockIdx.x * kStep; base < total; base += (int64_t)gridDim.x * kStep) {
    u32x4 v[kAmaxUnroll];
#pragma unroll
    for (int j = 0; j < kAmaxUnroll; ++j) {
      const int64_t f = base + j * kAmaxThreads + threadIdx.x;
      v[j] = f < total ? __builtin_nontemporal_load(&qkv[f]) : u32x4{0, 0, 0, 0};
    }
    int64_t col = (base + threadIdx.x) % row_units;
#pragma unroll
    for (int j = 0; j < kAmaxUnroll; ++j) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      const uint32_t a = amax8_bits(w);  // 0 for units past the end
      const int sec = col < q_units ? 0 : (col < q_units + kv_units ? 1 : 2);
      m[0] = sec == 0 ? max(m[0], a) : m[0];
      m[1] = sec == 1 ? max(m[1], a) : m[1];
      m[2] = sec == 2 ? max(m[2], a) : m[2];
      col += inc;
      if (col >= row_units) col -= row_units;  // col + inc < 2 row_units
    }
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    uint32_t x = row16_max_bits(m[i]);
    x = max(x, (uint32_t)__shfl_xor((int)x, 16));
    x = max(x, (uint32_t)__shfl_xor((int)x, 32));
    if (lane == 0) red[wave][i] = x;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    uint32_t x = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) x = max(x, red[w][threadIdx.x]);
    if (x > __hip_atomic_load(&amax_bits[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(&amax_bits[threadIdx.x], x);
  }
}

__global__ void kv_scales_kernel(const float* __restrict__ amax, int64_t n, float* __restrict__ scale, int pow2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scale[i] = group_scale(amax[i], pow2);
}

// One wave per token: K and V rows (Hkv heads of head_units 16-byte bf16
// units, read with row stride ld_units) are quantized with the per-tensor
// scales and written to slot slot[t] of the head-major paged caches
// [num_slots / block_size][Hkv][block_size][D] (skipped when negative or
// past the cache): each head's 8-byte code units go to its own panel.
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, int64_t ld_units, int64_t T, int64_t Hkv,
    int64_t head_units, const int64_t* __restrict__ slot, int64_t num_slots, int64_t block_size,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, u32x2* __restrict__ k_cache,
    u32x2* __restrict__ v_cache) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform over the wave
  const u32x4* kr = k + t * ld_units;
  const u32x4* vr = v + t * ld_units;
  const int64_t row_units = Hkv * head_units;
  // The first 128 units of K and V are loaded before the slot index is read,
  // so the two memory round trips overlap (a skipped token wastes them).
  u32x4 k1, v1, k2, v2;
  auto load = [&](int64_t u0) {
    const int64_t u1 = u0 + lane, u2 = u0 + 64 + lane;
    const bool l1 = u1 < row_units, l2 = u2 < row_units;
    k1 = l1 ? __builtin_nontemporal_load(&kr[u1]) : u32x4{0, 0, 0, 0};
    v1 = l1 ? __builtin_nontemporal_load(&vr[u1]) : u32x4{0, 0, 0, 0};
    k2 = l2 ? __builtin_nontemporal_load(&kr[u2]) : u32x4{0, 0, 0, 0};
    v2 = l2 ? __builtin_nontemporal_load(&vr[u2]) : u32x4{0, 0, 0, 0};
  };
  load(0);
  const int64_t sl = slot[t];
  if (sl < 0 || sl >= num_slots) return;  // uniform
  const float ks = *k_scale, vs = *v_scale;
  const float kinv = 1.0f / ks, vinv = 1.0f / vs;  // correctly rounded (inf for a zero scale: unused)
  const bool kf = ks >= kCalibratedMinScale && ks <= kCalibratedMaxScale;
  const bool vf = vs >= kCalibratedMinScale && vs <= kCalibratedMaxScale;
  // head-major pages: head h of slot sl is row sl % block_size of head h's
  // block_size x D panel in page sl / block_size
  const int64_t page = sl / block_size, row = sl % block_size;
  const int64_t first = (page * Hkv * block_size + row) * head_units;  // head 0's row (8-byte units)
  const int64_t head_stride = block_size * head_units;
  const uint32_t hu = (uint32_t)head_units;
  u32x2* kc = k_cache + first;
  u32x2* vc = v_cache + first;
  auto dst = [&](int64_t u) {  // unit u of the token's [Hkv][D] codes
    const uint32_t h = (uint32_t)u / hu;
    return (int64_t)h * head_stride + ((uint32_t)u - h * hu);
  };
  for (int64_t u0 = 0; u0 < row_units; u0 += 128) {
    if (u0 > 0) load(u0);  // uniform
    const int64_t u1 = u0 + lane, u2 = u0 + 64 + lane;
    const bool l1 = u1 < row_units, l2 = u2 < row_units;
    const uint32_t wk1[4] = {k1.x, k1.y, k1.z, k1.w}, wv1[4] = {v1.x, v1.y, v1.z, v1.w};
    const uint32_t wk2[4] = {k2.x, k2.y, k2.z, k2.w}, wv2[4] = {v2.x, v2.y, v2.z, v2.w};
    if (l1) {
      const int64_t d1 = dst(u1);
      __builtin_nontemporal_store(encode8_calibrated(wk1, ks, kinv, kf), &kc[d1]);
      __builtin_nontemporal_store(encode8_calibrated(wv1, vs, vinv, vf), &vc[d1]);
    }
    if (l2) {
      const int64_t d2 = dst(u2);
      __builtin_nontemporal_store(encode8_calibrated(wk2, ks, kinv, kf), &kc[d2]);
      __builtin_nontemporal_store(encode8_calibrated(wv2, vs, vinv, vf), &vc[d2]);
    }
  }
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status fp8blk_qkv_amax(const uint16_t* qkv, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                                         float* amax, int reset, hipStream_t stream) {
  if (T < 0 || Hq < 1 || Hkv < 1 || D < 1 || (reset != 0 && reset != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (D % 8) return FP8BLK_ERR_SHAPE;
  if (T == 0 && !reset) return FP8BLK_OK;  // nothing to do
  if (!amax || (T > 0 && !qkv)) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(amax, 4) || (T > 0 && !aligned(qkv, 16))) return FP8BLK_ERR_ALIGNMENT;
  const int64_t row_units = (Hq + 2 * Hkv) * D / 8;
  if (row_units > INT32_MAX || T > INT64_MAX / 2 / row_units) return FP8BLK_ERR_SHAPE;
  if (reset) hipLaunchKernelGGL(kv_amax_reset_kernel, dim3(1), dim3(64), 0, stream, amax);
  if (T > 0) {
    const int64_t total = T * row_units;
    const int64_t step = (int64_t)kAmaxThreads * kAmaxUnroll;
    const int64_t wgs = std::min<int64_t>((total + step - 1) / step, kAmaxMaxWGs);
    hipLaunchKernelGGL(qkv_amax_kernel, dim3((uint32_t)wgs), dim3(kAmaxThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(qkv), total, row_units, kAmaxThreads % row_units, Hq * D / 8,
                       Hkv * D / 8, reinterpret_cast<uint32_t*>(amax));
  }
  return launch_status();
}

extern "C" fp8blk_status fp8blk_kv_scales(const float* amax, int64_t n, float* scale, int pow2, hipStream_t stream) {
  if (n < 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (n == 0) return FP8BLK_OK;
  if (!amax || !scale) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(amax, 4) || !aligned(scale, 4)) return FP8BLK_ERR_ALIGNMENT;
  if ((n + 255) / 256 > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(kv_scales_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, amax, n, scale, pow2);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_kv_cache_write(const uint16_t* k, const uint16_t* v, int64_t ld, int64_t T,
                                               int64_t Hkv, int64_t D, const int64_t* slot, int64_t num_slots,
                                               int64_t block_size, const float* k_scale, const float* v_scale,
                                               uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream) {
  if (T < 0 || Hkv < 1 || D < 1 || num_slots < 0 || block_size < 1 || ld < Hkv * D) return FP8BLK_ERR_INVALID_ARG;
  if (D % 8 || ld % 8 || num_slots % block_size || Hkv * D > INT32_MAX) return FP8BLK_ERR_SHAPE;
  if (T == 0) return FP8BLK_OK;
  if (!k || !v || !slot || !k_scale || !v_scale || (num_slots > 0 && (!k_cache || !v_cache)))
    return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot, 8) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return FP8BLK_ERR_ALIGNMENT;
  const int64_t blocks = (T + 3) / 4;  // one wave per token
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(k), reinterpret_cast<const u32x4*>(v), ld / 8, T, Hkv, D / 8,
                     slot, num_slots, block_size, k_scale, v_scale, reinterpret_cast<u32x2*>(k_cache),
                     reinterpret_cast<u32x2*>(v_cache));
  return launch_status();
}
