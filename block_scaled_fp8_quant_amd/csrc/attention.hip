// FP8 decode attention over the paged FP8 KV cache, for gfx950.
//
// Method (upppp.jp NeMo RL FP8 article, «KVキャッシュとAttentionにも拡張»;
// greentreeone.com article, «Реальные прирост производительности»): with long
// outputs the KV cache and attention dominate rollout time, so both run in
// FP8 with the Q/K/V scales recalibrated every training step.
//
// The decode step: each sequence's query (Hq heads of D = 128) attends over
// its cached tokens. Q is quantized per tensor with the calibrated Q scale
// (the cache write's quantizer); the scores are exact FP8 products,
//     s[h][t] = (q8[h] . k8[t][g]) * q_scale * k_scale * sm_scale,
// g = h / (Hq/Hkv); softmax in fp32; out[h] = sum_t p[h][t] v8[t][g] v_scale,
// probabilities kept in fp32; bf16 output.
//
// One workgroup per (sequence, KV head); its four waves take interleaved
// 64-token tiles of the context and keep their own running maximum, sum and
// output (online softmax), merged through LDS at the end. Per tile:
//   * the 64 tokens' cache slots come from the block table (one per lane;
//     out-of-range tokens, blocks or slots are masked);
//   * QK^T: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 tokens, source 0 =
//     the group's Q rows (heads, padded to 16 with zeros), source 1 = 16 K
//     rows loaded straight from the cache. Lane l then holds the scores of
//     heads 4(l/16)..+3 for token l%16 of the subtile, so every head's
//     maximum and sum over the tile are reductions over one 16-lane DPP row;
//   * PV on the VALU in fp32: 16 lanes cover the 128 values of one V row
//     (8 bytes each, one coalesced 128-byte read), four rows in flight, and
//     each lane accumulates G x 8 outputs; p comes from LDS.
// The cache reads are the bound (K and V, 256 bytes per token and KV head).
#include "common.h"
#include "quant_common.h"

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2eAttn = 1.44269504088896341f;

__device__ __forceinline__ float row16_max_f(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row16_sum_f(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Make this wave's LDS writes visible to its own later LDS reads by other
// lanes (LDS operations of one wave complete in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

template <int G>  // query heads per KV head: 1, 2, 4 or 8
__global__ __launch_bounds__(256) void decode_attention_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, int64_t Hkv, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, int64_t num_slots, const int32_t* __restrict__ block_table,
    int64_t max_blocks, int64_t block_size, const int32_t* __restrict__ context_lens,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    float sm_scale, uint16_t* __restrict__ out, int64_t ldo) {
  constexpr int D = kHeadDim;
  __shared__ __attribute__((aligned(16))) uint32_t q8[G * D / 4];
  __shared__ int32_t slot_tile[4][64];
  __shared__ __attribute__((aligned(16))) float ptile[4][64][G];
  __shared__ float m_w[4][G], l_w[4][G];
  __shared__ __attribute__((aligned(16))) float acc_w[4][G][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.x / Hkv, gk = blockIdx.x % Hkv;
  const int64_t L = context_lens[b] > 0 ? context_lens[b] : 0;
  const float qs = *q_scale, ks = *k_scale, vs = *v_scale;

  // Q of the group's G heads -> E4M3 codes in LDS
  if (tid < G * D / 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + b * ldq + gk * G * D + 8 * tid);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const bool fast = qs >= kCalibratedMinScale && qs <= kCalibratedMaxScale;
    const u32x2 c = encode8_calibrated(ww, qs, 1.0f / qs, fast);
    q8[2 * tid] = c.x;
    q8[2 * tid + 1] = c.y;
  }
  __syncthreads();

  const int g = lane >> 4, c16 = lane & 15;
  // source 0 fragment: head row c16 (zero past G), K chunks g and g+4
  v8i qfrag = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  if (c16 < G) {
    const uint4 lo = *reinterpret_cast<const uint4*>(&q8[(c16 * D + 16 * g) / 4]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&q8[(c16 * D + 64 + 16 * g) / 4]);
    qfrag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  const float s2scale = qs * ks * sm_scale * kLog2eAttn;  // scores in the log2 domain
  const int64_t row_bytes = Hkv * D;                    // one slot of one cache

  // running state: lane group g holds heads 4g..4g+3 (entries r < 4)
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  for (int64_t t0 = (int64_t)wave * 64; t0 < L; t0 += 256) {  // uniform over the wave
    {  // slots of the tile's tokens
      const int64_t t = t0 + lane;
      int32_t slot = -1;
      if (t < L && t / block_size < max_blocks) {
        const int64_t blk = block_table[b * max_blocks + t / block_size];
        const int64_t s = blk * block_size + t % block_size;
        if (blk >= 0 && s < num_slots) slot = (int32_t)s;
      }
      slot_tile[wave][lane] = slot;
    }
    wave_lds_sync();

    // QK^T: scores (log2 domain) of heads 4g+r, tokens 16u + c16
    float s[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t slot = slot_tile[wave][16 * u + c16];
      v8i kfrag = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      if (slot >= 0) {
        const uint8_t* kr = k_cache + (int64_t)slot * row_bytes + gk * D;
        const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 16 * g));
        const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 64 + 16 * g));
        kfrag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qfrag, kfrag, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                     0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[u][r] = slot >= 0 ? d[r] * s2scale : -INFINITY;
    }

    // online softmax per head (lane group g, entry r): tile maximum over the
    // 64 tokens = 4 subtiles x the 16 lanes of the row
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mt = fmaxf(fmaxf(s[0][r], s[1][r]), fmaxf(s[2][r], s[3][r]));
      mt = row16_max_f(mt);
      const float mn = fmaxf(m_run[r], mt);
      const float ms = mn == -INFINITY ? 0.f : mn;  // no token yet: keep exp2 finite
      alpha[r] = __builtin_amdgcn_exp2f(m_run[r] - ms);
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[u][r] = __builtin_amdgcn_exp2f(s[u][r] - ms);
        psum += s[u][r];
      }
      l_run[r] = l_run[r] * alpha[r] + row16_sum_f(psum);
      m_run[r] = mn;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r < G) ptile[wave][16 * u + c16][4 * g + r] = s[u][r];
    wave_lds_sync();

    // PV: lane = (token phase j = g, value chunk c16); rescale, then 16 tokens
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h)  // head h's factor lives in lane group h/4, entry h%4
      al[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[h & 3]), 16 * (h >> 2)));
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const int tl = g + 4 * k;
      const int32_t slot = slot_tile[wave][tl];
      if (slot >= 0) {
        const u32x2 vw = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(v_cache + (int64_t)slot * row_bytes + gk * D + 8 * c16));
        float v[8];
        const f32x2 v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw.x, false);
        const f32x2 v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw.x, true);
        const f32x2 v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw.y, false);
        const f32x2 v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw.y, true);
        v[0] = v0.x; v[1] = v0.y; v[2] = v1.x; v[3] = v1.y;
        v[4] = v2.x; v[5] = v2.y; v[6] = v3.x; v[7] = v3.y;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = ptile[wave][tl][h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(p, v[e], acc[h][e]);
        }
      }
    }
    wave_lds_sync();  // the next tile overwrites slot_tile and ptile
  }

  // this wave's totals: sum the four token phases (lanes c16, +16, +32, +48)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16);
      acc[h][e] += __shfl_xor(acc[h][e], 32);
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc_w[wave][h][8 * c16 + e] = acc[h][e];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run[h & 3]), 16 * (h >> 2)));
    const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_run[h & 3]), 16 * (h >> 2)));
    if (lane == 0) {
      m_w[wave][h] = mh;
      l_w[wave][h] = lh;
    }
  }
  __syncthreads();

  // merge the four waves: thread (h, chunk) for h < G, 16 chunks of 8 values
  if (tid < G * 16) {
    const int h = tid >> 4, ch = tid & 15;
    float m = m_w[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = fmaxf(m, m_w[w][h]);
    const float ms = m == -INFINITY ? 0.f : m;
    float wsc[4], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wsc[w] = __builtin_amdgcn_exp2f(m_w[w][h] - ms);
      lsum += l_w[w][h] * wsc[w];
    }
    const float inv = lsum > 0.f ? vs / lsum : 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o0 = __builtin_fmaf(acc_w[w][h][8 * ch + e], wsc[w], o0);
        o1 = __builtin_fmaf(acc_w[w][h][8 * ch + e + 1], wsc[w], o1);
      }
      packed[e / 2] = (uint32_t)to_bf16_bits(o0 * inv) | ((uint32_t)to_bf16_bits(o1 * inv) << 16);
    }
    *reinterpret_cast<uint4*>(out + b * ldo + (gk * G + h) * D + 8 * ch) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status fp8blk_decode_attention(const uint16_t* q, int64_t ldq, int64_t B, int64_t Hq, int64_t Hkv,
                                                 int64_t D, const uint8_t* k_cache, const uint8_t* v_cache,
                                                 int64_t num_slots, const int32_t* block_table, int64_t max_blocks,
                                                 int64_t block_size, const int32_t* context_lens,
                                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                                 float sm_scale, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || num_slots < 0 || max_blocks < 1 || block_size < 1 ||
      !(sm_scale == sm_scale) || ldq < Hq * D || ldo < Hq * D)
    return FP8BLK_ERR_INVALID_ARG;
  const int64_t G = Hq / Hkv;
  if (D != kHeadDim || Hq % Hkv || (G != 1 && G != 2 && G != 4 && G != 8) || ldq % 8 || ldo % 8)
    return FP8BLK_ERR_SHAPE;
  if (B == 0) return FP8BLK_OK;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !q_scale || !k_scale || !v_scale || !out)
    return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(q_scale, 4) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return FP8BLK_ERR_ALIGNMENT;
  if (B * Hkv > INT32_MAX || num_slots > INT32_MAX) return FP8BLK_ERR_SHAPE;
  const dim3 grid((uint32_t)(B * Hkv));
#define FP8BLK_ATTN_LAUNCH(GV)                                                                                     \
  hipLaunchKernelGGL(decode_attention_kernel<GV>, grid, dim3(256), 0, stream, q, ldq, Hkv, k_cache, v_cache,         \
                     num_slots, block_table, max_blocks, block_size, context_lens, q_scale, k_scale, v_scale,       \
                     sm_scale, out, ldo)
  switch (G) {
    case 1: FP8BLK_ATTN_LAUNCH(1); break;
    case 2: FP8BLK_ATTN_LAUNCH(2); break;
    case 4: FP8BLK_ATTN_LAUNCH(4); break;
    default: FP8BLK_ATTN_LAUNCH(8); break;
  }
#undef FP8BLK_ATTN_LAUNCH
  return launch_status();
}
