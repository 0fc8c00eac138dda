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
// each probability carried as an fp16 head plus an fp16 remainder (22
// significant bits); bf16 output.
//
// Work decomposition: a workgroup of four waves takes one (sequence, KV head)
// and either the whole context (direct mode: it writes the bf16 output) or
// one chunk of it (split mode: it writes fp32 partials -- running maximum,
// sum and unnormalized output per head -- to the workspace, and a second
// kernel merges the chunks of each head). Splitting keeps the chip full when
// there are few (sequence, KV head) pairs.
// Within a workgroup the waves take interleaved 64-token tiles and keep
// their own online-softmax state, merged through LDS. Per tile:
//   * the 64 tokens' cache rows come from the block table (one per lane;
//     out-of-range tokens, blocks or slots are masked and read a zero row,
//     so every load is unconditional and all of them are issued together).
//     The caches are head-major pages [blocks][Hkv][block_size][D]: a
//     workgroup's rows of one page are one contiguous block_size x 128-byte
//     run;
//   * S^T = K Q^T on the fp16 matrix cores, four v_mfma_f32_16x16x32_f16
//     steps of 32 head dims per 16 tokens, source 0 = 16 K rows loaded
//     straight from the cache, source 1 = the group's Q rows (heads, padded
//     to 16 with zeros), both converted from E4M3 to fp16 in registers
//     (exact). The FP8 instruction would take the whole head in one step,
//     but it sums each group of 8 products in a window 13 bits below the
//     group's largest product, which with a large score scale moves the
//     scores by whole units and the softmax with them; the fp16 instruction
//     adds exact products in fp32. Lane (c, g) then holds head c's scores of
//     16 of the tile's tokens, and its three partner lanes (same c) the other
//     48: a head's maximum is the lane's own plus two cross-lane steps;
//   * O^T += V^T P^T on the same instruction, two 32-token steps per 16 head
//     dims: the probabilities are already where source 1 wants them (no LDS
//     round trip), the V rows go through a wave-private LDS tile and come
//     back transposed (ds_read_b64_tr_b8) as source 0. The matrix cores take
//     the G x 128 x 64 products per tile that the vector ALUs were the bound
//     on, padded to 16 heads.
// The cache reads are the bound (K and V, 256 bytes per token and KV head).
#include "common.h"
#include "quant_common.h"

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kHeadDim = 128;
constexpr float kLog2eAttn = 1.44269504088896341f;
constexpr float kSlackAttn = 8.0f;  // log2 of the largest unnormalised probability

// Byte offset of 16-byte chunk c of V row t in a wave's 64 x 128-byte tile.
// Rows t and t ^ 1 trade places when bit 4 of t is set, and chunk c sits at
// c ^ ((t >> 1) & 7): the row writes (rows 8j + k of the eight lane groups
// j at once, 16 bytes per lane) and the transposing reads (32 token rows,
// one chunk each) then spread over all the banks.
__device__ __forceinline__ int vswz(int t, int c) {
  return ((t ^ ((t >> 4) & 1)) << 7) + ((c ^ ((t >> 1) & 7)) << 4);
}

// what a masked token reads in place of its K and V rows
__device__ const uint32_t kZeroRow[kHeadDim / 4] = {};

// A cache row pointer marked as global memory, so that its loads are global
// (not flat) loads and do not hold up the LDS waits of the loop.
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
__device__ __forceinline__ gbytes as_global(const uint8_t* p) { return (gbytes)p; }

// fp32 maximum / sum over the four lanes c, c+16, c+32, c+48, by the
// lane-swap instructions (no LDS round trip): with both operands v,
// v_permlane16_swap returns (v[l], v[l+16]) in even 16-lane rows and
// (v[l-16], v[l]) in odd ones, v_permlane32_swap the same for halves (lane
// layout checked on the GPU), so combining the two results gives each lane
// the pair's maximum or sum, in the same order in both lanes of the pair.
__device__ __forceinline__ float cross4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float cross4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Make this wave's LDS writes visible to its own later LDS reads by other
// lanes (LDS operations of one wave complete in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Race-detection build (-DFP8BLK_DEBUG_BARRIERS=1): before each rewrite of
// an LDS region this wave has just read (the row exchange, the V tile) the
// wave also waits for all of its memory operations, so no rewrite can pass
// a read still in flight; the arithmetic is unchanged and the outputs must
// equal the normal build's bit for bit.
#ifndef FP8BLK_DEBUG_BARRIERS
#define FP8BLK_DEBUG_BARRIERS 0
#endif
__device__ __forceinline__ void debug_wave_sync() {
  if constexpr (FP8BLK_DEBUG_BARRIERS != 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
}

template <int G, bool SPLIT>  // G = query heads per KV head: 1, 2, 4 or 8
__global__ __launch_bounds__(256) void decode_attention_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, int64_t Hkv, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, int64_t num_slots, const int32_t* __restrict__ block_table,
    int64_t max_blocks, int64_t block_size, const int32_t* __restrict__ context_lens,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    float sm_scale, uint16_t* __restrict__ out, int64_t ldo, int64_t splits, int64_t chunk,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int64_t nchunks) {
  constexpr int D = kHeadDim;
  __shared__ __attribute__((aligned(16))) uint32_t q8[G * D / 4];
  __shared__ __attribute__((aligned(16))) int32_t row_tile[4][64];
  __shared__ __attribute__((aligned(1024))) uint8_t vlds[4][64 * kHeadDim];  // each wave's V rows of a tile
  __shared__ float m_w[4][G], l_w[4][G];
  __shared__ __attribute__((aligned(16))) float acc_w[4][G][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Block order: the KV heads of one chunk are consecutive blocks, spread
  // over the XCDs by the round-robin dispatch. With head-major pages this
  // and an XCD-aware order (all heads of a chunk on one XCD) measured the
  // same; with token-major slots the XCD-aware order was 9-10% faster.
  const int64_t gk = blockIdx.x % Hkv, cidx = blockIdx.x / Hkv;  // chunk cidx = b * splits + s
  if (cidx >= nchunks) return;
  const int64_t b = cidx / splits, sidx = cidx % splits;
  const int64_t wg = (b * Hkv + gk) * splits + sidx;          // partial index (split mode)
  const int64_t L = context_lens[b] > 0 ? context_lens[b] : 0;
  const int64_t c0 = SPLIT ? sidx * chunk : 0;  // this workgroup's tokens [c0, c1)
  const int64_t c1 = SPLIT ? (L < c0 + chunk ? L : c0 + chunk) : L;
  if (SPLIT && c0 >= L) return;  // an empty chunk (uniform over the workgroup); the merge skips it
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
  // fp16 Q for the four score steps: step s of lane group g covers head dims
  // 16g + 8s .. +7 (s < 2) and 64 + 16g + 8(s-2) .. +7, bytes 8s .. 8s+7 of
  // the fragment above; the K fragments take the same bytes of their rows
  f16x8 qh[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) qh[st] = e4m3x8_to_f16((uint32_t)qfrag[2 * st], (uint32_t)qfrag[2 * st + 1]);
  const float s2scale = qs * ks * sm_scale * kLog2eAttn;  // scores in the log2 domain
  const uint8_t* const zero = reinterpret_cast<const uint8_t*>(kZeroRow);
  // opaque to the compiler, so that the FMAs splitting the probabilities
  // below stay FMAs instead of being folded into subtractions
  float one = 1.0f;
  asm volatile("" : "+s"(one));

  // running state of this lane's head: lane (c16, g) with c16 < G works for
  // head c16 of the group; the four lanes of a head (c16, c16+16, c16+32,
  // c16+48) hold the same reference maximum and their own shares of the sum
  const bool head_lane = c16 < G;
  float m_run = -INFINITY, l_run = 0.f;
  v4f acc[8];  // O^T tiles [dt]: lane (c16, g) holds O[head c16][dim 16dt + 4g + r]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  uint8_t* const vtile = vlds[wave];  // this wave's V rows of the tile (64 x 128 bytes)

  // Software pipeline over this wave's tiles (tokens t0..t0+63, t0 advancing
  // by 256): while tile i is computed, the K and V rows of tile i+1 and the
  // block-table entries of tile i+2 are in flight. Loads past the last tile
  // read the zero row (their tokens are masked), so every load is
  // unconditional and the wait counts are the same in every iteration.
  const uint32_t bs32 = (uint32_t)block_size;
  const int32_t* const table_row = block_table + b * max_blocks;
  // token t's block index (t < 2^31): a shift for a power-of-two block size
  // (uniform branch), else a division
  const int bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctzll((uint64_t)block_size) : -1;
  const uint32_t mb32 = (uint32_t)max_blocks;  // < 2^31, checked on the host
  auto block_of = [&](int64_t t) {
    uint32_t bi;
    if (bs_shift >= 0)
      bi = (uint32_t)t >> bs_shift;
    else
      bi = (uint32_t)t / bs32;
    return bi;
  };
  auto table_entry = [&](int64_t t) {  // the block id of token t (block index clamped)
    const uint32_t bi = block_of(t);
    return table_row[bi < mb32 ? bi : mb32 - 1];
  };
  // The cache row of token t for this KV head: head-major pages
  // [num_slots / block_size][Hkv][block_size][D], so row (blk*Hkv + gk) *
  // block_size + offset, in units of D bytes, computed in 32 bits (below
  // num_slots * Hkv < 2^31, checked on the host, for every live token;
  // masked tokens' values are discarded); -1 for a masked token.
  auto token_row = [&](int64_t t, int32_t blk) {
    const uint32_t bi = block_of(t);
    const uint32_t off = (uint32_t)t - bi * bs32;
    const bool live = t < c1 && bi < mb32 && blk >= 0 && (int64_t)blk * block_size + off < num_slots;
    return live ? (int32_t)(((uint32_t)blk * (uint32_t)Hkv + (uint32_t)gk) * bs32 + off) : -1;
  };
  const int g8 = lane >> 3, c8 = lane & 7;
  int32_t krow[4], vrow[8];
  auto read_rows = [&](int32_t row) {  // exchange the tile's cache rows through LDS
    debug_wave_sync();
    row_tile[wave][lane] = row;
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < 4; ++u) krow[u] = row_tile[wave][16 * u + c16];
#pragma unroll
    for (int k = 0; k < 8; k += 4) {
      const int4 v4 = *reinterpret_cast<const int4*>(&row_tile[wave][8 * g8 + k]);
      vrow[k] = v4.x;
      vrow[k + 1] = v4.y;
      vrow[k + 2] = v4.z;
      vrow[k + 3] = v4.w;
    }
  };
  // K rows of tokens 16u + c16 (bytes 16g..+15 and 64+16g..+15), kept in the
  // cache hierarchy: the two halves of each row are read by two loads
  u32x4 klo[4], khi[4];
  auto row_or_zero = [&](const uint8_t* base, int32_t row) {  // branch-free
    const uint8_t* p = base + ((uint64_t)(uint32_t)(row > 0 ? row : 0) << 7);  // D = 128 bytes per row
    return as_global(row >= 0 ? p : zero);
  };
  auto load_k = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const gbytes kr = row_or_zero(k_cache, krow[u]);
      klo[u] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(kr + 16 * g);
      khi[u] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(kr + 64 + 16 * g);
    }
  };
  // V rows of tokens 8 g8 + k, bytes 16 c8..+15 (eight lanes per row): each
  // row is read once (streamed)
  auto load_v = [&](int k) {
    const gbytes vr = row_or_zero(v_cache, vrow[k]);
    return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(vr + 16 * c8));
  };

  int64_t t0 = c0 + (int64_t)wave * 64;
  if (t0 < c1) {  // uniform over the wave
    int32_t blk = table_entry(t0 + lane);
    const int32_t row0 = token_row(t0 + lane, blk);
    blk = table_entry(t0 + 256 + lane);  // tile i+1's entries
    read_rows(row0);
    load_k();
    u32x4 vw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) vw[k] = load_v(k);

    for (;;) {
      // S^T = K Q^T (source 0 = the 16 K rows of a subtile, source 1 = the
      // heads): lane (c16, g) gets s[u][r], the score of token 16u + 4g + r
      // for head c16 (log2 domain); the rows of those tokens tell the masked
      float s[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4f d = v4f{0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(klo[u].x, klo[u].y), qh[0], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(klo[u].z, klo[u].w), qh[1], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(khi[u].x, khi[u].y), qh[2], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(khi[u].z, khi[u].w), qh[3], d, 0, 0, 0);
        const int4 rows = *reinterpret_cast<const int4*>(&row_tile[wave][16 * u + 4 * g]);
        s[u][0] = rows.x >= 0 ? d[0] * s2scale : -INFINITY;
        s[u][1] = rows.y >= 0 ? d[1] * s2scale : -INFINITY;
        s[u][2] = rows.z >= 0 ? d[2] * s2scale : -INFINITY;
        s[u][3] = rows.w >= 0 ? d[3] * s2scale : -INFINITY;
      }
      // the scheduling barriers keep each stage's loads after the last use
      // of the registers they overwrite (one register set per stage)
      __builtin_amdgcn_sched_barrier(0);

      // next tile: its rows (entries loaded one tile ago), the entries of
      // the tile after it, its K rows
      const int64_t tn = t0 + 256;
      const int32_t row_n = token_row(tn + lane, blk);
      blk = table_entry(tn + 256 + lane);
      read_rows(row_n);
      load_k();
      __builtin_amdgcn_sched_barrier(0);

      // online softmax of this lane's head over the tile (16 scores in the
      // lane, the other 48 in its three partner lanes). The reference
      // maximum moves only when the tile's exceeds it by more than kSlack
      // (log2 units): probabilities stay at most 2^kSlack, and the
      // accumulators are rescaled only then.
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u) mt = fmaxf(mt, fmaxf(fmaxf(s[u][0], s[u][1]), fmaxf(s[u][2], s[u][3])));
      mt = cross4_max(mt);
      const float mn = mt > m_run + kSlackAttn ? mt : m_run;
      const float ms = mn == -INFINITY ? 0.f : mn;  // no token yet: keep exp2 finite
      const float alpha = __builtin_amdgcn_exp2f(m_run - ms);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[u][r] = __builtin_amdgcn_exp2f(s[u][r] - ms);
          ps += s[u][r];
        }
      l_run = l_run * alpha + ps;
      m_run = mn;
      if (__builtin_amdgcn_ballot_w64(head_lane && alpha != 1.0f) != 0) {  // uniform
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
      }

      // this tile's V rows into the wave's LDS rows (16-byte chunk c of row t
      // at chunk c ^ key(t)), then the next tile's V rows into the registers
#pragma unroll
      for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(vtile + vswz(8 * g8 + k, c8)) = vw[k];
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < 8; ++k) vw[k] = load_v(k);

      // O^T += V^T P^T over two 32-token chunks on the fp16 matrix cores.
      // Contraction slot (g, j) of chunk c is token 32c + 16(j/4) + 4g + j%4,
      // so source 1 (P^T: the probabilities of head c16) is this lane's
      // s[2c + j/4][j%4], split into an fp16 head and remainder (the
      // remainder's difference exact in the FMA). Source 0 (V^T) comes from
      // the transposing read ds_read_b64_tr_b8: in a 16-lane group, lanes 2j
      // and 2j+1 read the two 8-byte halves of token slot j's 16 values of the
      // dim tile, and lane i receives value i of each of the 8 slots;
      // converted to fp16 (exact for E4M3).
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f16x8 ph, pl;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float p0 = s[2 * c + j / 4][j % 4], p1 = s[2 * c + j / 4][j % 4 + 1];
          const f16x2 h = __builtin_convertvector(f32x2{p0, p1}, f16x2);
          const f16x2 l = __builtin_convertvector(
              f32x2{__builtin_fmaf(-(float)h[0], one, p0), __builtin_fmaf(-(float)h[1], one, p1)}, f16x2);
          ph[j] = h[0];
          ph[j + 1] = h[1];
          pl[j] = l[0];
          pl[j + 1] = l[1];
        }
        const int jj = c16 >> 1;
        const int tok = 32 * c + 16 * (jj >> 2) + 4 * g + (jj & 3);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vtile + vswz(tok, dt) + 8 * (c16 & 1)));
          const f16x8 vf = e4m3x8_to_f16((uint32_t)raw[0], (uint32_t)raw[1]);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[dt], 0, 0, 0);
        }
      }
      debug_wave_sync();
      t0 = tn;
      if (t0 >= c1) break;
    }
  }

  // this wave's totals: the four lanes of a head add their shares of the sum
  l_run = cross4_sum(l_run);
  if (head_lane) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_w[wave][c16][16 * dt + 4 * g + r] = acc[dt][r];
    if (g == 0) {
      m_w[wave][c16] = m_run;
      l_w[wave][c16] = l_run;
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
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[e] = __builtin_fmaf(acc_w[w][h][8 * ch + e], wsc[w], o[e]);
    }
    if (SPLIT) {  // partial of this chunk: unnormalized output, maximum, sum
      float4* dst = reinterpret_cast<float4*>(ws_acc + (wg * G + h) * D + 8 * ch);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (ch == 0) *reinterpret_cast<float2*>(ws_ml + (wg * G + h) * 2) = make_float2(m, lsum);
    } else {
      const float inv = lsum > 0.f ? vs / lsum : 0.f;
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        packed[e / 2] = (uint32_t)to_bf16_bits(o[e] * inv) | ((uint32_t)to_bf16_bits(o[e + 1] * inv) << 16);
      *reinterpret_cast<uint4*>(out + b * ldo + (gk * G + h) * D + 8 * ch) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
  }
}

// Merge of the chunk partials of one (sequence, query head): one wave, two
// output values per lane.
__global__ __launch_bounds__(64) void decode_attention_combine_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, int64_t splits, int64_t chunk, int64_t Hq,
    int64_t Hkv, const int32_t* __restrict__ context_lens, const float* __restrict__ v_scale,
    uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int64_t G = Hq / Hkv, gk = h / G, hh = h % G;
  const int64_t L = context_lens[b] > 0 ? context_lens[b] : 0;
  const int64_t full = (L + chunk - 1) / chunk;
  const int64_t n = full < splits ? full : splits;
  const int64_t p0 = (b * Hkv + gk) * splits;  // partial index of chunk 0
  float m = -INFINITY;
  for (int64_t s = 0; s < n; ++s) m = fmaxf(m, ws_ml[((p0 + s) * G + hh) * 2]);
  const float ms = m == -INFINITY ? 0.f : m;
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t s = 0; s < n; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + ((p0 + s) * G + hh) * 2);
    const float w = __builtin_amdgcn_exp2f(ml.x - ms);
    const float2 a = *reinterpret_cast<const float2*>(ws_acc + ((p0 + s) * G + hh) * kHeadDim + 2 * lane);
    lsum = __builtin_fmaf(ml.y, w, lsum);
    o0 = __builtin_fmaf(a.x, w, o0);
    o1 = __builtin_fmaf(a.y, w, o1);
  }
  const float inv = lsum > 0.f ? *v_scale / lsum : 0.f;
  *reinterpret_cast<uint32_t*>(out + b * ldo + h * kHeadDim + 2 * lane) =
      (uint32_t)to_bf16_bits(o0 * inv) | ((uint32_t)to_bf16_bits(o1 * inv) << 16);
}

constexpr int64_t kSplitUnit = 256;  // chunk sizes are multiples of one tile per wave
constexpr int64_t kFillWGs = 512;    // automatic split: about two workgroups per CU
constexpr int64_t kMinChunk = 2048;  // automatic split: the shortest chunk (a multiple of kSplitUnit)

// Tokens per chunk for the split path: the caller's, else (automatic) the
// whole addressable context -- no split -- when there are at least 512
// (sequence, KV head) pairs, otherwise chunks sized so that about 512
// workgroups run, but at least 2048 tokens long (measured: two workgroups
// per CU keep a long context's tiles coming faster than one, and chunks
// below 2048 tokens lose to the pipeline start and the merge).
int64_t split_chunk(int64_t B, int64_t Hkv, int64_t Lcap, int64_t split_tokens) {
  if (split_tokens > 0) return split_tokens;
  const int64_t pairs = B * Hkv;
  if (pairs >= kFillWGs) return ((Lcap + kSplitUnit - 1) / kSplitUnit) * kSplitUnit;
  const int64_t splits = (kFillWGs + pairs - 1) / pairs;
  const int64_t c = (Lcap + splits - 1) / splits;
  const int64_t chunk = ((c + kSplitUnit - 1) / kSplitUnit) * kSplitUnit;
  return chunk > kMinChunk ? chunk : kMinChunk;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

namespace {

// Shape checks shared by the workspace query and the call.
fp8blk_status attention_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t max_blocks,
                              int64_t block_size, int64_t split_tokens) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || max_blocks < 1 || block_size < 1 || split_tokens < 0)
    return FP8BLK_ERR_INVALID_ARG;
  const int64_t G = Hq / Hkv;
  if (D != kHeadDim || Hq % Hkv || (G != 1 && G != 2 && G != 4 && G != 8) || split_tokens % kSplitUnit ||
      max_blocks > INT32_MAX || block_size > INT32_MAX || B * Hq > INT32_MAX)
    return FP8BLK_ERR_SHAPE;
  return FP8BLK_OK;
}

// Chunks per (sequence, KV head) for the split path (1: direct).
int64_t attention_splits(int64_t B, int64_t Hkv, int64_t max_blocks, int64_t block_size, int64_t split_tokens,
                         int64_t* chunk) {
  const int64_t cap = max_blocks * block_size;  // tokens the block table can address
  const int64_t lcap = cap < INT32_MAX ? cap : INT32_MAX;
  *chunk = split_chunk(B, Hkv, lcap, split_tokens);
  return (lcap + *chunk - 1) / *chunk;
}

}  // namespace

extern "C" size_t fp8blk_decode_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                                          int64_t max_blocks, int64_t block_size,
                                                          int64_t split_tokens) {
  if (attention_shape(B, Hq, Hkv, D, max_blocks, block_size, split_tokens) != FP8BLK_OK || B == 0) return 0;
  int64_t chunk;
  const int64_t splits = attention_splits(B, Hkv, max_blocks, block_size, split_tokens, &chunk);
  if (splits <= 1) return 0;
  return (size_t)(B * Hq * splits) * (kHeadDim + 2) * sizeof(float);
}


extern "C" fp8blk_status fp8blk_decode_attention(const uint16_t* q, int64_t ldq, int64_t B, int64_t Hq, int64_t Hkv,
                                                 int64_t D, const uint8_t* k_cache, const uint8_t* v_cache,
                                                 int64_t num_slots, const int32_t* block_table, int64_t max_blocks,
                                                 int64_t block_size, const int32_t* context_lens,
                                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                                 float sm_scale, uint16_t* out, int64_t ldo, int64_t split_tokens,
                                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fp8blk_status st = attention_shape(B, Hq, Hkv, D, max_blocks, block_size, split_tokens);
  if (st != FP8BLK_OK) return st;
  if (num_slots < 0 || !(sm_scale == sm_scale) || ldq < Hq * D || ldo < Hq * D) return FP8BLK_ERR_INVALID_ARG;
  if (ldq % 8 || ldo % 8 || num_slots % block_size || num_slots > INT32_MAX / Hkv) return FP8BLK_ERR_SHAPE;
  if (B == 0) return FP8BLK_OK;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !q_scale || !k_scale || !v_scale || !out)
    return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(q_scale, 4) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4) || !aligned(workspace, 16))
    return FP8BLK_ERR_ALIGNMENT;
  const int64_t G = Hq / Hkv;
  int64_t chunk = 0, splits = 1;
  float *ws_acc = nullptr, *ws_ml = nullptr;
  if (workspace) {
    splits = attention_splits(B, Hkv, max_blocks, block_size, split_tokens, &chunk);
    if (splits > 1) {
      const size_t need = (size_t)(B * Hq * splits) * (kHeadDim + 2) * sizeof(float);
      if (workspace_bytes < need) return FP8BLK_ERR_INVALID_ARG;
      ws_acc = static_cast<float*>(workspace);
      ws_ml = ws_acc + B * Hq * splits * kHeadDim;
    }
  }
  const bool split = splits > 1;
  const int64_t nchunks = B * splits;
  const int64_t blocks = nchunks * Hkv;
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  const dim3 grid((uint32_t)blocks);
#define FP8BLK_ATTN_LAUNCH(GV, SV)                                                                                 \
  hipLaunchKernelGGL((decode_attention_kernel<GV, SV>), grid, dim3(256), 0, stream, q, ldq, Hkv, k_cache, v_cache,  \
                     num_slots, block_table, max_blocks, block_size, context_lens, q_scale, k_scale, v_scale,       \
                     sm_scale, out, ldo, splits, chunk, ws_acc, ws_ml, nchunks)
#define FP8BLK_ATTN_G(SV)                  \
  switch (G) {                             \
    case 1: FP8BLK_ATTN_LAUNCH(1, SV); break; \
    case 2: FP8BLK_ATTN_LAUNCH(2, SV); break; \
    case 4: FP8BLK_ATTN_LAUNCH(4, SV); break; \
    default: FP8BLK_ATTN_LAUNCH(8, SV); break; \
  }
  if (split) {
    FP8BLK_ATTN_G(true)
    st = launch_status();
    if (st != FP8BLK_OK) return st;
    hipLaunchKernelGGL(decode_attention_combine_kernel, dim3((uint32_t)(B * Hq)), dim3(64), 0, stream, ws_acc,
                       ws_ml, splits, chunk, Hq, Hkv, context_lens, v_scale, out, ldo);
  } else {
    FP8BLK_ATTN_G(false)
  }
#undef FP8BLK_ATTN_G
#undef FP8BLK_ATTN_LAUNCH
  return launch_status();
}
