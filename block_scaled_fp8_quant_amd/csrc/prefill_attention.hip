// FP8 prefill attention over the paged FP8 KV cache, for gfx950.
//
// Method (upppp.jp NeMo RL FP8 article, «KVキャッシュとAttentionにも拡張»;
// greentreeone.com article, «Реальные прирост производительности»): attention
// runs in FP8 over the FP8 KV cache with the recalibrated Q/K/V scales. The
// prefill step: a sequence's n new tokens are the last n of its L cached
// tokens (their K and V already written by the cache write), and new token i,
// at position p = L - n + i, attends causally to cached tokens 0..p:
//     s[t] = (q8 . k8[t]) * q_scale * k_scale * sm_scale,   t <= p
//     out  = bf16( sum_t softmax(s)[t] * v8[t] * v_scale )
// with q8 the per-tensor E4M3 quantization of the query (as the decode step).
//
// Work decomposition: a workgroup of four waves takes one (sequence, KV
// head, block of 128/G consecutive new tokens); its 128 rows are the (token,
// query head) pairs of that block, row = token * G + head, 32 per wave. The
// KV loop walks 64-token tiles up to the block's last position; each tile's
// K and V rows (one cache row of 128 bytes per token) are loaded by the
// whole workgroup into registers while the previous tile is computed, then
// written to LDS (two stages, one barrier per tile). Per tile and wave:
//   * S^T = K Q^T on the fp16 matrix cores (v_mfma_f32_16x16x32_f16, four
//     steps of 32 head dims), source 0 = 16 K rows (tokens), source 1 = 16
//     query rows, with the E4M3 values of K and of the quantized query in
//     fp16 (exact). The FP8 instruction would take the whole head in one
//     step, but it sums each group of 8 products in a window 13 bits below
//     the group's largest product, which with a large score scale moves the
//     scores by whole units and the softmax with them; the fp16 instruction
//     adds exact products in fp32. Lane (c, g) then holds the scores of
//     tokens 16u + 4g + r (r < 4) for query row c, so a row's maximum is an
//     in-lane maximum and two cross-lane steps;
//   * online softmax in the log2 domain (v_exp_f32), fp32;
//   * O^T += V^T P^T on the fp16 matrix cores (v_mfma_f32_16x16x32_f16),
//     source 1 = the probabilities straight from the score registers (the
//     token order of the contraction is chosen to match the score layout),
//     each probability split into an fp16 head and an fp16 remainder (two
//     MFMAs, ~2^-22 relative: the probabilities stay unquantized to within
//     fp32 accuracy), source 0 = V^T: the transpose of the tile's V rows read
//     from LDS with ds_read_b64_tr_b16. V is converted to fp16 (exact for
//     E4M3) once, by the thread that stores it to LDS, not by every wave.
// K and V are converted to fp16 once, by the thread that stores a row to
// LDS. Rows are 256 bytes padded to 288. A K fragment read (16 token rows,
// the four lane groups on consecutive 16-byte chunks of a row) then runs at
// about 230 bytes per clock per CU against 113 with 272-byte rows and the
// chunks of a group paired (an LDS probe of the exact patterns); for the
// transposing V reads 8 consecutive tokens fall in 8 different 32-byte bank
// groups. Every read offset stays an immediate.
#include "common.h"
#include "quant_common.h"

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kD = 128;         // head size
constexpr int kTile = 64;       // tokens per KV tile
constexpr int kRows = 128;      // score rows per workgroup: (token, head) pairs
constexpr int kKRow = 2 * kD + 32;  // bytes per fp16 K row in LDS (256 + 32 of padding)
constexpr int kVRow = 2 * kD + 32;  // bytes per fp16 V row in LDS (256 + 32 of padding)
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kSlack = 8.0f;  // log2 of the largest unnormalised probability

// A cache row pointer marked as global memory (global, not flat, loads).
typedef const __attribute__((address_space(1))) uint8_t* gbytes;

// what a masked token reads in place of its K and V rows
__device__ const uint32_t kZeroRow[kD / 4] = {};


// Race-detection build (-DFP8BLK_DEBUG_BARRIERS=1): extra workgroup
// barriers (after every wave's loads have landed) around each stage's use,
// same arithmetic, so the outputs must equal the normal build's bit for bit.
#ifndef FP8BLK_DEBUG_BARRIERS
#define FP8BLK_DEBUG_BARRIERS 0
#endif
__device__ __forceinline__ void debug_stage_sync() {
  if constexpr (FP8BLK_DEBUG_BARRIERS != 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

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

template <int G>  // query heads per KV head: 1, 2, 4 or 8
__global__ __launch_bounds__(256, 2) void prefill_attention_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, int64_t total_q, int64_t B, int64_t Hkv,
    const int32_t* __restrict__ cu_seqlens_q, int64_t nqb, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, int64_t num_slots, const int32_t* __restrict__ block_table,
    int64_t max_blocks, int64_t block_size, const int32_t* __restrict__ context_lens,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    float sm_scale, uint16_t* __restrict__ out, int64_t ldo) {
  constexpr int BQ = kRows / G;  // new tokens per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t kt[2][kTile * kKRow];
  __shared__ __attribute__((aligned(1024))) uint8_t vt[2][kTile * kVRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  // longest blocks first: the last token blocks attend the most tokens
  const int64_t pairs = B * Hkv;
  const int64_t bh = blockIdx.x % pairs, qblk = nqb - 1 - (int64_t)blockIdx.x / pairs;
  const int64_t b = bh / Hkv, gk = bh % Hkv;
  const int64_t row0 = cu_seqlens_q[b];
  int64_t n = (int64_t)cu_seqlens_q[b + 1] - row0;  // new tokens
  const int64_t L = context_lens[b] > 0 ? context_lens[b] : 0;
  const int64_t i0 = qblk * BQ;
  if (n <= i0 || row0 < 0) return;  // uniform: no new token in this block
  if (n > total_q - row0) n = total_q - row0;  // rows past q/out (offsets that break their contract)
  if (n <= i0) return;
  // positions of the block's first and last tokens; tiles up to the last
  const int64_t p_last = L - n + (i0 + BQ < n ? i0 + BQ : n) - 1;
  const int64_t t_end = p_last + 1 < L ? p_last + 1 : L;  // tokens [0, t_end) are needed
  const int ntiles = t_end > 0 ? (int)((t_end + kTile - 1) / kTile) : 0;
  // tiles before the block's first position need no causal mask (every token
  // of them is at most that position, hence below L)
  const int64_t p_first = L - n + i0;
  const float qs = *q_scale, ks = *k_scale, vs = *v_scale;

  // this lane's two score rows (one per 16-row tile qt): row 32*wave + 16qt + c16
  int64_t pos[2];
  bool active[2];
  int64_t orow[2];
  int ohead[2];
  v8i qfrag[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int r = 32 * wave + 16 * qt + c16;
    const int64_t i = i0 + r / G;
    active[qt] = i < n;
    pos[qt] = L - n + i;
    orow[qt] = row0 + i;
    ohead[qt] = (int)(gk * G + r % G);
    // source 1 fragment: query row r, head dims 32s + 8g .. +7 for the four
    // score steps s -> E4M3
    qfrag[qt] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if (active[qt]) {
      const uint16_t* src = q + orow[qt] * ldq + (int64_t)ohead[qt] * kD + 8 * g;
      const uint4 lo0 = *reinterpret_cast<const uint4*>(src);
      const uint4 lo1 = *reinterpret_cast<const uint4*>(src + 32);
      const uint4 hi0 = *reinterpret_cast<const uint4*>(src + 64);
      const uint4 hi1 = *reinterpret_cast<const uint4*>(src + 96);
      const bool fast = qs >= kCalibratedMinScale && qs <= kCalibratedMaxScale;
      const float inv = 1.0f / qs;
      const uint32_t w0[4] = {lo0.x, lo0.y, lo0.z, lo0.w}, w1[4] = {lo1.x, lo1.y, lo1.z, lo1.w};
      const uint32_t w2[4] = {hi0.x, hi0.y, hi0.z, hi0.w}, w3[4] = {hi1.x, hi1.y, hi1.z, hi1.w};
      const u32x2 c0 = encode8_calibrated(w0, qs, inv, fast), c1 = encode8_calibrated(w1, qs, inv, fast);
      const u32x2 c2 = encode8_calibrated(w2, qs, inv, fast), c3 = encode8_calibrated(w3, qs, inv, fast);
      qfrag[qt] = v8i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y, (int)c2.x, (int)c2.y, (int)c3.x, (int)c3.y};
    }
  }
  // the query codes in fp16 for the four score steps: step s of lane group g
  // covers head dims 32s + 8g .. +7 (bytes 8s .. 8s+7 of the fragment above);
  // K fragments use the same dims
  v8h qh[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int st = 0; st < 4; ++st) qh[qt][st] = e4m3x8_to_f16((uint32_t)qfrag[qt][2 * st], (uint32_t)qfrag[qt][2 * st + 1]);
  const float s2scale = qs * ks * sm_scale * kLog2e;
  // Tiles that need no causal mask keep the raw MFMA dot products and fold
  // the score scale into the exponent's argument (one FMA per score instead
  // of a multiply and a subtraction); with a positive scale the row maximum
  // of the raw products times the scale is the maximum of the scaled scores
  // exactly (rounding is monotonic). Other tiles scale each score and use
  // the same FMA with a multiplier of one, which is exact. `one` is opaque
  // to the compiler so that those FMAs, and the ones splitting the
  // probabilities below, stay FMAs (v_fma_mix for the fp16 operand) instead
  // of being folded into subtractions.
  const bool s2pos = s2scale > 0.f;
  float one = 1.0f;
  asm volatile("" : "+s"(one));

  // K/V tile loads: thread tid takes token tid/4 of the tile, bytes 32*(tid%4)..+31
  const int ltok = tid >> 2, lpart = tid & 3;
  const uint32_t bs32 = (uint32_t)block_size, mb32 = (uint32_t)max_blocks;  // both < 2^31 (host-checked)
  // a power-of-two block size divides by a shift (uniform branch)
  const int bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctzll((uint64_t)block_size) : -1;
  const int32_t* const table_row = block_table + b * max_blocks;
  // The cache row of token t (t < L + 64 < 2^31), -1 if masked. Branch-free:
  // the block index is clamped for the table read, and the row is computed
  // in 32 bits (below num_slots * Hkv < 2^31 for every live token; masked
  // tokens' values are discarded).
  auto cache_row = [&](int64_t t) -> int32_t {
    const uint32_t tu = (uint32_t)t;
    uint32_t bi;
    if (bs_shift >= 0)
      bi = tu >> bs_shift;
    else
      bi = tu / bs32;
    const int32_t blk = table_row[bi < mb32 ? bi : mb32 - 1];
    const uint32_t off = tu - bi * bs32;
    const bool live = t < t_end && bi < mb32 && blk >= 0 && (int64_t)blk * block_size + off < num_slots;
    return live ? (int32_t)(((uint32_t)blk * (uint32_t)Hkv + (uint32_t)gk) * bs32 + off) : -1;
  };
  // K/V rows: masked tokens read the zero row, so the loads are unconditional
  u32x4 kr[2], vr[2];
  const uint8_t* const zero_row = reinterpret_cast<const uint8_t*>(kZeroRow);
  auto load_tile = [&](int tile) {
    const int32_t row = cache_row((int64_t)tile * kTile + ltok);
    const gbytes kp = (gbytes)((row >= 0 ? k_cache + (int64_t)row * kD : zero_row) + 32 * lpart);
    const gbytes vp = (gbytes)((row >= 0 ? v_cache + (int64_t)row * kD : zero_row) + 32 * lpart);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kr[h] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(kp + 16 * h);
      vr[h] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(vp + 16 * h);
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // K and V dims 32*lpart + 16h .. +15 as fp16: bytes 64*lpart + 32h .. +31 of the row
      uint8_t* kdst = &kt[st][ltok * kKRow + 64 * lpart + 32 * h];
      *reinterpret_cast<v8h*>(kdst) = e4m3x8_to_f16(kr[h].x, kr[h].y);
      *reinterpret_cast<v8h*>(kdst + 16) = e4m3x8_to_f16(kr[h].z, kr[h].w);
      const v8h lo = e4m3x8_to_f16(vr[h].x, vr[h].y);
      const v8h hi = e4m3x8_to_f16(vr[h].z, vr[h].w);
      uint8_t* dst = &vt[st][ltok * kVRow + 64 * lpart + 32 * h];
      *reinterpret_cast<v8h*>(dst) = lo;
      *reinterpret_cast<v8h*>(dst + 16) = hi;
    }
  };

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  v4f acc[2][8];  // O^T tiles: [qt][dt], lane (c, g) holds O[row 16qt + c][dim 16dt + 4g + r]
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[qt][dt] = v4f{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    const int st = tile & 1;
    __syncthreads();  // stage st holds this tile; stage st^1 is no longer read
    debug_stage_sync();
    if (tile + 1 < ntiles) load_tile(tile + 1);  // in flight while this tile is computed
    const uint8_t* K = kt[st];
    const uint8_t* V = vt[st];
    const int64_t t0 = (int64_t)tile * kTile;

    // S^T: lane (c, g) gets s[u][qt][r] = score of token t0 + 16u + 4g + r, row 16qt + c
    float s[4][2][4];
    auto scores = [&](bool masked, bool raw) {
      // causal mask: token t0 + 16u + 4g + r is kept when t <= min(pos, L - 1),
      // i.e. 16u + r <= rel[qt] (tiles that need the mask lie within 64
      // tokens of the block's positions, so the differences are small ints)
      int rel[2] = {0, 0};
      if (masked) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) rel[qt] = (int)((pos[qt] < L - 1 ? pos[qt] : L - 1) - t0) - 4 * g;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint8_t* krow = K + (16 * u + c16) * kKRow + 16 * g;
        v4f d[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const v8h kfrag = *reinterpret_cast<const v8h*>(krow + 64 * st);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) d[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kfrag, qh[qt][st], d[qt], 0, 0, 0);
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[u][qt][r] = raw ? d[qt][r] : !masked || 16 * u + r <= rel[qt] ? d[qt][r] * s2scale : -INFINITY;
        }
      }
    };
    const bool unmasked = t0 + kTile - 1 <= p_first;  // uniform
    const bool raw = unmasked && s2pos;
    if (raw)
      scores(false, true);
    else if (unmasked)
      scores(false, false);
    else
      scores(true, false);
    const float mulv = raw ? s2scale : one;  // s * mulv is the scaled score
    // online softmax per row; p replaces s
    float alpha[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[u][qt][r]);
      mt = cross4_max(mt) * mulv;
      // The running maximum moves only when a tile's maximum exceeds it by
      // more than kSlack (log2 units): probabilities are then at most
      // 2^kSlack, well inside fp16 and fp32, and the accumulators are
      // rescaled only on such a jump instead of on nearly every tile (with
      // 16 rows per accumulator some row's maximum rises in most tiles).
      // The normalisation by the row sum at the end makes the result
      // independent of the reference point.
      const float mn = mt > m_run[qt] + kSlack ? mt : m_run[qt];
      const float ms = mn == -INFINITY ? 0.f : mn;  // no token yet: keep exp2 finite
      alpha[qt] = __builtin_amdgcn_exp2f(m_run[qt] - ms);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[u][qt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][qt][r], mulv, -ms));
          ps += s[u][qt][r];
        }
      l_run[qt] = l_run[qt] * alpha[qt] + ps;  // this lane's share; the four lanes of a row add up at the end
      m_run[qt] = mn;
      // alpha is exactly 1 where the running maximum did not change; a wave
      // whose rows all kept theirs skips the rescale (bit for bit the same)
      if (__builtin_amdgcn_ballot_w64(alpha[qt] != 1.0f) != 0) {  // uniform
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[qt][dt] *= alpha[qt];
      }
    }
    // O^T += V^T P^T over two 32-token chunks. Contraction slot (g, j) of
    // chunk c is token 32c + 16(j/4) + 4g + j%4: the probabilities a lane
    // holds for its row. V^T comes from two transposing reads per fragment
    // (slots j = 4h .. 4h+3): in a 16-lane group the four lanes 4j'..4j'+3
    // read the 16 fp16 values of the dim tile for token slot 4h + j' (8
    // bytes each), and lane i receives value i of each of the four slots
    // (the lane layout of ds_read_b64_tr_b16, checked on the GPU).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // head = fp16(p) two at a time; remainder = fp16(p - head), the
      // difference exact in the FMA (v_fma_mix_f32 reads the fp16 head)
      v8h ph[2], pl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float p0 = s[2 * c + j / 4][qt][j % 4], p1 = s[2 * c + j / 4][qt][j % 4 + 1];
          const v2h h = __builtin_convertvector(v2f{p0, p1}, v2h);
          // each remainder rounded to fp16 straight from the FMA (v_fma_mixlo/hi_f16)
          ph[qt][j] = h[0];
          ph[qt][j + 1] = h[1];
          pl[qt][j] = (_Float16)__builtin_fmaf(-(float)h[0], one, p0);
          pl[qt][j + 1] = (_Float16)__builtin_fmaf(-(float)h[1], one, p1);
        }
      const uint8_t* vrow = V + (32 * c + 4 * g + (c16 >> 2)) * kVRow + 8 * (c16 & 3);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vrow + 32 * dt));
        const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vrow + 16 * kVRow + 32 * dt));
        const v4h h0 = __builtin_bit_cast(v4h, r0), h1 = __builtin_bit_cast(v4h, r1);
        const v8h vf = v8h{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph[qt], acc[qt][dt], 0, 0, 0);
          acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[qt], acc[qt][dt], 0, 0, 0);
        }
      }
    }
    debug_stage_sync();
    if (tile + 1 < ntiles) store_tile(st ^ 1);  // the other stage was last read before this tile's barrier
    debug_stage_sync();
  }

  // normalise and store: lane (c, g) holds dims 16dt + 4g .. +3 of row 16qt + c
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float l = cross4_sum(l_run[qt]);
    if (!active[qt]) continue;
    const float inv = l > 0.f ? vs / l : 0.f;
    uint16_t* dst = out + orow[qt] * ldo + (int64_t)ohead[qt] * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint32_t lo = (uint32_t)to_bf16_bits(acc[qt][dt][0] * inv) | ((uint32_t)to_bf16_bits(acc[qt][dt][1] * inv) << 16);
      const uint32_t hi = (uint32_t)to_bf16_bits(acc[qt][dt][2] * inv) | ((uint32_t)to_bf16_bits(acc[qt][dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(lo, hi);
    }
  }
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status fp8blk_prefill_attention(const uint16_t* q, int64_t ldq, int64_t total_q, int64_t B,
                                                  int64_t Hq, int64_t Hkv, int64_t D, const int32_t* cu_seqlens_q,
                                                  int64_t max_seqlen_q, const uint8_t* k_cache, const uint8_t* v_cache,
                                                  int64_t num_slots, const int32_t* block_table, int64_t max_blocks,
                                                  int64_t block_size, const int32_t* context_lens,
                                                  const float* q_scale, const float* k_scale, const float* v_scale,
                                                  float sm_scale, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (B < 0 || total_q < 0 || Hq < 1 || Hkv < 1 || D < 1 || max_seqlen_q < 0 || max_blocks < 1 || block_size < 1 ||
      num_slots < 0 || !(sm_scale == sm_scale) || ldq < Hq * D || ldo < Hq * D)
    return FP8BLK_ERR_INVALID_ARG;
  const int64_t G = Hq / Hkv;
  if (D != kD || Hq % Hkv || (G != 1 && G != 2 && G != 4 && G != 8) || ldq % 8 || ldo % 8 ||
      num_slots % block_size || num_slots > INT32_MAX / Hkv || max_blocks > INT32_MAX || block_size > INT32_MAX)
    return FP8BLK_ERR_SHAPE;
  if (B == 0 || total_q == 0 || max_seqlen_q == 0) return FP8BLK_OK;
  if (!q || !cu_seqlens_q || !k_cache || !v_cache || !block_table || !context_lens || !q_scale || !k_scale ||
      !v_scale || !out)
    return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(cu_seqlens_q, 4) || !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(q_scale, 4) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return FP8BLK_ERR_ALIGNMENT;
  const int64_t bq = kRows / G;
  const int64_t nqb = (max_seqlen_q + bq - 1) / bq;
  if (B * Hkv * nqb > INT32_MAX) return FP8BLK_ERR_SHAPE;
  const dim3 grid((uint32_t)(B * Hkv * nqb));
#define FP8BLK_PREFILL_LAUNCH(GV)                                                                                 \
  hipLaunchKernelGGL((prefill_attention_kernel<GV>), grid, dim3(256), 0, stream, q, ldq, total_q, B, Hkv,        \
                     cu_seqlens_q, nqb, k_cache, v_cache, num_slots, block_table, max_blocks, block_size,         \
                     context_lens, q_scale, k_scale, v_scale, sm_scale, out, ldo)
  switch (G) {
    case 1: FP8BLK_PREFILL_LAUNCH(1); break;
    case 2: FP8BLK_PREFILL_LAUNCH(2); break;
    case 4: FP8BLK_PREFILL_LAUNCH(4); break;
    default: FP8BLK_PREFILL_LAUNCH(8); break;
  }
#undef FP8BLK_PREFILL_LAUNCH
  return launch_status();
}
