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
// The scale rule and the encoders are in quant_common.h.
#include <algorithm>

#include "common.h"
#include "quant_common.h"

namespace fp8blk {
namespace {

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
    // all 64 lanes take part in the row maximum
    const float sc = group_scale(__uint_as_float(row16_max_bits(amax8_bits(w))), pow2);
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

  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    mb = max(mb, amax8_bits(ww));
  }
  float m = __uint_as_float(row16_max_bits(mb));
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
// Transposed quantization for the backward GEMMs (FP8 training: upppp.jp
// «FP8適用の難所：数値のズレ問題», greentreeone.com «Технический прорыв»).
// Each backward GEMM reads its operands along its contraction dimension:
// wgrad contracts over the tokens, so dY and X are quantized in 128x1 groups
// (128 consecutive rows of one column) and written transposed; dgrad reads W
// along N, so the weight's 128x128 blocks are written transposed.

// X [M][K] -> Q^T [K][M], S^T [K][M/128]: one workgroup of 4W threads per
// 128 x W tile (rows m0.., columns k0..; W = 128 when K % 128 == 0 and
// K <= 16384, else 64: each row is read in 256- or 128-byte pieces). Thread t loads rows 2q,
// 2q+1 (q = t/(W/8), +32) of 16-byte column chunk t%(W/8) and stores each
// column's two values as one dword of LDS row k (a column of the tile) at
// dword q: W LDS rows of 128 values, row stride 65 dwords (the reads below
// hit 64 distinct banks; with W = 128 the writes are 2-way). Then thread
// t = 4k + p takes rows 32p..32p+31 of column k: the four lanes of a quad
// hold one 128-row group, reduced by two DPP steps, and store its 128 codes
// as one contiguous 128-byte run.
constexpr int kTStride = 65;  // dwords per LDS row
// 128-wide tiles up to this K (measured 2-13% faster than 64-wide at K = 4096 .. 14336 on 16384
// rows, 4% slower at K = 28672)
constexpr int64_t kQuantTWideMaxK = 16384;

//
// GROUPED: rows sorted by expert (offsets[E+1] on the device); the 128-row
// tiles start at each expert's first row and rows past the expert's end
// read as zero, and tile t of the concatenated per-expert tile lists is
// written at columns 128t.. of Q^T rows ld long (the padded token axis).
template <int W, bool GROUPED>
__global__ __launch_bounds__(4 * W) void quant_act_t_kernel(const u32x4* __restrict__ x, int64_t M, int64_t K,
                                                            u32x4* __restrict__ qt, float* __restrict__ st,
                                                            int pow2, const int32_t* __restrict__ offsets, int E,
                                                            int64_t ld) {
  static_assert(W == 64 || W == 128, "tile width: 8 or 16 sixteen-byte units per row");
  __shared__ uint32_t lds[W * kTStride];
  const int t = threadIdx.x;
  const int64_t k_tiles = K / W;
  const int64_t tile = blockIdx.x / k_tiles, k0 = (int64_t)(blockIdx.x % k_tiles) * W;
  int64_t m0 = tile * 128, rows = 128;  // source rows m0 .. m0 + rows - 1
  if (GROUPED) {
    int e, j;
    if (!locate_tile<128>(offsets, E, (int)tile, e, j) || (tile + 1) * 128 > ld) return;  // uniform
    // the expert's rows clamped to [0, M]: offsets that break their
    // contract give wrong codes, never a read outside x
    const RowRange r = clamp_rows(offsets[e], offsets[e + 1], M);
    m0 = r.lo + 128 * (int64_t)j;
    rows = r.hi - m0 < 128 ? r.hi - m0 : 128;
  } else {
    ld = M;
  }
  const int c = t % (W / 8), q = t / (W / 8);  // q < 32
  const int64_t row_units = K / 8;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 2 * (q + 32 * i) + h;
      v[2 * i + h] = (!GROUPED || r < rows) ? __builtin_nontemporal_load(&x[(m0 + r) * row_units + k0 / 8 + c])
                                            : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t e0[4] = {v[2 * i].x, v[2 * i].y, v[2 * i].z, v[2 * i].w};      // row 2q'
    const uint32_t e1[4] = {v[2 * i + 1].x, v[2 * i + 1].y, v[2 * i + 1].z, v[2 * i + 1].w};  // row 2q'+1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // column 8c + 2j (low halves) and 8c + 2j + 1 (high halves)
      lds[(8 * c + 2 * j) * kTStride + q + 32 * i] = __builtin_amdgcn_perm(e1[j], e0[j], 0x05040100u);
      lds[(8 * c + 2 * j + 1) * kTStride + q + 32 * i] = __builtin_amdgcn_perm(e1[j], e0[j], 0x07060302u);
    }
  }
  __syncthreads();
  const int k = t >> 2, p = t & 3;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = lds[k * kTStride + 16 * p + i];  // rows 32p + 2i, +1
  uint32_t mb = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) mb = max(mb, amax8_bits(&w[4 * g]));
  mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, true));
  mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x4E, 0xF, 0xF, true));
  const float sc = group_scale(__uint_as_float(mb), pow2);
  u32x2 code[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) code[g] = encode8(&w[4 * g], sc);
  const int64_t c0 = tile * 128;  // destination column (= m0 for the plain layout)
  u32x4* dst = qt + (k0 + k) * (ld / 16) + (c0 + 32 * p) / 16;
  __builtin_nontemporal_store(u32x4{code[0].x, code[0].y, code[1].x, code[1].y}, dst);
  __builtin_nontemporal_store(u32x4{code[2].x, code[2].y, code[3].x, code[3].y}, dst + 1);
  if (p == 0) st[(k0 + k) * (ld / 128) + c0 / 128] = sc;
}

// 4x4 byte transpose: a[i] holds row i (byte j = column j); returns column j
// in b[j] (byte i = row i).
__device__ __forceinline__ void transpose4x4(const uint32_t a[4], uint32_t b[4]) {
  const uint32_t p01l = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
  const uint32_t p01h = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
  const uint32_t p23l = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
  const uint32_t p23h = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
  b[0] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
  b[1] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
  b[2] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
  b[3] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
}

// W [N][K] -> QW^T [K][N], SW^T [K/128][N/128]: one workgroup per 128x128
// block. Thread t holds the 8x8 sub-block rows 8(t/16).., columns 8(t%16)..
// (eight 16-byte loads; the 16 threads of a row group read 256 contiguous
// bytes), the block maximum goes through DPP and LDS, the codes are
// transposed in registers (v_perm) and staged through LDS so that the
// transposed rows leave as 16-byte coalesced stores.
__global__ __launch_bounds__(256) void quant_weight_t_kernel(const u32x4* __restrict__ w, int64_t N, int64_t K,
                                                             u32x4* __restrict__ qt, float* __restrict__ st,
                                                             int pow2) {
  __shared__ float red[16];
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 32];  // transposed codes, 128 rows of 128 bytes
  const int t = threadIdx.x;
  const int64_t kblocks = K / kBlock;
  const int64_t bi = blockIdx.x / kblocks, bj = blockIdx.x % kblocks;
  {  // matrix blockIdx.y of a stack: W [E][N][K] -> W^T [E][K][N], scales [E][K/128][N/128]
    const int64_t e = blockIdx.y;
    w += e * N * (K / 8);
    qt += e * K * (N / 16);
    st += e * kblocks * (N / kBlock);
  }
  const int R = t >> 4, C = t & 15;
  const int64_t row_units = K / 8;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(&w[(bi * kBlock + 8 * R + i) * row_units + bj * 16 + C]);
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    mb = max(mb, amax8_bits(ww));
  }
  float m = __uint_as_float(row16_max_bits(mb));
  if ((t & 15) == 0) red[t >> 4] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
  const float sc = group_scale(m, pow2);
  // codes of rows 8R+i, columns 8C..8C+7: lo word = columns 0-3, hi = 4-7
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const u32x2 c = encode8(ww, sc);
    lo[i] = c.x;
    hi[i] = c.y;
  }
  // transposed: column 8C + j of W is row 8C + j of W^T, bytes = rows 8R..8R+7
  uint32_t c_lo[4], c_hi[4], d_lo[4], d_hi[4];
  transpose4x4(&lo[0], c_lo);  // rows 0-3, columns 0-3
  transpose4x4(&lo[4], c_hi);  // rows 4-7, columns 0-3
  transpose4x4(&hi[0], d_lo);  // rows 0-3, columns 4-7
  transpose4x4(&hi[4], d_hi);  // rows 4-7, columns 4-7
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tile[(8 * C + j) * 32 + 2 * R] = c_lo[j];
    tile[(8 * C + j) * 32 + 2 * R + 1] = c_hi[j];
    tile[(8 * C + 4 + j) * 32 + 2 * R] = d_lo[j];
    tile[(8 * C + 4 + j) * 32 + 2 * R + 1] = d_hi[j];
  }
  __syncthreads();
  const int64_t out_units = N / 16;  // 16-byte units per W^T row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = t + 256 * i, r = id >> 3, u = id & 7;  // 128 rows x 8 units
    const u32x4 val = *reinterpret_cast<const u32x4*>(&tile[r * 32 + 4 * u]);
    __builtin_nontemporal_store(val, &qt[(bj * kBlock + r) * out_units + bi * 8 + u]);
  }
  if (t == 0) st[bj * (N / kBlock) + bi] = sc;
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
  // across the rows: lane-swap instructions (each lane gets its pair's sum
  // in the same order as its partner), no LDS round trip
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two fp32 values to a packed bf16 pair (lo in the low half), round to
// nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Quantize one lane's 8 bf16 values w[0..3] as part of the 128-wide group
// formed by its 16-lane DPP row, and store codes, scale and (optionally)
// the bf16 values. `live` is uniform over the row; every lane of the wave
// must call this (DPP).
__device__ __forceinline__ void quant_store8(const uint32_t w[4], int pow2, bool live, u32x2* q_unit,
                                             float* s_group, bool first_lane, u32x4* y_unit) {
  const float sc = group_scale(__uint_as_float(row16_max_bits(amax8_bits(w))), pow2);
  const u32x2 codes = encode8(w, sc);
  if (live) {
    __builtin_nontemporal_store(codes, q_unit);
    if (first_lane) *s_group = sc;
    if (y_unit) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, y_unit);
  }
}

// Sum of squares of the 8 bf16 values of a 16-byte unit added to acc, one
// v_dot2_f32_bf16 per pair (exact bf16 products, fp32 accumulation).
__device__ __forceinline__ float sum_sq8(u32x4 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = __builtin_bit_cast(bf16x2, w[i]);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// ---------------------------------------------------------------- RMSNorm
// Workgroups of four waves, each taking `iters` (1 to 4) consecutive slices
// of rows: more rows per workgroup amortise gamma, fewer keep the grid
// large enough to fill the chip when M is small. Each row is handled by WPR waves (T = 64*WPR threads; thread t
// holds 16-byte units t, t+T, .. of the row, at most CU of them, so a
// 16-lane DPP row holds whole 128-wide groups). gamma is loaded once per
// workgroup and kept in registers; the next row's x is loaded while the
// current one is normalised and quantized. With WPR > 1 the waves of a row
// add their partial sums through LDS, in a fixed order (the result does not
// depend on timing).
constexpr int kRmsMaxIters = 4;
constexpr int64_t kRmsTargetWGs = 2048;  // 256 CUs x 8 resident four-wave workgroups
constexpr int kNontemporal = 2;  // cache-policy bits of a buffer load: nt (streamed once)

template <int WPR, int CU>
__global__ __launch_bounds__(256) void rmsnorm_quant_act_rows_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ gamma, float eps, int64_t M, int64_t K,
    u32x2* __restrict__ q, float* __restrict__ s, u32x4* __restrict__ y, int pow2, int iters) {
  constexpr int T = 64 * WPR;
  constexpr int RPW = 4 / WPR;  // rows per workgroup and iteration
  // gamma as fp32 when it fits, else packed and widened at each use
  constexpr bool kGammaF32 = CU <= 2;
  __shared__ float red[2][4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = wave / WPR, t = (wave % WPR) * 64 + lane;
  const int64_t units = K / 8, kb = K / kBlock;

  u32x4 gp[CU];
  float gf[kGammaF32 ? CU : 1][8];
#pragma unroll
  for (int c = 0; c < CU; ++c) {
    const int64_t u = t + (int64_t)c * T;
    gp[c] = u < units ? gamma[u] : u32x4{0, 0, 0, 0};
    if constexpr (kGammaF32) {
      const uint32_t g[4] = {gp[c].x, gp[c].y, gp[c].z, gp[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gf[c][2 * i] = bf16_lo(g[i]);
        gf[c][2 * i + 1] = bf16_hi(g[i]);
      }
    }
  }

  // Branch-free row loads: the resource covers the wave's row (nothing
  // past the last row), so units past the row end, and rows past M, read
  // as zeros. K <= 8192 here: offsets stay far below 2^32.
  const int64_t first = (int64_t)blockIdx.x * RPW * iters;
  auto load_row = [&](u32x4 (&v)[CU], int64_t row) {
    const bool in = row < M;
    const rsrc_t rs = make_rsrc(x + (in ? row : 0) * units, in ? (uint32_t)(K * 2) : 0u);
#pragma unroll
    for (int c = 0; c < CU; ++c)
      v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(t + c * T) * 16u, 0,
                                                                           kNontemporal));
  };
  u32x4 cur[CU];
  load_row(cur, first + sub);
  for (int it = 0; it < iters; ++it) {
    const int64_t base = first + it * RPW;
    if (base >= M) break;  // uniform over the workgroup
    const int64_t row = base + sub;
    const int buf = it & 1;

    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CU; ++c) ss = sum_sq8(cur[c], ss);
    // Issue the next row's loads only after this row's data has been
    // consumed: the wait the compiler places before the first use of
    // `cur` then does not also wait for the prefetch.
    asm volatile("" : "+v"(ss) : : "memory");
    u32x4 nxt[CU] = {};
    if (it + 1 < iters) load_row(nxt, row + RPW);  // uniform

    ss = wave_sum(ss);
    if constexpr (WPR > 1) {
      // double-buffered: a wave can only overwrite red[buf] two iterations
      // later, after every wave has passed the barrier of the next one
      if (lane == 0) red[buf][wave] = ss;
      __syncthreads();
      ss = red[buf][sub * WPR];
#pragma unroll
      for (int j = 1; j < WPR; ++j) ss += red[buf][sub * WPR + j];
    }
    // r = 1 / sqrt(mean + eps): correctly rounded fp32 division and square root
    const float r = 1.0f / sqrtf(ss / (float)K + eps);

#pragma unroll
    for (int c = 0; c < CU; ++c) {
      const int64_t u = t + (int64_t)c * T;
      const bool live = row < M && u < units;  // uniform over each 16-lane row
      const uint32_t xw[4] = {cur[c].x, cur[c].y, cur[c].z, cur[c].w};
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float g0, g1;
        if constexpr (kGammaF32) {
          g0 = gf[c][2 * i];
          g1 = gf[c][2 * i + 1];
        } else {
          const uint32_t g[4] = {gp[c].x, gp[c].y, gp[c].z, gp[c].w};
          g0 = bf16_lo(g[i]);
          g1 = bf16_hi(g[i]);
        }
        w[i] = pack_bf16(bf16_lo(xw[i]) * r * g0, bf16_hi(xw[i]) * r * g1);
      }
      const int64_t e = live ? row * units + u : 0;
      quant_store8(w, pow2, live, &q[e], &s[live ? row * kb + u / 16 : 0], (lane & 15) == 0,
                   y ? &y[e] : nullptr);
    }
#pragma unroll
    for (int c = 0; c < CU; ++c) cur[c] = nxt[c];
  }
}

// Rows too long for the register cache of the kernel above (K > 8192): one
// wave per row, the row read twice (the second time mostly from L2).
__global__ __launch_bounds__(256) void rmsnorm_quant_act_long_kernel(const u32x4* __restrict__ x,
                                                                     const u32x4* __restrict__ gamma, float eps,
                                                                     int64_t M, int64_t K, u32x2* __restrict__ q,
                                                                     float* __restrict__ s, u32x4* __restrict__ y,
                                                                     int pow2) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform over the wave
  const int64_t units = K / 8, kb = K / kBlock;
  const u32x4* xr = x + row * units;
  float ss = 0.0f;
  for (int64_t u = lane; u < units; u += 64) ss = sum_sq8(xr[u], ss);
  ss = wave_sum(ss);  // the lanes reconverge after the loop
  const float r = 1.0f / sqrtf(ss / (float)K + eps);
  for (int64_t u0 = 0; u0 < units; u0 += 64) {  // uniform
    const int64_t u = u0 + lane;
    const bool live = u < units;
    const u32x4 v = live ? xr[u] : u32x4{0, 0, 0, 0};
    const u32x4 gv = live ? gamma[u] : u32x4{0, 0, 0, 0};
    const uint32_t xw[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16(bf16_lo(xw[i]) * r * bf16_lo(gw[i]), bf16_hi(xw[i]) * r * bf16_hi(gw[i]));
    const int64_t e = live ? row * units + u : 0;
    quant_store8(w, pow2, live, &q[e], &s[live ? row * kb + u / 16 : 0], (lane & 15) == 0,
                 y ? &y[e] : nullptr);
  }
}

// ---------------------------------------------------------------- SiLU * up
// silu(g) * u = g * u / (1 + 2^a), a = -g log2(e), with the hardware exp2
// and reciprocal (each within 1 ulp). The reciprocal does not return
// subnormals, so 1 + 2^a must stay below 2^126: silu_mul_near serves
// g > -64 (a < 92.4). For g <= -64, silu_mul_far takes the denominator
// scaled by 2^-64 (2^-64 + 2^(a-64)) and scales the result back by an exact
// 2^-64 at the end; exp2 then overflows only where the exact result is far
// below the smallest bf16 subnormal. Relative error before the bf16
// rounding: below 2^-16 (dominated by the rounding of a, at most
// 2^-24 * |a| with |a| <= 192 where the result is not negligible); for
// g > 0 large, sigma is 1 to fp32 precision.
constexpr float kLog2e = 1.44269504088896341f;

__device__ __forceinline__ float silu_mul_near(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e)) * u;
}

__device__ __forceinline__ float silu_mul_far(float g, float u) {
  const bool far = g <= -64.0f;
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(-g, kLog2e, far ? -64.0f : 0.0f));
  const float h = g * __builtin_amdgcn_rcpf((far ? 0x1p-64f : 1.0f) + e) * u;
  return far ? h * 0x1p-64f : h;
}

// Whether any of the 8 packed bf16 gates is <= -64: the bit patterns of
// negative values grow with their magnitude, and -64 is 0xC280.
__device__ __forceinline__ bool any_gate_far(const uint32_t gw[4]) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, gw[0]);
#pragma unroll
  for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, gw[i]));
  return max((uint32_t)m.x, (uint32_t)m.y) >= 0xC280u;
}

// gu is [M][2F] = [gate | up] per row; the output groups are the M * F/128
// groups of h = silu(g) * u, laid out like quant_act_kernel's (a 16-lane
// row per group, 16 groups per wave).
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
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16(silu_mul_near(bf16_lo(gw[i]), bf16_lo(uw[i])),
                       silu_mul_near(bf16_hi(gw[i]), bf16_hi(uw[i])));
    if (__builtin_amdgcn_ballot_w64(any_gate_far(gw)) != 0) {  // uniform; gates <= -64 are rare
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16(silu_mul_far(bf16_lo(gw[i]), bf16_lo(uw[i])),
                         silu_mul_far(bf16_hi(gw[i]), bf16_hi(uw[i])));
    }
    const int64_t unit = gi < groups ? gi * 16 + (lane & 15) : 0;
    quant_store8(w, pow2, gi < groups, &q[unit], &s[gi < groups ? gi : 0], (lane & 15) == 0,
                 y ? &y[unit] : nullptr);
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

extern "C" fp8blk_status fp8blk_quant_act_t(const uint16_t* x, int64_t M, int64_t K, uint8_t* qt, float* st,
                                            int pow2, hipStream_t stream) {
  if (M < 0 || K <= 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (M % kBlock || K % 64) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !qt || !st) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(qt, 16) || !aligned(st, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t blocks = (M / kBlock) * (K / 64);  // the 64-wide count bounds the 128-wide one
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  if (K % 128 == 0 && K <= kQuantTWideMaxK)
    hipLaunchKernelGGL((quant_act_t_kernel<128, false>), dim3((uint32_t)(blocks / 2)), dim3(512), 0, stream,
                       reinterpret_cast<const u32x4*>(x), M, K, reinterpret_cast<u32x4*>(qt), st, pow2, nullptr, 0,
                       M);
  else
    hipLaunchKernelGGL((quant_act_t_kernel<64, false>), dim3((uint32_t)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(x), M, K, reinterpret_cast<u32x4*>(qt), st, pow2, nullptr, 0,
                       M);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_quant_act_t_grouped(const uint16_t* x, int64_t M, int64_t K, const int32_t* offsets,
                                                    int64_t E, int64_t ld, uint8_t* qt, float* st, int pow2,
                                                    hipStream_t stream) {
  if (M < 0 || K <= 0 || E < 1 || ld < 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (K % 64 || ld % kBlock || E > INT32_MAX - 1 || M > INT32_MAX) return FP8BLK_ERR_SHAPE;
  if (M == 0 || ld == 0) return FP8BLK_OK;
  if (!x || !offsets || !qt || !st) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(offsets, 4) || !aligned(qt, 16) || !aligned(st, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t tiles = ld / kBlock;  // the padded axis holds at most this many 128-token tiles
  const int64_t blocks = tiles * (K / 64);
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  if (K % 128 == 0 && K <= kQuantTWideMaxK)
    hipLaunchKernelGGL((quant_act_t_kernel<128, true>), dim3((uint32_t)(blocks / 2)), dim3(512), 0, stream,
                       reinterpret_cast<const u32x4*>(x), M, K, reinterpret_cast<u32x4*>(qt), st, pow2, offsets,
                       (int)E, ld);
  else
    hipLaunchKernelGGL((quant_act_t_kernel<64, true>), dim3((uint32_t)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(x), M, K, reinterpret_cast<u32x4*>(qt), st, pow2, offsets,
                       (int)E, ld);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_quant_weight_t_grouped(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                                                       uint8_t* qt, float* st, int pow2, hipStream_t stream) {
  if (E < 1 || N < 0 || K <= 0 || (pow2 != 0 && pow2 != 1)) return FP8BLK_ERR_INVALID_ARG;
  if (N % kBlock || K % kBlock || E > 65535) return FP8BLK_ERR_SHAPE;
  if (N == 0) return FP8BLK_OK;
  if (!w || !qt || !st) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(qt, 16) || !aligned(st, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t blocks = (N / kBlock) * (K / kBlock);
  if (blocks > INT32_MAX) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(quant_weight_t_kernel, dim3((uint32_t)blocks, (uint32_t)E), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(w), N, K, reinterpret_cast<u32x4*>(qt), st, pow2);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_quant_weight_t(const uint16_t* w, int64_t N, int64_t K, uint8_t* qt, float* st,
                                               int pow2, hipStream_t stream) {
  return fp8blk_quant_weight_t_grouped(w, 1, N, K, qt, st, pow2, stream);
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
  if ((M + 3) / 4 > INT32_MAX) return FP8BLK_ERR_SHAPE;  // the largest grid below: 4 rows per workgroup
  const int64_t units = K / 8;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const u32x4* gv = reinterpret_cast<const u32x4*>(gamma);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  u32x4* yv = reinterpret_cast<u32x4*>(y);
  // waves per row and cached units per lane: 8 to 16 values per lane in
  // registers for K <= 4096, 32 for K <= 8192
  auto launch = [&](auto kernel, int64_t rows_per_iter) {
    const int iters = (int)std::max<int64_t>(1, std::min<int64_t>(kRmsMaxIters, M / (rows_per_iter * kRmsTargetWGs)));
    const int64_t rows_per_wg = rows_per_iter * iters;
    const int64_t wgs = (M + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)wgs), dim3(256), 0, stream, xv, gv, eps, M, K, qv, s, yv, pow2,
                       iters);
  };
  if (units <= 128) {
    launch(rmsnorm_quant_act_rows_kernel<1, 2>, 4);
  } else if (units <= 256) {
    launch(rmsnorm_quant_act_rows_kernel<2, 2>, 2);
  } else if (units <= 512) {
    launch(rmsnorm_quant_act_rows_kernel<4, 2>, 1);
  } else if (units <= 1024) {
    launch(rmsnorm_quant_act_rows_kernel<4, 4>, 1);
  } else {
    const int64_t blocks = (M + 3) / 4;  // one wave per row
    hipLaunchKernelGGL(rmsnorm_quant_act_long_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, xv, gv, eps,
                       M, K, qv, s, yv, pow2);
  }
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

// Callers may pass any integer (the header promises "unknown status" for
// unknown codes), and a value outside the enumerators' range is undefined
// behaviour when read as the enum: the code is read as an int.
extern "C" const char* fp8blk_status_string(fp8blk_status status) {
  int code;
  static_assert(sizeof(code) == sizeof(status), "status codes are int-sized");
  __builtin_memcpy(&code, &status, sizeof(code));
  switch (code) {
    case FP8BLK_OK: return "ok";
    case FP8BLK_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad flag)";
    case FP8BLK_ERR_SHAPE: return "unsupported shape (K and N must be multiples of 128, GEMM K <= 2^24, E >= 1)";
    case FP8BLK_ERR_ALIGNMENT: return "misaligned pointer (data 16 bytes, scales 4 bytes)";
    case FP8BLK_ERR_HIP: return "HIP kernel launch or device query failed";
    case FP8BLK_ERR_SCRATCH: return "the call needs more device scratch than the library's static buffer holds";
  }
  return "unknown status";
}
