// Block-scaled FP8 (E4M3) GEMM and expert-grouped GEMM for gfx950.
//
// Method (greentreeone.com NeMo RL FP8 article, «Технический прорыв»): the
// linear layers multiply E4M3 operands quantised per 1x128 activation group
// and per 128x128 weight block; each 128-wide slice b of K carries the
// scales SA[m][b] and SW[n/128][b]:
//     Y[m][n] = sum_b SA[m][b] * SW[n/128][b] * sum_{k in b} A[m][k] * W[n][k]
// Mixture-of-experts use (upppp.jp NeMo RL FP8 article, «まとめ»): rows
// sorted by expert, each expert with its own weights.
//
// Kernel structure:
//   * one workgroup computes a BM x BN output tile; its K loop steps one
//     scale block (128) at a time, so the K tile IS the scale block;
//   * A and B K-tiles (row-major, K contiguous) are staged through LDS,
//     double buffered: the global loads of block b+1 are issued before the
//     MFMAs of block b and written to the other LDS buffer afterwards; one
//     barrier per K step;
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     chunk c ^ (r & 7), so the 16 rows an MFMA operand read touches hit
//     distinct banks;
//   * each wave owns a WM x WN sub-tile made of 16x16 tiles; one
//     v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit block scales)
//     yields the exact-in-fp32 partial dot product of one whole scale
//     block, which is folded into the fp32 accumulator with one FMA:
//     acc += partial * (SA[m][b] * SW[n/128][b]);
//   * the epilogue rounds to bf16 (nearest even) and stores.
#include "common.h"

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = kBlock;                  // K step = one scale block
constexpr int BM = 128, BN = 128;           // workgroup tile
constexpr int WAVES_M = 2, WAVES_N = 2;
constexpr int NT = 64 * WAVES_M * WAVES_N;  // threads per workgroup
constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
constexpr int TM = WM / 16, TN = WN / 16;   // 16x16 MFMA tiles per wave
constexpr int A_LD = BM * (BK / 16) / NT;   // 16-byte loads per thread per K step
constexpr int B_LD = BN * (BK / 16) / NT;
static_assert(A_LD * NT == BM * 8 && B_LD * NT == BN * 8, "tile/threads mismatch");
static_assert(BM <= NT, "one thread per A row loads the row scale");
static_assert(kBlock % WN == 0, "a wave's columns lie in one weight block");

struct Smem {
  uint8_t a[2][BM * BK];
  uint8_t b[2][BN * BK];
  float sa[2][BM];
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// Read the 32 K-bytes of operand row `row` that lane group g = lane/16
// supplies to the 16x16x128 MFMA. A and B use the same lane->K mapping, so
// the dot product over the block is independent of how the instruction
// orders K inside it.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int g) {
  const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(row, 2 * g));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(row, 2 * g + 1));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One BM x BN output tile at (m0, n0) of Y[M][N] = A[M][K] W[N][K]^T, with
// rows >= M of A read as row M-1 (valid memory) and never stored. M >= 1.
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                          const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                          int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
                                          int64_t m0, int64_t n0, Smem& sm) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = (wave / WAVES_N) * WM;
  const int wn = (wave % WAVES_N) * WN;
  const int g = lane >> 4;
  const int64_t KB = K / BK;

  const uint4* a_src[A_LD];
  int a_dst[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int cid = t + i * NT, row = cid >> 3, c = cid & 7;
    const int64_t gm = m0 + row < M ? m0 + row : M - 1;
    a_src[i] = reinterpret_cast<const uint4*>(qa + gm * K) + c;
    a_dst[i] = swz(row, c);
  }
  const uint4* b_src[B_LD];
  int b_dst[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int cid = t + i * NT, row = cid >> 3, c = cid & 7;
    b_src[i] = reinterpret_cast<const uint4*>(qw + (n0 + row) * K) + c;
    b_dst[i] = swz(row, c);
  }
  const float* sa_src = sa + (m0 + t < M ? m0 + t : M - 1) * KB;
  const float* sw_src = sw + ((n0 + wn) / kBlock) * KB;

  uint4 ra[A_LD], rb[B_LD];
  float rsa = 0.0f;
  auto gload = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = a_src[i][kb * (BK / 16)];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = b_src[i][kb * (BK / 16)];
    if (t < BM) rsa = sa_src[kb];
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&sm.a[st][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&sm.b[st][b_dst[i]]) = rb[i];
    if (t < BM) sm.sa[st][t] = rsa;
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t kb = 0; kb < KB; ++kb) {
    const int st = (int)(kb & 1);
    if (kb + 1 < KB) gload(kb + 1);
    const float swv = sw_src[kb];
    v8i bfr[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = read_frag(sm.b[st], wn + 16 * j + (lane & 15), g);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i afr = read_frag(sm.a[st], wm + 16 * i + (lane & 15), g);
      const v4f sa4 = *reinterpret_cast<const v4f*>(&sm.sa[st][wm + 16 * i + 4 * g]);
      const v4f sc = sa4 * swv;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sc[r], acc[i][j][r]);
      }
    }
    if (kb + 1 < KB) sstore(st ^ 1);
    __syncthreads();
  }

  // 16x16 accumulator layout: lane holds rows 4*(lane/16) + r, column lane%16
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm + 16 * i + 4 * g + r;
      if (row < M) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          y[row * N + n0 + wn + 16 * j + (lane & 15)] = to_bf16_bits(acc[i][j][r]);
      }
    }
}

__global__ __launch_bounds__(NT) void gemm_kernel(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                  const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                  int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
                                                  int n_tiles) {
  __shared__ Smem sm;
  const int64_t m_tile = blockIdx.x / n_tiles, n_tile = blockIdx.x % n_tiles;
  gemm_tile(qa, sa, qw, sw, M, N, K, y, m_tile * BM, n_tile * BN, sm);
}

// Find which expert owns M-tile `t` of the concatenated per-expert tile
// lists (expert e has ceil(M_e / BM) tiles). Every lane of the wave
// computes the same answer: lanes take 64 experts at a time and a wave
// prefix sum turns per-expert tile counts into tile ranges.
__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ off, int E, int t, int& expert,
                                            int& tile_in_expert) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int cnt = e < E ? (off[e + 1] - off[e] + BM - 1) / BM : 0;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int total = __shfl(incl, 63);
    if (t < base + total) {
      const bool mine = cnt > 0 && t >= base + incl - cnt && t < base + incl;
      const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
      expert = e0 + src;
      tile_in_expert = t - base - __shfl(incl - cnt, src);
      return true;
    }
    base += total;
  }
  return false;
}

__global__ __launch_bounds__(NT) void grouped_gemm_kernel(const uint8_t* __restrict__ qa,
                                                          const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw,
                                                          const float* __restrict__ sw,
                                                          const int32_t* __restrict__ offsets, int E,
                                                          int64_t N, int64_t K, uint16_t* __restrict__ y,
                                                          int n_tiles) {
  __shared__ Smem sm;
  const int t = blockIdx.x / n_tiles, n_tile = blockIdx.x % n_tiles;
  int e, tile;
  if (!locate_tile(offsets, E, t, e, tile)) return;  // uniform over the workgroup
  const int64_t row0 = offsets[e];
  const int64_t rows = offsets[e + 1] - row0;
  const int64_t KB = K / BK;
  gemm_tile(qa + row0 * K, sa + row0 * KB, qw + (int64_t)e * N * K, sw + (int64_t)e * (N / kBlock) * KB,
            rows, N, K, y + row0 * N, (int64_t)tile * BM, (int64_t)n_tile * BN, sm);
}

fp8blk_status check_gemm_args(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, const uint16_t* y) {
  if (M < 0 || N <= 0 || K <= 0) return FP8BLK_ERR_INVALID_ARG;
  if (N % kBlock || K % kBlock) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!qa || !sa || !qw || !sw || !y) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(y, 16) || !aligned(sa, 4) || !aligned(sw, 4))
    return FP8BLK_ERR_ALIGNMENT;
  return FP8BLK_OK;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status fp8blk_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                                     int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const fp8blk_status st = check_gemm_args(qa, sa, qw, sw, M, N, K, y);
  if (st != FP8BLK_OK || M == 0) return st;
  const int64_t n_tiles = N / BN;
  const int64_t m_tiles = (M + BM - 1) / BM;
  if (n_tiles * m_tiles > (1 << 24) || N % BN) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)(n_tiles * m_tiles)), dim3(NT), 0, stream, qa, sa, qw, sw, M,
                     N, K, y, (int)n_tiles);
  return launch_status();
}

extern "C" fp8blk_status fp8blk_grouped_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw,
                                             const float* sw, const int32_t* offsets, int64_t E,
                                             int64_t total_M, int64_t N, int64_t K, uint16_t* y,
                                             hipStream_t stream) {
  if (E < 1) return FP8BLK_ERR_SHAPE;
  if (E > INT32_MAX - 1 || total_M > INT32_MAX) return FP8BLK_ERR_SHAPE;
  const fp8blk_status st = check_gemm_args(qa, sa, qw, sw, total_M, N, K, y);
  if (st != FP8BLK_OK || total_M == 0) return st;
  if (!offsets) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(offsets, 4)) return FP8BLK_ERR_ALIGNMENT;
  const int64_t n_tiles = N / BN;
  // upper bound on the number of M-tiles: sum_e ceil(M_e/BM) <= total_M/BM + E
  const int64_t m_tiles = total_M / BM + E;
  if (n_tiles * m_tiles > (1 << 24) || N % BN) return FP8BLK_ERR_SHAPE;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((uint32_t)(n_tiles * m_tiles)), dim3(NT), 0, stream, qa, sa, qw,
                     sw, offsets, (int)E, N, K, y, (int)n_tiles);
  return launch_status();
}
