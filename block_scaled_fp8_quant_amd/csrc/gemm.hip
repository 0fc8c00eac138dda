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
//   * A and B K-tiles (row-major, K contiguous) and the block's scales are
//     staged through LDS, double buffered. The copies are direct
//     global->LDS buffer loads (buffer_load_dwordx4 / _dword ... lds): no
//     staging registers, and they run while the MFMAs of the previous block
//     do. The buffer range check turns rows past the end of an operand into
//     zeros, so partial tiles need no clamping;
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r sits at chunk
//     c ^ key(r), so the 16 rows an MFMA operand read touches spread over
//     the banks. A direct load writes lane l's 16 bytes at slot l of a 1 KB
//     window, so the swizzle is applied on the global side: the lane that
//     fills slot (row, p) fetches logical chunk p ^ key(row);
//   * each wave owns a WM x WN sub-tile of 16x16 tiles. One
//     v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, no block scales) gives the
//     exact fp32 partial dot product of one whole scale block;
//     the partials are folded into the fp32 accumulators with one FMA each,
//     acc += partial * (SA[m][b] * SW[n/128][b]), one 16-row m-subtile
//     behind the MFMAs so that no fold waits for an MFMA just issued; the
//     MFMA produces the transposed tile so that each lane's quad is 4
//     consecutive outputs of one row (one activation scale per quad);
//   * the K loop body is one basic block (no branches), so the compiler
//     cannot sink the MFMAs behind the barrier; the last m-subtile's MFMAs
//     of a block run while the next block's fragments are read;
//   * the epilogue rounds to bf16 (nearest even) and stores 8 bytes a lane;
//   * workgroups are handed out round-robin over the 8 XCDs; the tile order
//     gives each XCD a contiguous band of tiles so neighbours share A rows
//     and B columns in that XCD's L2;
//   * with many short tiles (at least three 256x256 tiles per CU, at most 64
//     K blocks) a persistent grid walks the same order, each workgroup
//     loading its next tile's first K blocks during its current tile's last
//     steps; the expert-grouped GEMM walks its tiles the same way whenever
//     they outnumber the resident workgroups.
#include <atomic>
#include <mutex>

#include "common.h"

#ifndef FP8BLK_GEMM_GROUP_M
#define FP8BLK_GEMM_GROUP_M 8
#endif
#ifndef FP8BLK_GEMM_PERSISTENT
#define FP8BLK_GEMM_PERSISTENT 1
#endif

// Race-detection build (-DFP8BLK_DEBUG_BARRIERS=1): every LDS stage
// transition of the K loop also waits for all of the wave's loads and passes
// a full workgroup barrier, so no stage can be read while a refill writes it
// or refilled while a wave still reads it. The arithmetic is unchanged: its
// outputs must equal the normal build's bit for bit (a GPU test compares
// them); a difference would expose a missing wait or barrier.
#ifndef FP8BLK_DEBUG_BARRIERS
#define FP8BLK_DEBUG_BARRIERS 0
#endif

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BK = kBlock;  // K step = one scale block
// 32-bit lane offsets into a tile's rows: 256 * K must stay below 2^32
constexpr int64_t kMaxK = int64_t(1) << 24;

// RB_ = false: B carries one scale per 128x128 block (weights), SW[N/128][KB].
// RB_ = true: B carries one scale per row and K block, SB[N][KB] (the wgrad
// operands: 128x1 groups on both sides), so the fold needs a scale per
// output column.
// Cache-policy bits of a buffer load: non-temporal (nt).
constexpr int kStreamAux = 2;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_ = 2, bool RB_ = false, bool STREAM_B_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_;
  static constexpr bool RB = RB_;
  // STREAM_B: B (the weights) is loaded with the non-temporal hint, for
  // calls where few row tiles read each weight block (decode steps, MoE
  // experts): the blocks then do not displace cache lines that are read
  // again. Interleaved A/B on the decode and MoE layers: 13-34% and 6-11%
  // faster; on the prefill shapes, whose weight blocks are read by 64 row
  // tiles, 2-5% slower, so those keep the default policy.
  static constexpr bool STREAM_B = STREAM_B_;
  static constexpr int B_AUX = STREAM_B ? kStreamAux : 0;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N, NT = 64 * WAVES;
  // PAIR (the 256x256 tiles): the first half of the waves issue every
  // refill load, their own windows, those of wave w + WAVES/2 and the
  // weight-scale window (RB: wave w + WAVES/2's B-row scale window). Waves w and w + WAVES/2 share a SIMD and the
  // older one, w, is issued first and finishes its rows of a K step well
  // ahead of the younger, which then runs alone until the step's barrier;
  // moving the younger wave's loads to the older balances the pair
  // (5-10% faster on the prefill GEMMs, 5-15% on the wgrad GEMMs; on the
  // 256x128 tile it measured
  // faster with hot operands but slower with the weights cold in HBM).
  static constexpr bool PAIR = WAVES_M_ * WAVES_N_ == 8 && BM == 256 && BN == 256;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  // 1 KB direct-load windows (8 rows of 128 bytes) per wave per K step
  static constexpr int A_WIN = BM / 8 / WAVES, B_WIN = BN / 8 / WAVES;
  static_assert(A_WIN * 8 * WAVES == BM && B_WIN * 8 * WAVES == BN, "rows per wave");
  static_assert(BM % 64 == 0 && BM / 64 < WAVES, "row scales: one dword window per wave, one wave left for the weight scales");
  static_assert(!RB || (BN % 64 == 0 && BM / 64 + BN / 64 <= WAVES), "RB: one dword window per wave for A and B rows");
  static_assert(kBlock % WN == 0, "a wave's columns lie in one weight block");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "16x16 MFMA tiles");
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  // A tile, B tile, BM row scales, then a 256-byte window of weight scales
  // (RB: BN row scales of B)
  static constexpr int STAGE = A_BYTES + B_BYTES + BM * 4 + (RB ? BN * 4 : 256);
  static constexpr int LDS = STAGES * STAGE + 4 * WAVES;  // stages, then one scale verdict per wave
  // direct loads one wave issues per stage: its A and B windows and one scale window
  static constexpr int LOADS_PER_STAGE = A_WIN + B_WIN + 1;
  static_assert(STAGES >= 2 && STAGES <= 8, "stage index is kb mod STAGES (a multiply for 3)");
  static_assert(LOADS_PER_STAGE * 2 * (STAGES - 1) <= 63, "outstanding loads fit the vmcnt counter");
};

// Tile configurations, picked per call from the problem shape (host side):
//   Big   256x256, 8 waves of 128x64, 2 stages: large M and N (one workgroup
//         per CU);
//   Mid   128x128, 4 waves of 64x64, 2 stages: medium problems, expert groups
//         of ~100+ rows (two workgroups per CU);
//   Small  64x64,  4 waves of 64x16, 4 stages: few rows (decode steps, small
//         experts); a step holds little MFMA work, so three blocks stay in
//         flight to cover the load latency (two workgroups per CU);
//   Skinny 256x128, 8 waves of 64x64, 3 stages: at most 256 rows with enough
//         column tiles to fill most CUs (a decode step's wide linears): one
//         workgroup covers every row, so each weight block is read by one
//         workgroup, and a wave has 16 MFMAs per K step instead of Small's 4
//         (1.7x faster than Small on a 256 x 28672 x 4096 decode GEMM). With
//         one workgroup per CU its streaming is bound by the blocks in
//         flight: the third stage (148 KB of LDS) keeps two ahead instead of
//         one (7-11% faster with the weights cold in HBM).
#ifndef FP8BLK_MID_STAGES
#define FP8BLK_MID_STAGES 2
#endif
#ifndef FP8BLK_SMALL_STAGES
#define FP8BLK_SMALL_STAGES 4
#endif
using Big = Tile<256, 256, 2, 4>;
using Mid = Tile<128, 128, 2, 2, FP8BLK_MID_STAGES>;
using Small = Tile<64, 64, 1, 4, FP8BLK_SMALL_STAGES>;
using BigRB = Tile<256, 256, 2, 4, 2, true>;
using MidRB = Tile<128, 128, 2, 2, FP8BLK_MID_STAGES, true>;
using SmallRB = Tile<64, 64, 1, 4, FP8BLK_SMALL_STAGES, true>;
using Skinny = Tile<256, 128, 4, 2, 3>;
// the same tiles with streamed weights
using BigS = Tile<256, 256, 2, 4, 2, false, true>;
using MidS = Tile<128, 128, 2, 2, FP8BLK_MID_STAGES, false, true>;
using SmallS = Tile<64, 64, 1, 4, FP8BLK_SMALL_STAGES, false, true>;
using SkinnyS = Tile<256, 128, 4, 2, 3, false, true>;
// weights are streamed when each weight block is read by at most this many
// row tiles
constexpr int64_t kStreamMaxRowTiles = 4;
static_assert(Big::LDS <= 160 * 1024 && Mid::LDS <= 160 * 1024 && Small::LDS <= 160 * 1024 &&
                  Skinny::LDS <= 160 * 1024,
              "LDS budget");
static_assert(BigRB::LDS <= 160 * 1024 && MidRB::LDS <= 160 * 1024 && SmallRB::LDS <= 160 * 1024, "LDS budget");

// 16-byte chunk c of LDS row r is stored at chunk c ^ key(r), so the 16
// rows that one operand read touches (same logical chunk) are spread over
// different physical chunks. key = (r >> 1) & 7 and key = r & 7 measured
// the same: with 8 waves reading, both run at the rate of a contiguous 1 KB
// read (256 bytes per clock per CU); without the swizzle, 73.
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_key(row)) << 4); }

// The 32 K-bytes of operand row `row` that lane group g = lane/16 supplies to
// the 16x16x128 MFMA: logical chunks g and g+4 (bytes 16g.. and 64+16g..).
// A and B use the same lane->K mapping, so the block's dot product does not
// depend on how the instruction orders K inside it. With this pairing the
// 16 lanes of each LDS pass (one lane group, 16 rows) hit 16 distinct bank
// groups; chunks 2g and 2g+1 measured 1.7x slower (bank conflicts).
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int g) {
  const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(row, g));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(row, g + 4));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]; the maximum in a field means "do not wait").
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding global load, including the direct
// loads of the next stage that are meant to stay in flight. This wave's LDS
// reads are completed first. Builtins rather than inline asm, so that the
// compiler's own wait-count tracking stays exact (after an asm statement it
// waits for every LDS read before the next MFMA); the signal fences keep it
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until all of this wave's global loads (direct loads into LDS
// included) have completed.
__device__ __forceinline__ void wait_vm0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The race-detection build's extra synchronisation (nothing otherwise).
__device__ __forceinline__ void debug_stage_sync() {
  if constexpr (FP8BLK_DEBUG_BARRIERS != 0) {
    wait_vm0();
    __syncthreads();
  }
}

// Wait until at most N of this wave's global loads are outstanding (loads
// complete in order, so the older ones have landed). N <= 63.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct global->LDS loads through buffer resources (make_rsrc). A resource
// covers the tile's rows from its first row to the end of the operand (at
// most 4 GB); the hardware range check returns zeros for rows past the end,
// so partial tiles need no clamping. Lane offsets are 32-bit: BM * K < 2^32.
// AUX: the load's cache-policy bits (kStreamAux: non-temporal).
template <int AUX = 0>
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, lds_u8* lds_window) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_window, 16, voff, soff, 0, AUX);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, lds_u8* lds_window) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_window, 4, voff, soff, 0, 0);
}

// Per-lane constants of the direct loads. A load fills one 1 KB LDS window
// (8 rows of 128 bytes); lane l writes slot l = (row l/8, physical chunk
// l%8), so it fetches logical chunk (l%8) ^ key(row): byte offset
// row * K + chunk * 16 within the tile's rows, plus 128 bytes per K step.
// The scalar part of a tile's load plan: where its operands' rows and
// scales start and how many bytes follow them (wave-uniform values).
struct TileBases {
  const void *a, *b, *s;        // first byte of the tile's rows (scales: row or column block)
  uint32_t a_len, b_len, s_len;  // bytes from there to the operand's end (clamped to 4 GB - 1)
  const void* w;                 // PAIR: the weight-scale window's plan
  uint32_t w_len;
  // PAIR: the rows of wave w + WAVES/2 (the tile's second half), with their
  // own resources. The buffer range check covers the VGPR offset only, not
  // the scalar one, so a row distance passed as the scalar offset would let
  // a row past the operand's end through; a resource that starts at the
  // second half's first row puts that row under the check.
  const void *a2, *b2;
  uint32_t a2_len, b2_len;
};

// A tile's load plan: per-lane offsets (they depend only on the lane and
// the row length, so every tile of a launch shares them) and its bases.
template <class C>
struct LoadPlan {
  uint32_t a_off[C::A_WIN], b_off[C::B_WIN], s_off, w_off;
  TileBases t;
};



// Direct loads of K block kb into `stage`; with live == false every
// resource has length zero, so the loads fetch nothing. No branches: the
// loop around this must stay one basic block. The first BM/64 waves load
// the tile's activation scales (64 rows each); the others all load the
// same BN/128 weight scales into the stage's last window.
// `ln` is the plan of the workgroup's next tile (a persistent kernel loads
// that tile's first blocks during the current tile's last steps): with
// cur == false the block comes from it. Two tiles of one launch share the
// per-lane offsets (they depend on the lane and the row length only), so
// only the scalar bases and lengths are selected (no branch).
template <class C>
__device__ __forceinline__ void issue_stage(lds_u8* stage, const LoadPlan<C>& lp, const TileBases& ln, bool cur,
                                            int kb, int wave, bool live) {
  const uint32_t koff = (uint32_t)kb * BK;
  const rsrc_t a = make_rsrc(cur ? lp.t.a : ln.a, live ? (cur ? lp.t.a_len : ln.a_len) : 0u);
  const rsrc_t b = make_rsrc(cur ? lp.t.b : ln.b, live ? (cur ? lp.t.b_len : ln.b_len) : 0u);
  const rsrc_t s = make_rsrc(cur ? lp.t.s : ln.s, live ? (cur ? lp.t.s_len : ln.s_len) : 0u);
#pragma unroll
  for (int i = 0; i < C::A_WIN; ++i) dma16(a, lp.a_off[i], koff, stage + (wave * C::A_WIN + i) * 1024);
#pragma unroll
  for (int i = 0; i < C::B_WIN; ++i)
    dma16<C::B_AUX>(b, lp.b_off[i], koff, stage + C::A_BYTES + (wave * C::B_WIN + i) * 1024);
  // RB: waves past the B windows repeat the last one (same rows, same data)
  const int window = wave < C::BM / 64 ? wave
                     : C::RB ? C::BM / 64 + (wave - C::BM / 64 < C::BN / 64 ? wave - C::BM / 64 : C::BN / 64 - 1)
                             : C::BM / 64;
  dma4(s, lp.s_off, (uint32_t)kb * 4, stage + C::A_BYTES + C::B_BYTES + window * 256);
}

// PAIR: wave w < WAVES/2 issues the loads of its own windows and of wave
// w + WAVES/2's (the same lane offsets into the second half's resources,
// which start a fixed row distance further: the swizzle key repeats every 16
// rows), its activation-scale window and the weight-scale window; the other
// waves issue nothing.
template <class C>
__device__ __forceinline__ void issue_stage_pair(lds_u8* stage, const LoadPlan<C>& lp, const TileBases& ln,
                                                 bool cur, int kb, int wave, bool live) {
  constexpr int H = C::WAVES / 2;
  const uint32_t koff = (uint32_t)kb * BK;
  const rsrc_t a = make_rsrc(cur ? lp.t.a : ln.a, live ? (cur ? lp.t.a_len : ln.a_len) : 0u);
  const rsrc_t b = make_rsrc(cur ? lp.t.b : ln.b, live ? (cur ? lp.t.b_len : ln.b_len) : 0u);
  const rsrc_t s = make_rsrc(cur ? lp.t.s : ln.s, live ? (cur ? lp.t.s_len : ln.s_len) : 0u);
  const rsrc_t w = make_rsrc(cur ? lp.t.w : ln.w, live ? (cur ? lp.t.w_len : ln.w_len) : 0u);
  const rsrc_t a2 = make_rsrc(cur ? lp.t.a2 : ln.a2, live ? (cur ? lp.t.a2_len : ln.a2_len) : 0u);
  const rsrc_t b2 = make_rsrc(cur ? lp.t.b2 : ln.b2, live ? (cur ? lp.t.b2_len : ln.b2_len) : 0u);
#pragma unroll
  for (int i = 0; i < C::A_WIN; ++i) {
    dma16(a, lp.a_off[i], koff, stage + (wave * C::A_WIN + i) * 1024);
    dma16(a2, lp.a_off[i], koff, stage + ((wave + H) * C::A_WIN + i) * 1024);
  }
#pragma unroll
  for (int i = 0; i < C::B_WIN; ++i) {
    dma16<C::B_AUX>(b, lp.b_off[i], koff, stage + C::A_BYTES + (wave * C::B_WIN + i) * 1024);
    dma16<C::B_AUX>(b2, lp.b_off[i], koff, stage + C::A_BYTES + ((wave + H) * C::B_WIN + i) * 1024);
  }
  dma4(s, lp.s_off, (uint32_t)kb * 4, stage + C::A_BYTES + C::B_BYTES + wave * 256);
  // weights: the one weight-scale window; RB: the B-row scales of wave w + WAVES/2
  dma4(w, lp.w_off, (uint32_t)kb * 4, stage + C::A_BYTES + C::B_BYTES + (C::BM / 64 + (C::RB ? wave : 0)) * 256);
}

template <class C>
__device__ __forceinline__ void refill(lds_u8* stage, const LoadPlan<C>& lp, int kb, int wave, bool live) {
  if constexpr (C::PAIR) {
    if (wave < C::WAVES / 2) issue_stage_pair<C>(stage, lp, lp.t, true, kb, wave, live);  // uniform
  } else {
    issue_stage<C>(stage, lp, lp.t, true, kb, wave, live);
  }
}

// acc[j] += p[j] * sc for the TN accumulator quads of one m-subtile.
template <class C>
__device__ __forceinline__ void fold_row(v4f (&acc)[C::TN], const v4f (&p)[C::TN], float sc) {
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(p[j][r], sc, acc[j][r]);
}

// RB: acc[j][r] += p[j][r] * sa * sb[j][r], sb = the scales of the lane's
// output columns 16j + 4g + r.
template <class C>
__device__ __forceinline__ void fold_row_rb(v4f (&acc)[C::TN], const v4f (&p)[C::TN], float sa, const v4f (&sb)[C::TN]) {
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(p[j][r] * sa, sb[j][r], acc[j][r]);
}

// The fold path's MFMAs want the plain product of a block (no block scales).
// With both scale operands the constant 0 the compiler emits the unscaled
// v_mfma_f32_16x16x128_f8f6f4 (there is no separate builtin for it), which
// saves the scale operands' register and measured 1-2% faster than the scaled
// form with unit (127) scales; the GEMM tests compare its results with the
// oracle, so a compiler that treated 0 as the scale 2^-127 would fail them.
constexpr int kNoScale = 0;

template <class C>
__device__ __forceinline__ void mfma_row(v4f (&p)[C::TN], const v8i (&wfr)[C::TN], const v8i& afr) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], afr, zero, 0, 0, 0, kNoScale, 0, kNoScale);
}

// Compiler scheduling fence: nothing is moved across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// A scale the MFMA can apply itself: 0 (an all-zero group or block, whose
// codes are all zero) or an exact power of two 2^-126 .. 2^127 (positive,
// zero mantissa, normal exponent). Its E8M0 code is then the fp32 exponent
// field.
__device__ __forceinline__ bool e8m0_exact(uint32_t b) {  // bitwise, no branches
  const uint32_t e = (b >> 23) & 0xFFu;
  return (b == 0u) | (((b & 0x807FFFFFu) == 0u) & (e != 0u) & (e != 0xFFu));
}
__device__ __forceinline__ uint32_t e8m0_of(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }

__device__ __forceinline__ bool v4_e8m0_exact(v4i v) {
  return e8m0_exact((uint32_t)v[0]) & e8m0_exact((uint32_t)v[1]) & e8m0_exact((uint32_t)v[2]) &
         e8m0_exact((uint32_t)v[3]);
}
__device__ __forceinline__ bool wave_all(bool ok) { return __builtin_amdgcn_ballot_w64(!ok) == 0; }

// Whether every scale of a tile is e8m0_exact, decided once per workgroup:
// wave w checks BM/WAVES of the tile's activation-scale rows (each row's KB
// scales are contiguous, so a wave's share is one run of floats; rows past
// M read as zero) and the last wave also the weight scales of the tile's
// column blocks. The first 1 KB of each share is loaded before the tile's
// first direct loads, so waiting for it leaves those in flight; the rest is
// read only while everything seen so far is a power of two (scales from the
// amax/448 rule almost never are, so most tiles decide on that first 1 KB:
// eight early loads per wave measured ~5000 clocks of tile start-up, most of
// them out of range but still through the address unit). Each wave's
// verdict goes to LDS and is read by all after the barrier that follows the
// first direct loads.
template <class C>
struct ScaleScan {
  static constexpr int ROWS = C::BM / C::WAVES;  // activation-scale rows per wave
  rsrc_t a, w;
  uint32_t a_bytes, w_bytes;
  v4i a0, w0;
};

template <class C>
__device__ __forceinline__ void scan_begin(ScaleScan<C>& sc, const float* sa, const float* sw, int64_t M, int64_t N,
                                           int64_t m0, int64_t n0, int wave, int KB, int lane) {
  using S = ScaleScan<C>;
  const int64_t r0 = m0 + (int64_t)wave * S::ROWS;
  const int64_t rows = M - r0;
  const int64_t a_rows = rows <= 0 ? 0 : (rows < S::ROWS ? rows : S::ROWS);
  sc.a_bytes = (uint32_t)S::ROWS * (uint32_t)KB * 4u;
  sc.a = make_rsrc(sa + r0 * KB, clamp_len(a_rows * KB * 4));
  // last wave: the tile's weight-scale blocks n0/128 .. (n0+BN-1)/128 that exist
  constexpr int kColBlocks = (C::BN + kBlock - 1) / kBlock;
  const int64_t blocks = N / kBlock - n0 / kBlock;
  const int64_t w_blocks = blocks < kColBlocks ? blocks : kColBlocks;
  sc.w_bytes = wave == C::WAVES - 1 ? (uint32_t)(w_blocks * KB * 4) : 0u;
  sc.w = make_rsrc(sw + (n0 / kBlock) * KB, sc.w_bytes);
  sc.a0 = __builtin_amdgcn_raw_buffer_load_b128(sc.a, (uint32_t)lane * 16u, 0, 0);
  sc.w0 = __builtin_amdgcn_raw_buffer_load_b128(sc.w, (uint32_t)lane * 16u, 0, 0);
}

// This wave's verdict (wave-uniform). Loads past a resource's end read as
// zero, which passes. The rest of the share is read only if the first 1 KB
// (and the weight scales' first 1 KB) left the answer open.
template <class C>
__device__ __forceinline__ bool scan_end(const ScaleScan<C>& sc, int lane) {
  const bool ok = wave_all(v4_e8m0_exact(sc.w0) & v4_e8m0_exact(sc.a0));
  if (!ok) return false;  // uniform
  bool rest = true;
  for (uint32_t off = 1024u; off < sc.a_bytes; off += 8192u) {
    v4i v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(sc.a, off + (uint32_t)u * 1024u + (uint32_t)lane * 16u, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) rest = rest & v4_e8m0_exact(v[u]);
  }
  for (uint32_t off = 1024u; off < sc.w_bytes; off += 4096u) {
    v4i v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(sc.w, off + (uint32_t)u * 1024u + (uint32_t)lane * 16u, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) rest = rest & v4_e8m0_exact(v[u]);
  }
  return wave_all(rest);
}

// The K loop of one wave, entered after the barrier that follows block 0's
// arrival (every wave of the workgroup runs the same variant). POW2 == false: each block's 16x16 partials come from
// unit-scale MFMAs and are folded into the fp32 accumulators with one FMA,
// acc += partial * (SA * SW). POW2 == true (every scale of the wave is 0 or
// a power of two): the MFMA applies SW and SA itself as E8M0 block scales
// (source 0 = weights: the wave's SW; source 1 = activations: the lane's
// row's SA) and accumulates into acc directly, with no fold.
// lpn / has_next / s0 (persistent kernels): the refills past block KB - 1
// load the next tile's first blocks (same K) from plan lpn instead of
// nothing, and this tile's block kb lives in stage (kb + s0) mod STAGES
// (s0 carries the stage of the previous tiles' blocks). has_next == false,
// s0 == 0: one tile, the refills past the end fetch nothing.
template <class C, bool POW2, bool LOADER = true>
__device__ __forceinline__ void k_loop(lds_u8* smem, uint8_t* smem_generic, const LoadPlan<C>& lp, int wave, int KB,
                                       int wm, int wn, int g, int c16, v4f (&acc)[C::TM][C::TN],
                                       const TileBases& lpn, bool has_next, int s0) {
  constexpr int S = C::STAGES, LPS = C::LOADS_PER_STAGE;
  // Step kb, one basic block: (1) the previous step's last-row MFMAs, then
  // this stage's weight fragments, first activation fragment and scales are
  // read while they run; (2) rows 0..TM-2, each reading the next row's
  // activation fragment and folding the previous row's partials while its
  // own MFMAs run; (3) wait for this wave's loads of block kb+1 and barrier
  // (every wave has read all of block kb, and block kb+1 is in LDS), then
  // refill block kb's stage with block kb+STAGES. Folds trail their MFMAs by
  // one row, so no fold waits for an MFMA just issued.
  v8i wfr[C::TN], afr[2];
  v4f srow[C::TM / 4];
  float swv = 0.f;
  // RB: B-row scales of the lane's output columns. They are replaced by the
  // new block's right after row 0's fold, the last fold of the previous
  // block (its last two rows fold in (1) and at row 0).
  v4f sbn[C::RB ? C::TN : 1];
#pragma unroll
  for (int j = 0; j < (C::RB ? C::TN : 1); ++j) sbn[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::TN; ++j) wfr[j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  afr[0] = afr[1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  v4f pp[C::TN];  // partials of the previous row, not yet folded
#pragma unroll
  for (int j = 0; j < C::TN; ++j) pp[j] = v4f{0.f, 0.f, 0.f, 0.f};
  float sc_prev = 0.f, sc_last = 0.f;
  uint32_t ew = 0, ea_last = 0;  // E8M0 scales (POW2)
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < KB; ++kb) {
    debug_stage_sync();
    const int st = (kb + s0) % S;
    const uint8_t* sA = smem_generic + st * C::STAGE;
    {  // (1); on the first step the operands are zero
      // The last row's MFMA j is the last use of weight fragment j, so the
      // next block's fragment j is read into it right after: the reads spread
      // over the tail MFMAs, and row 0 can start once its first fragments land.
      v4f p[C::TN];
      afr[0] = read_frag(sA, wm + c16, g);
      const float* sc = reinterpret_cast<const float*>(sA + C::A_BYTES + C::B_BYTES);
#pragma unroll
      for (int q = 0; q < C::TM / 4; ++q) srow[q] = *reinterpret_cast<const v4f*>(sc + wm + c16 * C::TM + 4 * q);
      const float swv_new = C::RB ? 0.f : sc[C::BM + wn / kBlock];
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        if constexpr (POW2)
          acc[C::TM - 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wfr[j], afr[(C::TM - 1) & 1], acc[C::TM - 1][j], 0, 0, 0, (int)ew, 0, (int)ea_last);
        else
          p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], afr[(C::TM - 1) & 1], zero, 0, 0, 0,
                                                                  kNoScale, 0, kNoScale);
        wfr[j] = read_frag(sA + C::A_BYTES, wn + 16 * j + c16, g);
      }
      if constexpr (!POW2) {
        if constexpr (C::RB)
          fold_row_rb<C>(acc[C::TM - 2], pp, sc_prev, sbn);
        else
          fold_row<C>(acc[C::TM - 2], pp, sc_prev);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) pp[j] = p[j];
        sc_prev = sc_last;
      }
      swv = swv_new;
      ew = e8m0_of(swv);
      // first activation fragment and the scales (TM / 4 + 3 reads)
      __builtin_amdgcn_sched_group_barrier(0x100, C::TM / 4 + 2 + (C::RB ? 0 : 1), 0);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // tail MFMA j
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next block's weight fragment j
      }
      sched_fence();
    }
#pragma unroll
    for (int i = 0; i < C::TM - 1; ++i) {  // (2)
      afr[(i + 1) & 1] = read_frag(sA, wm + 16 * (i + 1) + c16, g);
      if constexpr (POW2) {
        const uint32_t ea = e8m0_of(srow[i / 4][i % 4]);
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], afr[i & 1], acc[i][j], 0, 0, 0, (int)ew,
                                                                       0, (int)ea);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next fragment reads
      } else {
        v4f p[C::TN];
        mfma_row<C>(p, wfr, afr[i & 1]);
        if constexpr (C::RB) {
          fold_row_rb<C>(acc[i == 0 ? C::TM - 1 : i - 1], pp, sc_prev, sbn);
          if (i == 0) {  // the previous block's folds are done: this block's B scales
            const float* sc = reinterpret_cast<const float*>(sA + C::A_BYTES + C::B_BYTES);
#pragma unroll
            for (int j = 0; j < C::TN; ++j) sbn[j] = *reinterpret_cast<const v4f*>(sc + C::BM + wn + 16 * j + 4 * g);
          }
        } else {
          fold_row<C>(acc[i == 0 ? C::TM - 1 : i - 1], pp, sc_prev);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) pp[j] = p[j];
        sc_prev = C::RB ? srow[i / 4][i % 4] : srow[i / 4][i % 4] * swv;  // RB: the A scale alone
        if (C::RB && i == 0)
          __builtin_amdgcn_sched_group_barrier(0x100, 2 + C::TN, 0);  // next fragment and the B scales
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next fragment reads
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, C::RB ? 8 : 4, 0);   // its quad's fold
        }
      }
      sched_fence();
    }
    if constexpr (POW2)
      ea_last = e8m0_of(srow[(C::TM - 1) / 4][(C::TM - 1) % 4]);
    else
      sc_last = C::RB ? srow[(C::TM - 1) / 4][(C::TM - 1) % 4] : srow[(C::TM - 1) / 4][(C::TM - 1) % 4] * swv;
    wait_vm<LPS * (C::PAIR ? 2 : 1) * (S - 2)>();  // (3) block kb+1 has landed
    lds_barrier();
    {  // block kb + S of this tile, or block kb + S - KB of the next
      const bool cur = kb + S < KB;
      const int kl = cur ? kb + S : kb + S - KB;
      const bool live = cur | (has_next & (kl < KB));
      if constexpr (!C::PAIR)
        issue_stage<C>(smem + st * C::STAGE, lp, lpn, cur, kl, wave, live);
      else if constexpr (LOADER)
        issue_stage_pair<C>(smem + st * C::STAGE, lp, lpn, cur, kl, wave, live);
    }
    debug_stage_sync();
    sched_fence();
  }
  if constexpr (POW2) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      acc[C::TM - 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], afr[(C::TM - 1) & 1],
                                                                           acc[C::TM - 1][j], 0, 0, 0, (int)ew, 0,
                                                                           (int)ea_last);
  } else {
    v4f p[C::TN];
    mfma_row<C>(p, wfr, afr[(C::TM - 1) & 1]);
    if constexpr (C::RB) {
      fold_row_rb<C>(acc[C::TM - 2], pp, sc_prev, sbn);
      fold_row_rb<C>(acc[C::TM - 1], p, sc_last, sbn);
    } else {
      fold_row<C>(acc[C::TM - 2], pp, sc_prev);
      fold_row<C>(acc[C::TM - 1], p, sc_last);
    }
  }
  // no load may still be writing LDS when the workgroup ends (a next tile's
  // blocks stay in flight: the caller waits for them)
  if (!has_next) wait_vm0();
}

// The scalar bases and lengths of the tile at (m0, n0): its operands'
// rows and scales (rows past M or N fall outside the resources and read as
// zeros). Wave-uniform.
template <class C>
__device__ __forceinline__ void plan_bases(TileBases& t, const uint8_t* qa, const float* sa, const uint8_t* qw,
                                           const float* sw, int64_t M, int64_t N, int64_t m0, int64_t n0, int64_t ld,
                                           int64_t kb0, int wave) {
  const int64_t KBld = ld / BK;  // scales per operand row
  t.a = qa + m0 * ld + kb0 * BK;
  t.b = qw + n0 * ld + kb0 * BK;
  t.a_len = clamp_len((M - m0) * ld - kb0 * BK);
  t.b_len = clamp_len((N - n0) * ld - kb0 * BK);
  if (wave < C::BM / 64) {  // activation scales of the tile's rows
    t.s = sa + m0 * KBld + kb0;
    t.s_len = clamp_len(((M - m0) * KBld - kb0) * 4);
  } else if constexpr (C::RB) {  // B-row scales (sw is SB[N][KB])
    t.s = sw + n0 * KBld + kb0;
    t.s_len = clamp_len(((N - n0) * KBld - kb0) * 4);
  } else {  // weight scales of the tile's column blocks
    t.s = sw + (n0 / kBlock) * KBld + kb0;
    t.s_len = clamp_len(((N / kBlock - n0 / kBlock) * KBld - kb0) * 4);
  }
  if constexpr (C::PAIR && C::RB) {  // B-row scales of tile rows 64w + lane
    t.w = sw + n0 * KBld + kb0;
    t.w_len = clamp_len(((N - n0) * KBld - kb0) * 4);
  } else if constexpr (C::PAIR) {
    t.w = sw + (n0 / kBlock) * KBld + kb0;
    t.w_len = clamp_len(((N / kBlock - n0 / kBlock) * KBld - kb0) * 4);
  }
  if constexpr (C::PAIR) {  // the second half's rows, each range-checked against its operand's end
    constexpr int64_t ha = C::WAVES / 2 * C::A_WIN * 8, hb = C::WAVES / 2 * C::B_WIN * 8;
    t.a2 = qa + (m0 + ha) * ld + kb0 * BK;
    t.b2 = qw + (n0 + hb) * ld + kb0 * BK;
    t.a2_len = clamp_len((M - m0 - ha) * ld - kb0 * BK);
    t.b2_len = clamp_len((N - n0 - hb) * ld - kb0 * BK);
  }
}

// A tile's whole load plan: the per-lane offsets of its direct loads (they
// depend only on the lane and the row length ld) and its bases.
template <class C>
__device__ __forceinline__ void plan_tile(LoadPlan<C>& lp, const uint8_t* qa, const float* sa, const uint8_t* qw,
                                          const float* sw, int64_t M, int64_t N, int64_t m0, int64_t n0, int64_t ld,
                                          int64_t kb0, int wave, int lane) {
  const int64_t KBld = ld / BK;  // scales per operand row
#pragma unroll
  for (int i = 0; i < C::A_WIN; ++i) {
    const int row = (wave * C::A_WIN + i) * 8 + (lane >> 3);
    lp.a_off[i] = (uint32_t)row * (uint32_t)ld + (((lane & 7) ^ swz_key(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::B_WIN; ++i) {
    const int row = (wave * C::B_WIN + i) * 8 + (lane >> 3);
    lp.b_off[i] = (uint32_t)row * (uint32_t)ld + (((lane & 7) ^ swz_key(row)) << 4);
  }
  if (wave < C::BM / 64) {
    // Activation scales, permuted so that the TM scales one lane needs
    // (rows wm + 16i + l%16, i < TM) are contiguous: slot t = h*WM + c*TM + i
    // holds tile row h*WM + 16i + c.
    const int t = wave * 64 + lane, h = t / C::WM, rem = t % C::WM;
    const int row = h * C::WM + 16 * (rem % C::TM) + rem / C::TM;
    lp.s_off = (uint32_t)row * (uint32_t)(KBld * 4);
  } else if constexpr (C::RB) {
    // B-row scales of tile rows bw*64 + lane, in natural order (sw is SB[N][KB])
    const int bw = wave - C::BM / 64 < C::BN / 64 ? wave - C::BM / 64 : C::BN / 64 - 1;
    lp.s_off = (uint32_t)(bw * 64 + lane) * (uint32_t)(KBld * 4);
  } else {  // weight scales of column blocks n0/128 + lane (lanes past the tile's blocks repeat)
    constexpr int kColBlocks = (C::BN + kBlock - 1) / kBlock;  // a 64-wide tile lies in one block
    lp.s_off = (uint32_t)(lane % kColBlocks) * (uint32_t)(KBld * 4);
  }
  lp.w_off = 0u;
  if constexpr (C::PAIR && C::RB) {  // B-row scales of tile rows 64w + lane
    lp.w_off = (uint32_t)(wave * 64 + lane) * (uint32_t)(KBld * 4);
  } else if constexpr (C::PAIR) {
    constexpr int kColBlocks = (C::BN + kBlock - 1) / kBlock;
    lp.w_off = (uint32_t)(lane % kColBlocks) * (uint32_t)(KBld * 4);
  }
  plan_bases<C>(lp.t, qa, sa, qw, sw, M, N, m0, n0, ld, kb0, wave);
}

// bf16 (nearest even) store of a finished tile: lane holds
// Y[m0 + wm + 16i + l%16][n0 + wn + 16j + 4*(l/16) + r], r < 4 (rows N
// long); rows past M are not stored. The caller skips waves whose columns
// are past N.
template <class C>
__device__ __forceinline__ void store_tile(const v4f (&acc)[C::TM][C::TN], uint16_t* __restrict__ y, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int wm, int wn, int g, int c16) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int64_t row = m0 + wm + 16 * i + c16;
    if (row < M) {
      uint16_t* yr = y + row * N + n0 + wn + 4 * g;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const uint32_t lo = (uint32_t)to_bf16_bits(acc[i][j][0]) | ((uint32_t)to_bf16_bits(acc[i][j][1]) << 16);
        const uint32_t hi = (uint32_t)to_bf16_bits(acc[i][j][2]) | ((uint32_t)to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(yr + 16 * j) = make_uint2(lo, hi);
      }
    }
  }
}

// One BM x BN output tile at (m0, n0) of Y[M][N] = A[M][K] W[N][K]^T; rows
// >= M of A and >= N of W read as zeros and are never stored. M >= 1.
//
// The MFMA computes the transposed tile: source 0 is a 16-row weight
// fragment (n), source 1 a 16-row activation fragment (m), so lane l holds
// Y[m = l%16][n = 4*(l/16) + r], r < 4. Each lane therefore needs a single
// activation scale per 16-row m-subtile (16 lanes read 16 consecutive
// floats: no LDS bank conflict), the weight scale is uniform over the
// wave, and the 4 accumulators of a quad are 4 consecutive outputs of one
// row, stored as one 8-byte write.
//
// K is the contraction length of this tile (K / 128 blocks), starting at K
// block kb0 of operand rows ld bytes long (ld / 128 scales per row); the
// plain GEMMs pass ld = K and kb0 = 0, the grouped wgrad an expert's token
// range on the padded token axis (per-row scales only: the weight-block
// scan below assumes ld = K, kb0 = 0).
//
// PARTIAL: the tile's fp32 sums go to part[M][N] (16-byte stores, y is not
// used) and the K loop always folds (the split-K GEMM passes a K range of
// the operands, which the power-of-two scan does not handle).
template <class C, bool PARTIAL = false>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                          const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                          int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
                                          int64_t m0, int64_t n0, uint8_t* smem_generic, int64_t ld, int64_t kb0,
                                          float* __restrict__ part = nullptr) {
  static_assert(C::TM % 4 == 0, "activation fragments alternate between two registers; scales read 4 at a time");
  lds_u8* smem = (lds_u8*)smem_generic;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
  const int wm = (wave / C::WAVES_N) * C::WM;
  const int wn = (wave % C::WAVES_N) * C::WN;
  const int g = lane >> 4, c16 = lane & 15;
  const int KB = __builtin_amdgcn_readfirstlane((int)(K / BK));  // K <= 2^24
  const int64_t KBld = ld / BK;                                   // scales per operand row

  LoadPlan<C> lp;
  plan_tile<C>(lp, qa, sa, qw, sw, M, N, m0, n0, ld, kb0, wave, lane);
  // N % 128 == 0 and WN divides 128: a wave's columns are all in or all out
  const bool cols_valid = n0 + wn < N;

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // STAGES LDS stages, each holding a K block of both operands and its
  // scales; block kb lives in stage kb % STAGES and STAGES-1 blocks are in
  // flight while one is computed. The loop body is branch-free: past the
  // last block the refill uses resources of length zero (out-of-range loads
  // fetch nothing) and the fragments read ahead are not used.
  // PAIR: the loading and the other waves run their own copy of the loop
  // (no branch inside it); loading waves have twice the loads per stage
  const bool loader = !C::PAIR || wave < C::WAVES / 2;
  if constexpr (C::RB || PARTIAL) {
    // per-row scales on both operands, or a K range: always the fold path
#pragma unroll
    for (int b = 0; b < C::STAGES; ++b) refill<C>(smem + b * C::STAGE, lp, b, wave, b < KB);
    wait_vm<C::LOADS_PER_STAGE * (C::PAIR ? 2 : 1) * (C::STAGES - 1)>();  // block 0 has landed
    lds_barrier();
    if (loader)
      k_loop<C, false, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
    else
      k_loop<C, false, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
  } else {
    ScaleScan<C> scan;
    scan_begin<C>(scan, sa, sw, M, N, m0, n0, wave, KB, lane);
#pragma unroll
    for (int b = 0; b < C::STAGES; ++b) refill<C>(smem + b * C::STAGE, lp, b, wave, b < KB);
    uint32_t* verdict = reinterpret_cast<uint32_t*>(smem_generic + C::STAGES * C::STAGE);
    const bool ok = scan_end<C>(scan, lane);
    if (lane == 0) verdict[wave] = ok ? 1u : 0u;
    // block 0 has landed (the scan's later loads too); PAIR: twice the loads per stage
    wait_vm<C::LOADS_PER_STAGE * (C::PAIR ? 2 : 1) * (C::STAGES - 1)>();
    lds_barrier();
    bool pow2 = true;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) pow2 = pow2 & (verdict[w] != 0u);
    if (pow2) {
      if (loader)
        k_loop<C, true, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
      else
        k_loop<C, true, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
    } else {
      if (loader)
        k_loop<C, false, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
      else
        k_loop<C, false, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, lp.t, false, 0);
    }
  }

  if (!cols_valid) return;
  // lane holds Y[m0 + wm + 16i + l%16][n0 + wn + 16j + 4*(l/16) + r], r < 4 (Y rows N long)
  if constexpr (PARTIAL) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int64_t row = m0 + wm + 16 * i + c16;
      if (row < M) {
        float* pr = part + row * N + n0 + wn + 4 * g;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) *reinterpret_cast<v4f*>(pr + 16 * j) = acc[i][j];
      }
    }
    return;
  }
  store_tile<C>(acc, y, M, N, m0, n0, wm, wn, g, c16);
}

// Tile order: blocks are dealt to XCDs round-robin (block b runs on XCD
// b % 8); renumber so each XCD sees a contiguous range, then walk that
// range in bands of GROUP_M tile rows so that concurrently running tiles
// share A rows and B columns.
__device__ __forceinline__ void tile_of_block(int64_t bid, int64_t nblocks, int64_t m_tiles, int64_t n_tiles,
                                              int64_t& m_tile, int64_t& n_tile) {
  int64_t lid = bid;
  if (nblocks % 8 == 0) lid = (bid % 8) * (nblocks / 8) + bid / 8;
  const int64_t per_group = (int64_t)FP8BLK_GEMM_GROUP_M * n_tiles;
  const int64_t group = lid / per_group;
  const int64_t first_m = group * FP8BLK_GEMM_GROUP_M;
  const int64_t rows = m_tiles - first_m < FP8BLK_GEMM_GROUP_M ? m_tiles - first_m : FP8BLK_GEMM_GROUP_M;
  const int64_t in_group = lid % per_group;
  m_tile = first_m + in_group % rows;
  n_tile = in_group / rows;
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                       const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                       int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
                                                       int64_t m_tiles, int64_t n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS];
  int64_t m_tile, n_tile;
  tile_of_block(blockIdx.x, gridDim.x, m_tiles, n_tiles, m_tile, n_tile);
  gemm_tile<Cfg>(qa, sa, qw, sw, M, N, K, y, m_tile * Cfg::BM, n_tile * Cfg::BN, smem, K, 0);
}

// Split-K GEMM for few rows (M <= BM: one row tile): workgroup b computes
// column tile b / splits over K blocks [s KB / splits, (s+1) KB / splits),
// s = b % splits, and writes its fp32 sums to part[s][M][N].
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_splitk_kernel(const uint8_t* __restrict__ qa,
                                                              const float* __restrict__ sa,
                                                              const uint8_t* __restrict__ qw,
                                                              const float* __restrict__ sw, int64_t M, int64_t N,
                                                              int64_t K, float* __restrict__ part, int splits) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS];
  const int n_tile = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (uint32_t)splits));
  const int split = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (uint32_t)splits));
  const int64_t KB = K / BK;
  const int64_t kb_lo = KB * split / splits, kb_hi = KB * (split + 1) / splits;
  gemm_tile<Cfg, true>(qa, sa, qw, sw, M, N, (kb_hi - kb_lo) * BK, nullptr, 0, (int64_t)n_tile * Cfg::BN, smem, K,
                       kb_lo, part + (int64_t)split * M * N);
}

// y = bf16(sum over s of part[s]), s in order (the result does not depend on
// timing); 4 outputs per thread, M * N a multiple of 4.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const v4f* __restrict__ part, int splits, int64_t n4,
                                                            uint2* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  v4f sum = part[i];
  for (int s = 1; s < splits; ++s) sum += part[(int64_t)s * n4 + i];
  const uint32_t lo = (uint32_t)to_bf16_bits(sum[0]) | ((uint32_t)to_bf16_bits(sum[1]) << 16);
  const uint32_t hi = (uint32_t)to_bf16_bits(sum[2]) | ((uint32_t)to_bf16_bits(sum[3]) << 16);
  y[i] = make_uint2(lo, hi);
}

// Expert ranges come from the device offsets clamped to [0, total_M]
// (expert_tile), so offsets that break their contract give wrong values,
// never a read outside qa/sa or a write outside y.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void grouped_gemm_kernel(const uint8_t* __restrict__ qa,
                                                               const float* __restrict__ sa,
                                                               const uint8_t* __restrict__ qw,
                                                               const float* __restrict__ sw,
                                                               const int32_t* __restrict__ offsets, int E,
                                                               int64_t total_M, int64_t N, int64_t K,
                                                               uint16_t* __restrict__ y, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS];
  // uniform (readfirstlane): the division runs on the vector unit
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / n_tiles));
  const int n_tile = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % n_tiles));
  int e = 0, tile = 0;
  const int found = __builtin_amdgcn_readfirstlane((int)locate_tile<Cfg::BM>(offsets, E, t, e, tile));
  e = __builtin_amdgcn_readfirstlane(e);
  tile = __builtin_amdgcn_readfirstlane(tile);
  if (!found) return;  // uniform over the workgroup
  // uniform (readfirstlane): they size the buffer resources of every K step
  int64_t row0, rows, m0;
  if (!expert_tile(__builtin_amdgcn_readfirstlane(offsets[e]), __builtin_amdgcn_readfirstlane(offsets[e + 1]),
                   total_M, tile, Cfg::BM, row0, rows, m0))
    return;  // uniform
  const int64_t KB = K / BK;
  gemm_tile<Cfg>(qa + row0 * K, sa + row0 * KB, qw + (int64_t)e * N * K, sw + (int64_t)e * (N / kBlock) * KB,
                 rows, N, K, y + row0 * N, m0, (int64_t)n_tile * Cfg::BN, smem, K, 0);
}

// The expert-grouped GEMM's tile `v` (M-tile v / n_tiles of the concatenated
// per-expert tile lists, column tile v % n_tiles): its expert and rows
// (expert_tile's clamped range). False when the tile list is shorter or the
// tile holds no row. All values uniform.
struct GroupTile {
  int e;
  int64_t row0, rows, m0, n0;
};
template <class Cfg>
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ offsets, int E, int64_t total_M, int n_tiles,
                                             int64_t v, GroupTile& gt, bool& past_end) {
  const int t = __builtin_amdgcn_readfirstlane((int)(v / n_tiles));
  const int n_tile = __builtin_amdgcn_readfirstlane((int)(v % n_tiles));
  int e = 0, tile = 0;
  const int found = __builtin_amdgcn_readfirstlane((int)locate_tile<Cfg::BM>(offsets, E, t, e, tile));
  past_end = !found;  // tile lists are concatenated: no later M-tile exists either
  if (!found) return false;
  gt.e = __builtin_amdgcn_readfirstlane(e);
  if (!expert_tile(__builtin_amdgcn_readfirstlane(offsets[gt.e]), __builtin_amdgcn_readfirstlane(offsets[gt.e + 1]),
                   total_M, __builtin_amdgcn_readfirstlane(tile), Cfg::BM, gt.row0, gt.rows, gt.m0))
    return false;
  gt.n0 = (int64_t)n_tile * Cfg::BN;
  return true;
}

// The next live tile at or after v, stepping by `stride` (false: none).
template <class Cfg>
__device__ __forceinline__ bool next_grouped_tile(const int32_t* __restrict__ offsets, int E, int64_t total_M,
                                                  int n_tiles, int64_t vtiles, int64_t stride, int64_t& v,
                                                  GroupTile& gt) {
  for (; v < vtiles; v += stride) {
    bool past_end = false;
    if (grouped_tile<Cfg>(offsets, E, total_M, n_tiles, v, gt, past_end)) return true;
    if (past_end) break;
  }
  return false;
}

// Persistent expert-grouped GEMM: workgroup b computes the live tiles
// b, b + G, b + 2G, ... of the same tile space as grouped_gemm_kernel (G =
// the grid), one after another, and loads each next tile's first K blocks
// during the current tile's last steps, so the next tile does not start by
// waiting for its operands (MoE layers have short K loops: 6 K blocks for a
// 768-wide down projection, where the start of a tile otherwise took about
// as long as its K loop). The fold path is used for every tile (no
// power-of-two scan: it would wait for the prefetched blocks).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void grouped_gemm_persistent_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, int E, int64_t total_M, int64_t N, int64_t K,
    uint16_t* __restrict__ y, int n_tiles, int64_t vtiles) {
  using C = Cfg;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_generic[Cfg::LDS];
  lds_u8* smem = (lds_u8*)smem_generic;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave / C::WAVES_N) * C::WM;
  const int wn = (wave % C::WAVES_N) * C::WN;
  const int g = lane >> 4, c16 = lane & 15;
  const int KB = __builtin_amdgcn_readfirstlane((int)(K / BK));
  const int64_t KBs = K / BK;  // scales per row
  const int64_t stride = gridDim.x;
  const bool loader = !C::PAIR || wave < C::WAVES / 2;

  int64_t v = blockIdx.x;
  GroupTile cur;
  if (!next_grouped_tile<Cfg>(offsets, E, total_M, n_tiles, vtiles, stride, v, cur)) return;  // uniform
  LoadPlan<C> lp;
  plan_tile<C>(lp, qa + cur.row0 * K, sa + cur.row0 * KBs, qw + (int64_t)cur.e * N * K,
               sw + (int64_t)cur.e * (N / kBlock) * KBs, cur.rows, N, cur.m0, cur.n0, K, 0, wave, lane);
#pragma unroll
  for (int b = 0; b < C::STAGES; ++b) refill<C>(smem + b * C::STAGE, lp, b, wave, b < KB);
  int s0 = 0;
  for (;;) {
    // the next tile (its expert lookup overlaps this tile's loads in flight)
    int64_t vn = v + stride;
    GroupTile nxt = cur;
    const bool has_next = next_grouped_tile<Cfg>(offsets, E, total_M, n_tiles, vtiles, stride, vn, nxt);
    TileBases nb;  // (the current tile's when there is no next: then nothing is loaded from it)
    plan_bases<C>(nb, qa + nxt.row0 * K, sa + nxt.row0 * KBs, qw + (int64_t)nxt.e * N * K,
                  sw + (int64_t)nxt.e * (N / kBlock) * KBs, nxt.rows, N, nxt.m0, nxt.n0, K, 0, wave);
    v4f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // Every memory operation of this wave has completed: this tile's first
    // blocks (the first tile's issued above, later tiles' during the
    // previous loop) and the previous tile's stores. The vector memory
    // counter counts stores too, and waves whose columns are past N store
    // nothing, so a partial count would not tell every wave that its share
    // of block 0 has landed; waiting for all is exact for every wave (and
    // measured as fast as an exact count with counted buffer stores).
    wait_vm0();
    lds_barrier();
    if (loader)
      k_loop<C, false, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
    else
      k_loop<C, false, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
    if (cur.n0 + wn < N)  // N % 128 == 0 and WN divides 128: a wave's columns are all in or all out
      store_tile<C>(acc, y + cur.row0 * N, cur.rows, N, cur.m0, cur.n0, wm, wn, g, c16);
    if (!has_next) break;  // uniform; k_loop waited for every load
    s0 = (s0 + KB) % C::STAGES;
    lp.t = nb;
    cur = nxt;
    v = vn;
  }
}

// Persistent dense GEMM: a grid of as many workgroups as the CUs hold at
// once; workgroup b (dealt to XCD b % 8) walks its XCD's contiguous range of
// tile numbers in steps of the XCD's workgroup count, each number placed by
// the same banded order as gemm_kernel's, so the tiles running together
// on an XCD at any time are neighbours as there. During a tile's last steps
// its refills load the next tile's first K blocks, so a tile starts on
// landed operands instead of a full memory latency (with one 256x256
// workgroup per CU nothing else on the CU covers that start). The
// power-of-two scan of each tile runs at its start, after the previous
// tile's K loop.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_persistent_kernel(const uint8_t* __restrict__ qa,
                                                                  const float* __restrict__ sa,
                                                                  const uint8_t* __restrict__ qw,
                                                                  const float* __restrict__ sw, int64_t M, int64_t N,
                                                                  int64_t K, uint16_t* __restrict__ y, int64_t m_tiles,
                                                                  int64_t n_tiles) {
  using C = Cfg;
  static_assert(!C::RB, "row-scaled tiles take gemm_kernel");
  __shared__ __attribute__((aligned(1024))) uint8_t smem_generic[Cfg::LDS];
  lds_u8* smem = (lds_u8*)smem_generic;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave / C::WAVES_N) * C::WM;
  const int wn = (wave % C::WAVES_N) * C::WN;
  const int g = lane >> 4, c16 = lane & 15;
  const int KB = __builtin_amdgcn_readfirstlane((int)(K / BK));
  const bool loader = !C::PAIR || wave < C::WAVES / 2;
  // tile numbers x * per_xcd .. of XCD x = b % 8, in steps of the XCD's
  // gridDim.x / 8 workgroups (the grid is a multiple of 8)
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t per_xcd = (tiles + 7) / 8;
  const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8, step = gridDim.x / 8;
  auto tile_at = [&](int64_t i, int64_t& m0, int64_t& n0) {  // false: no i-th tile
    const int64_t within = i * step + slot;
    const int64_t lid = xcd * per_xcd + within;
    if (within >= per_xcd || lid >= tiles) return false;
    const int64_t per_group = (int64_t)FP8BLK_GEMM_GROUP_M * n_tiles;
    const int64_t first_m = lid / per_group * FP8BLK_GEMM_GROUP_M;
    const int64_t rows = m_tiles - first_m < FP8BLK_GEMM_GROUP_M ? m_tiles - first_m : FP8BLK_GEMM_GROUP_M;
    const int64_t in_group = lid % per_group;
    m0 = (first_m + in_group % rows) * C::BM;
    n0 = in_group / rows * C::BN;
    return true;
  };

  int64_t i = 0, m0 = 0, n0 = 0;
  if (!tile_at(0, m0, n0)) return;  // uniform
  uint32_t* verdict = reinterpret_cast<uint32_t*>(smem_generic + C::STAGES * C::STAGE);
  ScaleScan<C> scan;
  scan_begin<C>(scan, sa, sw, M, N, m0, n0, wave, KB, lane);
  LoadPlan<C> lp;
  plan_tile<C>(lp, qa, sa, qw, sw, M, N, m0, n0, K, 0, wave, lane);
#pragma unroll
  for (int b = 0; b < C::STAGES; ++b) refill<C>(smem + b * C::STAGE, lp, b, wave, b < KB);
  int s0 = 0;
  for (;;) {
    int64_t nm0 = m0, nn0 = n0;
    const bool has_next = tile_at(i + 1, nm0, nn0);
    TileBases nb;  // (the current tile's when there is no next: then nothing is loaded from it)
    plan_bases<C>(nb, qa, sa, qw, sw, M, N, nm0, nn0, K, 0, wave);
    v4f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
      for (int b = 0; b < C::TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
    const bool ok = scan_end<C>(scan, lane);
    if (lane == 0) verdict[wave] = ok ? 1u : 0u;
    // this tile's first blocks have landed (and, after the first tile, the
    // previous tile's stores are done: see the grouped persistent kernel)
    wait_vm0();
    lds_barrier();
    bool pow2 = true;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) pow2 = pow2 & (verdict[w] != 0u);
    // (every wave has read the verdicts before any wave's next write: the K
    // loop passes a barrier per block)
    if (pow2) {
      if (loader)
        k_loop<C, true, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
      else
        k_loop<C, true, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
    } else {
      if (loader)
        k_loop<C, false, true>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
      else
        k_loop<C, false, false>(smem, smem_generic, lp, wave, KB, wm, wn, g, c16, acc, nb, has_next, s0);
    }
    if (n0 + wn < N)  // N % 128 == 0 and WN divides 128: a wave's columns are all in or all out
      store_tile<C>(acc, y, M, N, m0, n0, wm, wn, g, c16);
    if (!has_next) break;  // uniform; k_loop waited for every load
    s0 = (s0 + KB) % C::STAGES;
    lp.t = nb;
    m0 = nm0;
    n0 = nn0;
    ++i;
    scan_begin<C>(scan, sa, sw, M, N, m0, n0, wave, KB, lane);
  }
}

// Grouped wgrad: dW_e [N][K] = the row-scaled product of rows of A = Q(dY^T)
// [N][ld] and B = Q(X^T) [K][ld] over expert e's 128-token blocks of the
// padded token axis (they start at block tiles_before<128>(offsets, e)).
// One workgroup per (expert, output tile). Expert ranges are clamped to the
// ld / 128 blocks of the operands, so offsets that break their contract give
// wrong values, never an access outside the buffers.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void grouped_rowscaled_kernel(const uint8_t* __restrict__ qa,
                                                                    const float* __restrict__ sa,
                                                                    const uint8_t* __restrict__ qb,
                                                                    const float* __restrict__ sb,
                                                                    const int32_t* __restrict__ offsets, int64_t ld,
                                                                    int64_t N, int64_t K, uint16_t* __restrict__ y,
                                                                    int tiles_per_expert, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS];
  const int e = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / tiles_per_expert));
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % tiles_per_expert));
  const int64_t lb = ld / BK;
  int64_t kb0 = tiles_before<BK>(offsets, e);
  kb0 = kb0 < 0 ? 0 : (kb0 > lb ? lb : kb0);
  int64_t kbn = tile_count(__builtin_amdgcn_readfirstlane(offsets[e]), __builtin_amdgcn_readfirstlane(offsets[e + 1]),
                           BK);
  kbn = kbn > lb - kb0 ? lb - kb0 : kbn;
  gemm_tile<Cfg>(qa, sa, qb, sb, N, K, kbn * BK, y + (int64_t)e * N * K, (int64_t)(t / n_tiles) * Cfg::BM,
                 (int64_t)(t % n_tiles) * Cfg::BN, smem, ld, kb0);
}

fp8blk_status check_gemm_args(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, const uint16_t* y) {
  if (M < 0 || N <= 0 || K <= 0) return FP8BLK_ERR_INVALID_ARG;
  if (N % kBlock || K % kBlock || K > kMaxK) return FP8BLK_ERR_SHAPE;
  if (M == 0) return FP8BLK_OK;
  if (!qa || !sa || !qw || !sw || !y) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(y, 16) || !aligned(sa, 4) || !aligned(sw, 4))
    return FP8BLK_ERR_ALIGNMENT;
  return FP8BLK_OK;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

namespace fp8blk {
namespace {

constexpr int64_t kCUs = 256;  // MI355X compute units
constexpr int64_t kPersistentMaxKB = 64;  // K blocks per tile up to which the dense GEMM walks tiles

// Workgroups of a tile configuration one CU holds at once (LDS-bound).
template <class Cfg>
constexpr int64_t per_cu() {
  return (160 * 1024) / Cfg::LDS;
}

template <class Cfg>
fp8blk_status launch_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, int64_t M,
                          int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int64_t n_tiles = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t m_tiles = (M + Cfg::BM - 1) / Cfg::BM;
  if (n_tiles * m_tiles > (1 << 24)) return FP8BLK_ERR_SHAPE;
  // The persistent kernel when every workgroup walks at least three tiles
  // and the tiles are short (at most 64 K blocks), where a tile's start is
  // a noticeable share of it. Interleaved A/B on the Llama-3.1-8B prefill
  // linears (bitwise equal outputs): K = 4096 +2.6 to +3.3%, the K = 14336
  // down projection 3.5% slower (four tiles per workgroup: the static walk
  // balances worse than the hardware's dispatch), Qwen3-8B qkv with 1.5
  // tiles per workgroup 1.6% slower.
  if constexpr (!Cfg::RB && FP8BLK_GEMM_PERSISTENT) {
    const int64_t slots = kCUs * per_cu<Cfg>();
    if (n_tiles * m_tiles >= 3 * slots && K / BK >= Cfg::STAGES && K / BK <= kPersistentMaxKB) {
      hipLaunchKernelGGL(gemm_persistent_kernel<Cfg>, dim3((uint32_t)slots), dim3(Cfg::NT), 0, stream, qa, sa, qw,
                         sw, M, N, K, y, m_tiles, n_tiles);
      return launch_status();
    }
  }
  hipLaunchKernelGGL(gemm_kernel<Cfg>, dim3((uint32_t)(n_tiles * m_tiles)), dim3(Cfg::NT), 0, stream, qa, sa, qw,
                     sw, M, N, K, y, m_tiles, n_tiles);
  return launch_status();
}

// Cfg, or its streamed-weights twin CfgS when each weight block is read by
// at most kStreamMaxRowTiles row tiles.
template <class Cfg, class CfgS>
fp8blk_status launch_gemm_policy(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, int64_t M,
                                 int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if ((M + Cfg::BM - 1) / Cfg::BM <= kStreamMaxRowTiles)
    return launch_gemm<CfgS>(qa, sa, qw, sw, M, N, K, y, stream);
  return launch_gemm<Cfg>(qa, sa, qw, sw, M, N, K, y, stream);
}

// More tiles than the CUs hold at once (and at least STAGES K blocks): the
// persistent kernel (each workgroup walks its tiles with the next tile's
// first blocks prefetched); otherwise one workgroup per tile, which keeps
// the power-of-two scan.
template <class Cfg>
fp8blk_status launch_grouped(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                             const int32_t* offsets, int64_t E, int64_t total_M, int64_t N, int64_t K, uint16_t* y,
                             hipStream_t stream) {
  const int64_t n_tiles = (N + Cfg::BN - 1) / Cfg::BN;
  // upper bound on the number of M-tiles: sum_e ceil(M_e/BM) <= total_M/BM + E
  const int64_t m_tiles = total_M / Cfg::BM + E;
  const int64_t vtiles = n_tiles * m_tiles;
  if (vtiles > (1 << 24)) return FP8BLK_ERR_SHAPE;
  const int64_t slots = kCUs * per_cu<Cfg>();
  // the persistent kernel loads a next tile's first STAGES blocks during the
  // current tile's last STAGES steps: it needs at least STAGES K blocks
  if (vtiles > slots && K / BK >= Cfg::STAGES) {
    hipLaunchKernelGGL(grouped_gemm_persistent_kernel<Cfg>, dim3((uint32_t)slots), dim3(Cfg::NT), 0, stream, qa, sa,
                       qw, sw, offsets, (int)E, total_M, N, K, y, (int)n_tiles, vtiles);
  } else {
    hipLaunchKernelGGL(grouped_gemm_kernel<Cfg>, dim3((uint32_t)vtiles), dim3(Cfg::NT), 0, stream, qa, sa, qw, sw,
                       offsets, (int)E, total_M, N, K, y, (int)n_tiles);
  }
  return launch_status();
}

template <class Cfg>
int64_t tiles_of(int64_t M, int64_t N) {
  return ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
}

// K ranges of fp8blk_gemm_ws: 0 (the plain path) unless the rows fit one
// 256-row tile, its 256x128 column tiles are too few to fill the CUs and K
// is long (at least 64 blocks); then as many ranges as give about one
// workgroup per CU, each at least 8 K blocks long. Measured against the
// plain path at 256 rows: K = 14336 and 28672 gain 25-40%, K = 4096 loses
// (the fp32 partials, S * M * N * 4 bytes written and read back, then
// outweigh the weights).
int64_t splitk_count(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > Skinny::BM || N <= 0 || K <= 0 || N % kBlock || K % kBlock || K > kMaxK) return 0;
  const int64_t n_tiles = N / Skinny::BN, kb = K / kBlock;
  if (n_tiles >= kCUs * 3 / 4 || kb < 64) return 0;  // the plain path is faster
  const int64_t s = std::min<int64_t>(kCUs / n_tiles, kb / 8);
  return s >= 2 ? s : 0;
}

}  // namespace
}  // namespace fp8blk

// At most 256 rows with at least 3/4 of the CUs' worth of 256x128 tiles:
// Skinny. Otherwise the largest tile that still gives every CU at least two
// workgroups' worth of tiles; below that, the smallest.
extern "C" fp8blk_status fp8blk_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                                     int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const fp8blk_status st = check_gemm_args(qa, sa, qw, sw, M, N, K, y);
  if (st != FP8BLK_OK || M == 0) return st;
  if (M <= Skinny::BM && tiles_of<Skinny>(M, N) >= kCUs * 3 / 4)  // one row tile: weights streamed
    return launch_gemm<SkinnyS>(qa, sa, qw, sw, M, N, K, y, stream);
  if (tiles_of<Big>(M, N) >= kCUs) return launch_gemm_policy<Big, BigS>(qa, sa, qw, sw, M, N, K, y, stream);
  if (tiles_of<Mid>(M, N) >= 2 * kCUs) return launch_gemm_policy<Mid, MidS>(qa, sa, qw, sw, M, N, K, y, stream);
  return launch_gemm_policy<Small, SmallS>(qa, sa, qw, sw, M, N, K, y, stream);
}

extern "C" size_t fp8blk_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  const int64_t s = splitk_count(M, N, K);
  return s ? (size_t)(s * M * N) * sizeof(float) : 0;
}

namespace fp8blk {
namespace {

// The split-K path: `splits` K ranges over 256x128 tiles write their fp32
// sums to part[splits][M][N] (every element of each range's slice is
// written, so part needs no clearing); a second kernel adds the ranges in
// order and rounds to bf16.
fp8blk_status launch_splitk(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, int64_t M,
                            int64_t N, int64_t K, uint16_t* y, float* part, int64_t splits, hipStream_t stream) {
  const int64_t n_tiles = N / SkinnyS::BN;  // one row tile: weights streamed
  hipLaunchKernelGGL(gemm_splitk_kernel<SkinnyS>, dim3((uint32_t)(n_tiles * splits)), dim3(SkinnyS::NT), 0, stream, qa,
                     sa, qw, sw, M, N, K, part, (int)splits);
  const fp8blk_status ls = launch_status();
  if (ls != FP8BLK_OK) return ls;
  const int64_t n4 = M * N / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)((n4 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const v4f*>(part), (int)splits, n4, reinterpret_cast<uint2*>(y));
  return launch_status();
}

// Scratch of fp8blk_gemm_noalloc: the split-K partials in a static device
// array, so the call allocates nothing. Each GPU the library runs on holds
// its own copy until the process ends. Host code must not pass `scratch`
// itself to a kernel (on the host the name stands for a host-side shadow,
// not a device address): its device address is looked up once per device
// and kept in scratch_ptr.
static_assert(FP8BLK_GEMM_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) float scratch[FP8BLK_GEMM_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 256;
std::atomic<float*> scratch_ptr[kMaxDevices];
std::mutex scratch_mutex;

// The device address of the current device's scratch array (hipGetSymbolAddress
// with that device current, once per device; no allocation).
fp8blk_status current_scratch(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8BLK_ERR_HIP;
  float* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mutex);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return FP8BLK_ERR_HIP;
      p = static_cast<float*>(addr);
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8BLK_OK;
}

}  // namespace
}  // namespace fp8blk

// Few rows and few column tiles: the K loop is cut into splitk_count ranges
// over 256x128 tiles, whose fp32 sums go to the workspace; a second kernel
// adds them in range order and rounds to bf16. Otherwise fp8blk_gemm.
extern "C" fp8blk_status fp8blk_gemm_ws(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                                        int64_t M, int64_t N, int64_t K, uint16_t* y, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  const fp8blk_status st = check_gemm_args(qa, sa, qw, sw, M, N, K, y);
  if (st != FP8BLK_OK || M == 0) return st;
  const int64_t splits = splitk_count(M, N, K);
  if (!workspace || splits == 0) return fp8blk_gemm(qa, sa, qw, sw, M, N, K, y, stream);
  if (!aligned(workspace, 16)) return FP8BLK_ERR_ALIGNMENT;
  if (workspace_bytes < fp8blk_gemm_workspace_size(M, N, K)) return FP8BLK_ERR_INVALID_ARG;
  return launch_splitk(qa, sa, qw, sw, M, N, K, y, static_cast<float*>(workspace), splits, stream);
}

// fp8blk_gemm_ws with the library's static scratch as the workspace: the
// same kernels, the same split count, so the same bits. The size check and
// every argument check come before the first HIP call.
extern "C" fp8blk_status fp8blk_gemm_noalloc(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                                             int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const fp8blk_status st = check_gemm_args(qa, sa, qw, sw, M, N, K, y);
  if (st != FP8BLK_OK || M == 0) return st;
  const int64_t splits = splitk_count(M, N, K);
  if (splits == 0) return fp8blk_gemm(qa, sa, qw, sw, M, N, K, y, stream);
  if (fp8blk_gemm_workspace_size(M, N, K) > (size_t)FP8BLK_GEMM_SCRATCH_BYTES) return FP8BLK_ERR_SCRATCH;
  float* part = nullptr;
  const fp8blk_status ps = current_scratch(&part);
  if (ps != FP8BLK_OK) return ps;
  return launch_splitk(qa, sa, qw, sw, M, N, K, y, part, splits, stream);
}

// Expert groups: 256-row tiles when the average expert has at least 256
// rows and K >= 2048, 128-row tiles when it has at least 128, else 64-row
// tiles (less padding in partly filled tiles).
extern "C" fp8blk_status fp8blk_gemm_rowscaled(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                               const float* sb, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                               hipStream_t stream) {
  const fp8blk_status st = check_gemm_args(qa, sa, qb, sb, M, N, K, y);
  if (st != FP8BLK_OK || M == 0) return st;
  if (tiles_of<BigRB>(M, N) >= kCUs) return launch_gemm<BigRB>(qa, sa, qb, sb, M, N, K, y, stream);
  if (tiles_of<MidRB>(M, N) >= 2 * kCUs) return launch_gemm<MidRB>(qa, sa, qb, sb, M, N, K, y, stream);
  return launch_gemm<SmallRB>(qa, sa, qb, sb, M, N, K, y, stream);
}

// Expert-grouped wgrad (row scales on both operands): the tile from the
// output's tile count, as for fp8blk_gemm_rowscaled.
extern "C" fp8blk_status fp8blk_grouped_gemm_rowscaled(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                                       const float* sb, const int32_t* offsets, int64_t E,
                                                       int64_t ld, int64_t N, int64_t K, uint16_t* y,
                                                       hipStream_t stream) {
  if (E < 1 || ld < 0 || N <= 0 || K <= 0) return FP8BLK_ERR_INVALID_ARG;
  if (N % kBlock || K % kBlock || ld % kBlock || ld > kMaxK || E > INT32_MAX - 1) return FP8BLK_ERR_SHAPE;
  if (!qa || !sa || !qb || !sb || !offsets || !y) return FP8BLK_ERR_INVALID_ARG;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(y, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      !aligned(offsets, 4))
    return FP8BLK_ERR_ALIGNMENT;
  auto launch = [&](auto cfg) {
    using Cfg = decltype(cfg);
    const int64_t n_tiles = K / Cfg::BN + (K % Cfg::BN != 0);
    const int64_t per = (N / Cfg::BM + (N % Cfg::BM != 0)) * n_tiles;
    if (per * E > INT32_MAX) return FP8BLK_ERR_SHAPE;
    hipLaunchKernelGGL(grouped_rowscaled_kernel<Cfg>, dim3((uint32_t)(per * E)), dim3(Cfg::NT), 0, stream, qa, sa,
                       qb, sb, offsets, ld, N, K, y, (int)per, (int)n_tiles);
    return launch_status();
  };
  if (tiles_of<BigRB>(N, K) * E >= kCUs) return launch(BigRB{});
  if (tiles_of<MidRB>(N, K) * E >= 2 * kCUs) return launch(MidRB{});
  return launch(SmallRB{});
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
  // 256x256 tiles (with the paired refill loads) when the average expert
  // fills one and K is long enough to amortise their start: measured on the
  // Qwen3-30B-A3B routing, +7% at K = 2048 and 6144, -6% at K = 768
  // weights streamed when experts average at most kStreamMaxRowTiles row tiles
  if (total_M >= 256 * E && K >= 2048)
    return total_M <= kStreamMaxRowTiles * Big::BM * E
               ? launch_grouped<BigS>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream)
               : launch_grouped<Big>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream);
  if (total_M >= 128 * E)
    return total_M <= kStreamMaxRowTiles * Mid::BM * E
               ? launch_grouped<MidS>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream)
               : launch_grouped<Mid>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream);
  return total_M <= kStreamMaxRowTiles * Small::BM * E
             ? launch_grouped<SmallS>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream)
             : launch_grouped<Small>(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream);
}
