/*
 * fp8blk.h -- C ABI of libfp8blk.so: block-scaled FP8 (E4M3) W8A8 linear
 * layers on AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the greentreeone.com article "NVIDIA NeMo RL
 * достигает ускорения на 48% благодаря сквозному обучению с точностью FP8",
 * section «Технический прорыв»: linear layers run on FP8 E4M3 operands
 * quantised in 128x128 blocks (weights) and 1x128 groups (activations).
 * The power-of-two scale option comes from the upppp.jp NeMo RL FP8 article,
 * section «設定方法» (and the greentreeone.com article, «Почему это важно для
 * экономики ИИ»); the mixture-of-experts use from upppp.jp «まとめ».
 *
 * Readings where the pages are silent (fixed by this library):
 *   - E4M3 is the OCP variant (max 448, no infinities, NaN = S.1111.111);
 *     codes are written as uint8_t, round-to-nearest-even, saturating at
 *     +-448, never NaN; the sign of zero is kept.
 *   - scale s = amax / 448 rounded to fp32 (pow2 = 0), or the smallest power
 *     of two with 448 * s >= amax (pow2 = 1); an all-zero group/block has
 *     s = 0. s is the dequantisation multiplier: x ~ dec(q) * s.
 *   - q = E4M3(RN_fp32(x / s)): the IEEE fp32 quotient, then the E4M3
 *     rounding.
 *   - Y = X W^T with W stored [N][K] row-major; every 128-wide slice of K is
 *     one scale block; fp32 accumulation; output bf16 (round to nearest even).
 *
 * Data types at the boundary: bf16 is passed as uint16_t bit patterns, E4M3
 * as uint8_t codes, scales as IEEE float. Every matrix is row-major and
 * dense (leading dimension = number of columns).
 *
 * Ownership and execution: the caller allocates and owns every buffer (all
 * pointers are device pointers unless stated). A call validates its
 * arguments on the host, enqueues its kernels on `stream` and returns; it
 * never allocates, frees, copies to or from the host, or synchronises. The
 * library keeps no state: concurrent calls on different streams are safe.
 * Inputs and outputs must not overlap. Identical inputs give bitwise
 * identical outputs (no atomics, fixed reduction order).
 *
 * Errors: every argument check happens before any HIP call, so a rejected
 * call has no effect. Device-side faults surface at the caller's next
 * synchronisation. Behaviour is undefined for non-finite inputs and for
 * grouped-GEMM offsets that are not nondecreasing from 0 to total_M.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BLK_OK = 0,
  FP8BLK_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad flag */
  FP8BLK_ERR_SHAPE = 2,       /* K or N not a multiple of 128, GEMM K > 2^24, E < 1 */
  FP8BLK_ERR_ALIGNMENT = 3,   /* data pointer not 16-byte aligned, scales not 4-byte */
  FP8BLK_ERR_HIP = 4          /* a kernel launch failed */
} fp8blk_status;

/* Number of elements of one activation group / weight block edge. */
#define FP8BLK_BLOCK 128

/*
 * 1x128 activation quantisation (greentreeone.com, «Технический прорыв»).
 *   x  [M][K] bf16 in (16-byte aligned)
 *   q  [M][K] E4M3 codes out (16-byte aligned)
 *   s  [M][K/128] fp32 scales out (4-byte aligned); s[m][g] covers
 *      x[m][128g .. 128g+127]
 *   M >= 0 (M == 0: no-op), K > 0 and K % 128 == 0, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_quant_act(const uint16_t* x, int64_t M, int64_t K,
                               uint8_t* q, float* s, int pow2, hipStream_t stream);

/*
 * 128x128 weight quantisation (greentreeone.com, «Технический прорыв»).
 *   w  [N][K] bf16 in (nn.Linear layout, 16-byte aligned)
 *   q  [N][K] E4M3 codes out (16-byte aligned)
 *   s  [N/128][K/128] fp32 scales out; s[i][j] covers rows 128i.., columns 128j..
 *   N >= 0 (N == 0: no-op), N % 128 == 0, K > 0 and K % 128 == 0, pow2 in {0, 1}.
 * An expert stack [E][N][K] with N % 128 == 0 is quantised as one [E*N][K]
 * matrix; its scales are then [E][N/128][K/128].
 */
fp8blk_status fp8blk_quant_weight(const uint16_t* w, int64_t N, int64_t K,
                                  uint8_t* q, float* s, int pow2, hipStream_t stream);

/*
 * Block-scaled GEMM (greentreeone.com, «Технический прорыв»: FP8 math in the
 * linear layers):
 *   y[m][n] = bf16( sum_b sa[m][b] * sw[n/128][b] *
 *                   sum_{k in block b} E4M3(qa[m][k]) * E4M3(qw[n][k]) )
 *   qa [M][K] codes, sa [M][K/128]  -- as written by fp8blk_quant_act
 *   qw [N][K] codes, sw [N/128][K/128] -- as written by fp8blk_quant_weight
 *   y  [M][N] bf16 out (16-byte aligned)
 *   M >= 0 (M == 0: no-op), N > 0, K > 0, N % 128 == 0, K % 128 == 0,
 *   K <= 2^24 (the kernels address a 256-row tile with 32-bit offsets).
 */
fp8blk_status fp8blk_gemm(const uint8_t* qa, const float* sa,
                          const uint8_t* qw, const float* sw,
                          int64_t M, int64_t N, int64_t K,
                          uint16_t* y, hipStream_t stream);

/*
 * Expert-grouped block-scaled GEMM for mixture-of-experts layers (upppp.jp,
 * «まとめ»; greentreeone.com, «Реальные прирост производительности»): rows
 * offsets[e] .. offsets[e+1]-1 of (qa, sa) are multiplied by expert e's
 * weights (qw + e*N*K, sw + e*(N/128)*(K/128)) exactly as in fp8blk_gemm.
 *   qa [total_M][K], sa [total_M][K/128]: rows sorted by expert
 *   qw [E][N][K], sw [E][N/128][K/128]
 *   offsets: DEVICE int32 [E+1], offsets[0] = 0, nondecreasing,
 *            offsets[E] = total_M (not checked; read on the device only, so
 *            the call needs no host synchronisation); empty experts allowed
 *   y  [total_M][N] bf16 out
 *   E >= 1, total_M >= 0 (0: no-op), N, K > 0, N % 128 == 0, K % 128 == 0,
 *   K <= 2^24.
 */
fp8blk_status fp8blk_grouped_gemm(const uint8_t* qa, const float* sa,
                                  const uint8_t* qw, const float* sw,
                                  const int32_t* offsets, int64_t E, int64_t total_M,
                                  int64_t N, int64_t K,
                                  uint16_t* y, hipStream_t stream);

/*
 * Fused producers: the bf16 input of a linear layer is computed and quantised
 * in one pass, so it is never written to and read back from HBM. Both pages
 * count the quantisation kernels as overhead and name kernel fusion as the
 * remedy (upppp.jp, «重要度サンプリングで精度を保つ»; greentreeone.com,
 * «Реальные прирост производительности»), and keep normalisation and the
 * nonlinearities in bf16 (greentreeone.com, «Технический прорыв»).
 *
 * Each call computes the producer in fp32, rounds every value once to bf16
 * (nearest, ties to even), and quantises exactly those bf16 values as
 * fp8blk_quant_act does: (q, s) equal fp8blk_quant_act applied to the bf16
 * values, bit for bit. If y is not NULL the bf16 values are also written
 * there (for a consumer that needs them unquantised); y may be NULL.
 * Results that overflow bf16 are undefined, like non-finite inputs.
 */

/*
 * RMSNorm + 1x128 quantisation, the input of the qkv and gate_up linears:
 *   v[m][k] = bf16( x[m][k] * r[m] * gamma[k] ),
 *   r[m]    = 1 / sqrt( (sum_k x[m][k]^2) / K + eps )   (fp32)
 *   x     [M][K] bf16 in (16-byte aligned)
 *   gamma [K]    bf16 in (16-byte aligned)
 *   eps   finite, >= 0 (with eps == 0 an all-zero row has no defined result)
 *   q [M][K] codes, s [M][K/128] scales out: as fp8blk_quant_act of v
 *   y [M][K] bf16 out (v itself), or NULL (16-byte aligned if not NULL)
 *   M >= 0 (M == 0: no-op), K > 0 and K % 128 == 0, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_rmsnorm_quant_act(const uint16_t* x, const uint16_t* gamma, float eps,
                                       int64_t M, int64_t K, uint8_t* q, float* s,
                                       uint16_t* y, int pow2, hipStream_t stream);

/*
 * SiLU(gate) * up + 1x128 quantisation, the input of the down linear:
 *   h[m][f] = bf16( g / (1 + exp(-g)) * u ),  g = gu[m][f], u = gu[m][F + f]
 *   gu [M][2F] bf16 in: each row is [gate (F) | up (F)], the gate_up
 *      linear's output with gate and up weights stacked in that order
 *      (16-byte aligned)
 *   q [M][F] codes, s [M][F/128] scales out: as fp8blk_quant_act of h
 *   y [M][F] bf16 out (h itself), or NULL (16-byte aligned if not NULL)
 *   M >= 0 (M == 0: no-op), F > 0 and F % 128 == 0, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_silu_mul_quant_act(const uint16_t* gu, int64_t M, int64_t F,
                                        uint8_t* q, float* s, uint16_t* y, int pow2,
                                        hipStream_t stream);

/* Static, NUL-terminated description of a status code (host memory). */
const char* fp8blk_status_string(fp8blk_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
