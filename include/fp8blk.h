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
 * identical outputs (sums in a fixed order; the only atomics are the
 * order-independent maxima of fp8blk_qkv_amax).
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
  FP8BLK_ERR_HIP = 4,         /* a kernel launch (or a device query) failed */
  FP8BLK_ERR_SCRATCH = 5      /* the call needs more than the library's static scratch */
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
 * fp8blk_gemm with a caller-owned workspace that lets few-row problems with
 * a long contraction (M <= 256, too few 256x128 column tiles to fill the
 * CUs, K >= 8192: a decode step's down projection, the dgrad of a wide
 * linear) split the K loop: each of S K ranges (S from M, N, K) writes its
 * fp32 sums of the same y formula to the workspace, and a second kernel on
 * the same stream adds the S ranges in order and rounds to bf16. The result
 * is within the same accumulation tolerance as fp8blk_gemm's (it adds the
 * same products in another order) and the same call always gives the same
 * bits.
 *   arguments as fp8blk_gemm, plus
 *   workspace    NULL, or device memory of at least
 *                fp8blk_gemm_workspace_size(M, N, K) bytes (16-byte aligned,
 *                owned by the caller, contents undefined on entry and exit).
 *                Calls that share a workspace must be ordered on one stream.
 * With a NULL workspace, or when the size query gives 0, the call is exactly
 * fp8blk_gemm. A workspace smaller than the size query's value is
 * FP8BLK_ERR_INVALID_ARG.
 */
fp8blk_status fp8blk_gemm_ws(const uint8_t* qa, const float* sa,
                             const uint8_t* qw, const float* sw,
                             int64_t M, int64_t N, int64_t K, uint16_t* y,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Workspace bytes fp8blk_gemm_ws uses for (M, N, K) (host only, no HIP
 * call): S * M * N * 4 when it splits K into S ranges, else 0 (also for
 * invalid shapes). Never more than 256 rows x 32768 columns x 4 bytes
 * (32 MiB): the split count times the column count is at most 256 column
 * tiles of 128.
 */
size_t fp8blk_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/* Bytes of the static device scratch behind fp8blk_gemm_noalloc (32 MiB). */
#define FP8BLK_GEMM_SCRATCH_BYTES (32u << 20)

/*
 * fp8blk_gemm_ws for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments as fp8blk_gemm (no workspace), same kernels, same split
 * count and therefore the same bits as fp8blk_gemm_ws with a workspace; the
 * split-K partials live in a static device array of
 * FP8BLK_GEMM_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine. The first call on each device
 * looks the array's device address up (hipGetSymbolAddress with that device
 * current; make that first call outside graph capture) and keeps it.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's partials (each call writes every partial it reads, so nothing is
 * cleared): calls on one device that overlap in time (unordered streams,
 * several host threads) race and give undefined results; order them on one
 * stream. Returns FP8BLK_ERR_SCRATCH (before any HIP call) if the split
 * needs more than FP8BLK_GEMM_SCRATCH_BYTES, which the present split rule
 * never does; FP8BLK_ERR_HIP if the address lookup fails.
 */
fp8blk_status fp8blk_gemm_noalloc(const uint8_t* qa, const float* sa,
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
 * Backward GEMMs of a linear layer Y = X W^T (FP8 training in Megatron Core:
 * upppp.jp, «FP8適用の難所：数値のズレ問題»; greentreeone.com, «Технический
 * прорыв»). The pages describe the forward recipe only; here each backward
 * GEMM quantizes its operands along its own contraction dimension:
 *   dgrad  dX = dY W:   fp8blk_quant_act(dY) (1x128 groups along N) and
 *          fp8blk_quant_weight_t(W) (the 128x128 blocks, transposed), then
 *          fp8blk_gemm(Q(dY), S(dY), QW^T, SW^T, M, K, N, dX);
 *   wgrad  dW = dY^T X: fp8blk_quant_act_t of dY and of X (128x1 groups: 128
 *          consecutive tokens of one column), then
 *          fp8blk_gemm_rowscaled(Q(dY^T), S, Q(X^T), S, N, K, M, dW).
 */

/*
 * 128x1 quantisation, written transposed: the 1x128 group quantisation of
 * X^T. For each column k and token block b, the 128 values
 * x[128b .. 128b+127][k] form one group (scale rule as fp8blk_quant_act).
 *   x  [M][K] bf16 in (16-byte aligned)
 *   qt [K][M] E4M3 codes out (16-byte aligned): qt[k][m] codes x[m][k]
 *   st [K][M/128] fp32 scales out
 *   M >= 0 (0: no-op), M % 128 == 0, K > 0 and K % 64 == 0, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_quant_act_t(const uint16_t* x, int64_t M, int64_t K,
                                 uint8_t* qt, float* st, int pow2, hipStream_t stream);

/*
 * 128x128 weight quantisation written transposed: the same blocks, codes and
 * scales as fp8blk_quant_weight, in the layout the dgrad GEMM reads.
 *   w  [N][K] bf16 in (16-byte aligned)
 *   qt [K][N] E4M3 codes out: qt[k][n] codes w[n][k] (16-byte aligned)
 *   st [K/128][N/128] fp32 scales out: st[j][i] is the scale of block (i, j)
 *   N >= 0 (0: no-op), N % 128 == 0, K > 0 and K % 128 == 0, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_quant_weight_t(const uint16_t* w, int64_t N, int64_t K,
                                    uint8_t* qt, float* st, int pow2, hipStream_t stream);

/*
 * GEMM with per-row scales on both operands (the wgrad GEMM):
 *   y[m][n] = bf16( sum_b sa[m][b] * sb[n][b] *
 *                   sum_{k in block b} E4M3(qa[m][k]) * E4M3(qb[n][k]) )
 *   qa [M][K] codes, sa [M][K/128]; qb [N][K] codes, sb [N][K/128] (one
 *   scale per row and K block, e.g. from fp8blk_quant_act_t)
 *   y  [M][N] bf16 out (16-byte aligned)
 *   M >= 0 (M == 0: no-op), N > 0, K > 0, N % 128 == 0, K % 128 == 0,
 *   K <= 2^24.
 */
fp8blk_status fp8blk_gemm_rowscaled(const uint8_t* qa, const float* sa,
                                    const uint8_t* qb, const float* sb,
                                    int64_t M, int64_t N, int64_t K,
                                    uint16_t* y, hipStream_t stream);

/*
 * Backward GEMMs of the expert-grouped layer (rows sorted by expert,
 * offsets[E+1] int32 on the device as for fp8blk_grouped_gemm; weights
 * [E][N][K]), the dense rules per expert:
 *   dgrad  dX_e = dY_e W_e: fp8blk_quant_act(dY), fp8blk_quant_weight_t_grouped
 *          (W) -> [E][K][N], then fp8blk_grouped_gemm(..., E, M, K, N, dX);
 *   wgrad  dW_e = dY_e^T X_e over expert e's tokens: fp8blk_quant_act_t_grouped
 *          of dY and of X, then fp8blk_grouped_gemm_rowscaled.
 * Reading for ragged experts (the pages are silent): the 128x1 groups start
 * at each expert's first token and an expert's last group is completed with
 * zero rows (zeros change neither the maximum nor the sums). The transposed
 * operands live on a padded token axis of ld columns where expert e owns
 * columns pad[e] .. pad[e+1], pad[e] = sum_{e' < e} ceil(M_e' / 128) * 128;
 * ld >= pad[E] (M + 127 E always suffices, rounded up to a multiple of 128).
 * Offsets are device data and not checked (nondecreasing, offsets[0] = 0,
 * offsets[E] = M): when they break this the results are undefined, but no
 * kernel reads or writes outside the buffers sized from M, E and ld.
 */

/*
 * fp8blk_quant_weight_t for each matrix of a stack: w [E][N][K] -> qt
 * [E][K][N], st [E][K/128][N/128]. 1 <= E <= 65535; otherwise as
 * fp8blk_quant_weight_t (which is this with E = 1).
 */
fp8blk_status fp8blk_quant_weight_t_grouped(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                                            uint8_t* qt, float* st, int pow2, hipStream_t stream);

/*
 * 128x1 quantisation of x [M][K] (rows sorted by expert) per expert, written
 * transposed on the padded token axis: for expert e and its j-th group of
 * 128 rows (offsets[e] + 128j ..), qt[k][pad[e] + 128j + i] codes
 * x[offsets[e] + 128j + i][k] for the expert's rows and 0 past them, and
 * st[k][pad[e]/128 + j] is the group's scale. Columns past pad[E] are not
 * written.
 *   x [M][K] bf16 (16-byte aligned); qt [K][ld] codes (16-byte aligned);
 *   st [K][ld/128] fp32; offsets [E+1] int32 (device)
 *   M >= 0 (0: no-op), K % 64 == 0, ld % 128 == 0, E >= 1, pow2 in {0, 1}.
 */
fp8blk_status fp8blk_quant_act_t_grouped(const uint16_t* x, int64_t M, int64_t K,
                                         const int32_t* offsets, int64_t E, int64_t ld,
                                         uint8_t* qt, float* st, int pow2, hipStream_t stream);

/*
 * Grouped wgrad GEMM: for each expert e,
 *   y[e][n][k] = bf16( sum over e's blocks b of sa[n][b] * sb[k][b] *
 *                      sum_{t in block b} E4M3(qa[n][t]) * E4M3(qb[k][t]) )
 * over the blocks pad[e]/128 .. pad[e+1]/128 of the padded token axis (an
 * expert without tokens gets zeros).
 *   qa [N][ld] codes, sa [N][ld/128]; qb [K][ld] codes, sb [K][ld/128]
 *   (fp8blk_quant_act_t_grouped of dY and X); offsets [E+1] int32 (device)
 *   y  [E][N][K] bf16 out (16-byte aligned)
 *   E >= 1, N > 0, K > 0, N, K and ld multiples of 128, ld <= 2^24.
 */
fp8blk_status fp8blk_grouped_gemm_rowscaled(const uint8_t* qa, const float* sa,
                                            const uint8_t* qb, const float* sb,
                                            const int32_t* offsets, int64_t E, int64_t ld,
                                            int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

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

/*
 * FP8 KV cache (upppp.jp, «KVキャッシュとAttentionにも拡張»; greentreeone.com,
 * «Реальные прирост производительности»): the KV cache is stored in FP8, and
 * because the policy's weights change every training step, the Q, K and V
 * scales are recomputed from BF16 activations at the end of each step for
 * the next rollout. The pages give no granularity; this library keeps one
 * scale per tensor (Q, K, V of one attention layer) with the linear layers'
 * rule (s = amax/448 in fp32, or the power-of-two option).
 *
 * Recalibration, step 1: running maxima of |Q|, |K|, |V| over the chunks of
 * a calibration batch.
 *   qkv  [T][(Hq + 2*Hkv)*D] bf16 in: the qkv projection's output, each row
 *        laid out [Q heads (Hq*D) | K heads (Hkv*D) | V heads (Hkv*D)]
 *        (16-byte aligned)
 *   amax [3] fp32 in/out (device): |Q|, |K|, |V| maxima; reset = 1 sets them
 *        to 0 first (the batch's first chunk), reset = 0 folds this chunk
 *        into them. The result does not depend on the order of the work
 *        (max is exact and order-independent).
 *   T >= 0 (T == 0 only applies reset), Hq, Hkv >= 1, D >= 1 and D % 8 == 0.
 */
fp8blk_status fp8blk_qkv_amax(const uint16_t* qkv, int64_t T, int64_t Hq, int64_t Hkv,
                              int64_t D, float* amax, int reset, hipStream_t stream);

/*
 * Recalibration, step 2: scale[i] = the scale rule applied to amax[i]
 * (device arrays of n fp32; amax 0 gives scale 0), pow2 in {0, 1}.
 */
fp8blk_status fp8blk_kv_scales(const float* amax, int64_t n, float* scale, int pow2,
                               hipStream_t stream);

/*
 * KV-cache quantize-and-write: for each token t with 0 <= slot[t] <
 * num_slots, head h of its K row goes to page slot[t] / block_size, panel h,
 * row slot[t] % block_size of the paged cache:
 *   k_cache[slot[t] / block_size][h][slot[t] % block_size][d]
 *       = E4M3(RN_fp32(k[t][h*D + d] / k_scale[0])),
 * and likewise v into v_cache with v_scale[0]. Codes saturate at +-448
 * (tokens may exceed the calibrated range); a zero scale writes +-0. Tokens
 * with a negative slot (padding) or one past the cache write nothing.
 *   k, v    [T][ld] bf16 in, the first Hkv*D columns of each row used (so
 *           they may point into a qkv projection output: ld = (Hq+2Hkv)*D)
 *           (16-byte aligned, ld % 8 == 0, ld >= Hkv*D)
 *   slot    [T] int64 (device)
 *   k_scale, v_scale: one fp32 each (device), e.g. from fp8blk_kv_scales
 *   k_cache, v_cache [num_slots / block_size][Hkv][block_size][D] E4M3
 *           codes (16-byte aligned): pages of block_size tokens, head-major
 *           within a page, so the rows of one KV head in a page are
 *           contiguous (what the decode attention reads)
 *   num_slots a multiple of block_size (whole pages), Hkv*D < 2^31
 *   The slots of one call must be distinct (else which token lands is
 *   unspecified). T >= 0 (0: no-op), Hkv >= 1, D >= 1 and D % 8 == 0,
 *   block_size >= 1.
 */
fp8blk_status fp8blk_kv_cache_write(const uint16_t* k, const uint16_t* v, int64_t ld, int64_t T,
                                    int64_t Hkv, int64_t D, const int64_t* slot, int64_t num_slots,
                                    int64_t block_size, const float* k_scale, const float* v_scale,
                                    uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream);

/*
 * FP8 decode attention over the paged FP8 KV cache (upppp.jp,
 * «KVキャッシュとAttentionにも拡張»: with long outputs the KV cache and
 * attention dominate rollout time, and both run in FP8; greentreeone.com,
 * «Реальные прирост производительности»). Each sequence's new query token
 * attends over its cached tokens:
 *   q8 = E4M3(RN_fp32(q / q_scale)) (as the cache write quantizes K and V)
 *   s[h][t] = (sum_d q8[h][d] * k8[t][g][d]) * q_scale * k_scale * sm_scale,
 *             g = h / (Hq / Hkv)
 *   out[h][d] = bf16( sum_t softmax_t(s[h])[t] * v8[t][g][d] * v_scale )
 * with the softmax and the weighted sum in fp32 (each probability enters the
 * weighted sum as an fp16 head plus an fp16 remainder, about 2^-22 relative).
 *   q            [B][ldq] bf16: the first Hq*D values of row b are sequence b's
 *                query heads (so q may point into a qkv projection output)
 *   k_cache, v_cache [num_slots / block_size][Hkv][block_size][D] E4M3
 *                codes, head-major pages (fp8blk_kv_cache_write);
 *                num_slots a multiple of block_size, num_slots*Hkv < 2^31
 *   block_table  [B][max_blocks] int32 (device): token t of sequence b is
 *                row t % block_size of page block_table[b][t / block_size]
 *                (slot block_table[b][t / block_size] * block_size + t % block_size)
 *   context_lens [B] int32 (device): cached tokens per sequence
 *   q_scale, k_scale, v_scale: one fp32 each (device)
 *   sm_scale     softmax scale (1/sqrt(D) for standard attention)
 *   out          [B][ldo] bf16 out: Hq heads x D per row (16-byte aligned)
 *   split_tokens 0 (the library picks) or a multiple of 256: tokens per chunk
 *                when the context is split (see workspace)
 *   workspace    NULL: one workgroup per (sequence, KV head) covers the whole
 *                context and writes out directly. Otherwise device memory of
 *                at least fp8blk_decode_attention_workspace_size(...) bytes
 *                (16-byte aligned, owned by the caller, contents undefined on
 *                entry and exit): each context is cut into chunks of
 *                split_tokens tokens processed in parallel, their fp32
 *                partials (maximum, sum, unnormalized output per head) are
 *                kept here and merged by a second kernel on the same stream.
 *                Calls that share a workspace must be ordered on one stream.
 *   D == 128; Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8}; ldq and ldo
 *   multiples of 8 and >= Hq*D; B >= 0 (0: no-op); block_size, max_blocks >= 1.
 * Tokens whose block index is past max_blocks, whose block id is negative or
 * whose slot is past num_slots are skipped; a sequence without tokens gives
 * zeros. A workspace smaller than the size query's value is
 * FP8BLK_ERR_INVALID_ARG.
 */
fp8blk_status fp8blk_decode_attention(const uint16_t* q, int64_t ldq, int64_t B, int64_t Hq,
                                      int64_t Hkv, int64_t D, const uint8_t* k_cache,
                                      const uint8_t* v_cache, int64_t num_slots,
                                      const int32_t* block_table, int64_t max_blocks,
                                      int64_t block_size, const int32_t* context_lens,
                                      const float* q_scale, const float* k_scale,
                                      const float* v_scale, float sm_scale,
                                      uint16_t* out, int64_t ldo, int64_t split_tokens,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * Workspace bytes fp8blk_decode_attention needs with these arguments for the
 * split path (host only, no HIP call). 0 when the context is not split (the
 * block table addresses at most one chunk) or the arguments are invalid.
 * The chunk count depends only on B, Hkv, max_blocks * block_size and
 * split_tokens, never on the context lengths.
 */
size_t fp8blk_decode_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                              int64_t max_blocks, int64_t block_size,
                                              int64_t split_tokens);

/*
 * FP8 prefill attention over the paged FP8 KV cache (upppp.jp,
 * «KVキャッシュとAttentionにも拡張»; greentreeone.com, «Реальные прирост
 * производительности»): a prompt's (or a prompt chunk's) new tokens attend
 * causally over the cache. Sequence b's n_b = cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] new tokens are the last n_b of its context_lens[b] cached
 * tokens (their K and V already written by fp8blk_kv_cache_write), so new
 * token i sits at position p = context_lens[b] - n_b + i and attends to
 * cached tokens 0..p (the decode step is n_b = 1):
 *   q8 = E4M3(RN_fp32(q / q_scale)) (as the cache write quantizes K and V)
 *   s[h][t] = (sum_d q8[h][d] * k8[t][g][d]) * q_scale * k_scale * sm_scale,
 *             g = h / (Hq / Hkv), t <= p
 *   out[h][d] = bf16( sum_t softmax_t(s[h])[t] * v8[t][g][d] * v_scale )
 * with the softmax and the sums in fp32 (the probabilities enter the
 * weighted sum to within fp32 accuracy, unquantized).
 *   q            [total_q][ldq] bf16: row cu_seqlens_q[b] + i holds new token
 *                i of sequence b, its Hq query heads in the first Hq*D values
 *                (q may point into a qkv projection output)
 *   total_q      rows of q and of out (host); rows past it are never touched
 *   cu_seqlens_q [B+1] int32 (device): cu_seqlens_q[0] = 0, nondecreasing,
 *                cu_seqlens_q[B] <= total_q (not checked: offsets that break
 *                this give wrong rows, never an access outside q or out)
 *   max_seqlen_q a host bound on n_b (tokens past it are not computed)
 *   k_cache, v_cache, num_slots, block_table, max_blocks, block_size,
 *   context_lens, q_scale, k_scale, v_scale, sm_scale: as for
 *                fp8blk_decode_attention (tokens whose block is out of the
 *                table, negative or past num_slots are skipped)
 *   out          [total_q][ldo] bf16 out: Hq heads x D per row of a new
 *                token (16-byte aligned); other rows are left untouched
 *   D == 128; Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8}; ldq and ldo
 *   multiples of 8 and >= Hq*D; B >= 0, total_q >= 0 and max_seqlen_q >= 0
 *   (any of them 0: no-op); block_size, max_blocks >= 1. A new token whose
 *   position is negative (n_b > context_lens[b]) attends to nothing: zeros.
 */
fp8blk_status fp8blk_prefill_attention(const uint16_t* q, int64_t ldq, int64_t total_q, int64_t B,
                                       int64_t Hq, int64_t Hkv, int64_t D,
                                       const int32_t* cu_seqlens_q, int64_t max_seqlen_q,
                                       const uint8_t* k_cache, const uint8_t* v_cache,
                                       int64_t num_slots, const int32_t* block_table,
                                       int64_t max_blocks, int64_t block_size,
                                       const int32_t* context_lens, const float* q_scale,
                                       const float* k_scale, const float* v_scale, float sm_scale,
                                       uint16_t* out, int64_t ldo, hipStream_t stream);

/* Static, NUL-terminated description of a status code (host memory). */
const char* fp8blk_status_string(fp8blk_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
