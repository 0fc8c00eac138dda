"""Block-scaled FP8 GEMM for the oracle (test infrastructure only).

The greentreeone.com NeMo RL article, section «Технический прорыв», says the
linear layers do their math in FP8 on the quantised operands (W8A8). Readings
taken where it is silent: Y = X W^T with W stored [N, K] (no bias, no
activation); each 128-wide slice b of the reduction dimension is one scale
block, so

    Y[m, n] = sum_b SA[m, b] * SW[n // 128, b] * sum_{k in b} dec(QA[m, k]) * dec(QW[n, k])

computed here exactly up to the final float64 additions; the GPU keeps fp32
accumulators and writes bf16, and is judged against this with the tolerance
|y - y_ref| <= 2**-7 * |y_ref| + 1e-3 * rms(y_ref).

Mixture-of-experts (upppp.jp «まとめ»; greentreeone.com «Реальные прирост
производительности»): rows sorted by expert, offsets[e] .. offsets[e+1] use
expert e's weights.

Pins (tests/test_oracle_gemm.py): exact rational brute force with
``fractions`` on tiny shapes; a closed-form integer case; agreement between
the block-wise form (``gemm_ref``) and the dequantised BLAS form
(``gemm_ref_blas``); zero blocks contribute exactly zero; doubling one row's
scales doubles that output row; the grouped form reduces to the plain GEMM
for a single expert and to exact brute force on a tiny routed case.
"""

import numpy as np

from .e4m3 import decode
from .quant import GROUP


def dequant_act(q, s):
    """dec(Q[M, K]) * S[M, K/128], float64 (exact: 4-bit times 24-bit)."""
    d = decode(q)
    m, k = d.shape
    return (d.reshape(m, k // GROUP, GROUP)
            * np.asarray(s, np.float64)[:, :, None]).reshape(m, k)


def dequant_weight(q, s):
    """dec(Q[N, K]) * S[N/128, K/128] broadcast over 128x128 blocks, float64."""
    d = decode(q)
    n, k = d.shape
    s = np.asarray(s, np.float64)
    return (d.reshape(n // GROUP, GROUP, k // GROUP, GROUP)
            * s[:, None, :, None]).reshape(n, k)


def _check_shapes(qa, sa, qw, sw):
    m, k = qa.shape
    n, k2 = qw.shape
    if k != k2 or k % GROUP or n % GROUP:
        raise ValueError("gemm oracle: need QA[M,K], QW[N,K], K and N multiples of 128")
    if sa.shape != (m, k // GROUP) or sw.shape != (n // GROUP, k // GROUP):
        raise ValueError("gemm oracle: scale shapes do not match")


def gemm_ref(qa, sa, qw, sw):
    """Block-wise form: per K-block exact integer-grid dot products, then
    scaled by SA[m, b] * SW[n // 128, b] and summed over blocks. float64 [M, N].

    Each inner sum is exact in float64: every product of two decoded codes is
    a multiple of 2**-18 of magnitude at most 448**2 < 2**18, so 128 of them
    sum to an integer multiple of 2**-18 below 2**25, i.e. at most 43 bits.
    """
    qa = np.asarray(qa, np.uint8)
    qw = np.asarray(qw, np.uint8)
    sa = np.asarray(sa, np.float32)
    sw = np.asarray(sw, np.float32)
    _check_shapes(qa, sa, qw, sw)
    m, k = qa.shape
    n = qw.shape[0]
    da = decode(qa)
    dw = decode(qw)
    sw_rows = np.repeat(sw.astype(np.float64), GROUP, axis=0)  # [N, K/128]
    y = np.zeros((m, n), dtype=np.float64)
    for b in range(k // GROUP):
        cols = slice(b * GROUP, (b + 1) * GROUP)
        partial = da[:, cols] @ dw[:, cols].T                  # exact
        y += (sa[:, b].astype(np.float64)[:, None] * sw_rows[:, b][None, :]) * partial
    return y


def gemm_ref_blas(qa, sa, qw, sw):
    """Dequantised form: (dec(QA) * SA) @ (dec(QW) * SW)^T in float64."""
    qa = np.asarray(qa, np.uint8)
    qw = np.asarray(qw, np.uint8)
    sa = np.asarray(sa, np.float32)
    sw = np.asarray(sw, np.float32)
    _check_shapes(qa, sa, qw, sw)
    return dequant_act(qa, sa) @ dequant_weight(qw, sw).T


def gemm_rows_ref(qa_rows, sa_rows, qw_block_rows, sw_block_rows):
    """``gemm_ref`` on a subset: some activation rows against some whole
    128-row weight blocks (their QW rows and their SW block rows). Used for
    sampled checks of outputs too large for the full oracle."""
    return gemm_ref(qa_rows, sa_rows, qw_block_rows, sw_block_rows)


def grouped_gemm_ref(qa, sa, qw, sw, offsets):
    """Expert-grouped GEMM: rows offsets[e] .. offsets[e+1]-1 of (QA, SA)
    against expert e's (QW[e], SW[e]). QW is [E, N, K], SW [E, N/128, K/128],
    offsets int [E+1] nondecreasing from 0 to total rows. float64 [sum M_e, N].
    """
    qa = np.asarray(qa, np.uint8)
    qw = np.asarray(qw, np.uint8)
    offsets = np.asarray(offsets, dtype=np.int64)
    e_count, n, _ = qw.shape
    if offsets.shape != (e_count + 1,) or offsets[0] != 0 or offsets[-1] != qa.shape[0]:
        raise ValueError("grouped gemm oracle: offsets must be [E+1] from 0 to total rows")
    if np.any(np.diff(offsets) < 0):
        raise ValueError("grouped gemm oracle: offsets must be nondecreasing")
    y = np.zeros((qa.shape[0], n), dtype=np.float64)
    for e in range(e_count):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = gemm_ref(qa[lo:hi], np.asarray(sa)[lo:hi], qw[e], np.asarray(sw)[e])
    return y


def tolerance_ok(y, y_ref, rms=None):
    """Acceptance test for a bf16 GEMM output against the oracle.

    Elementwise |y - y_ref| <= 2**-7 * |y_ref| + 1e-3 * rms(y_ref), with rms
    over the whole output of the call unless given. Returns (ok, worst) where
    worst is the largest ratio |y - y_ref| / bound (<= 1 passes).
    """
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rms
    err = np.abs(y - y_ref)
    if y.size == 0:
        return True, 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio))
    return bool(np.all(np.isfinite(y)) and worst <= 1.0), worst
