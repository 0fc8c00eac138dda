"""Backward block-FP8 GEMMs of a linear layer (test infrastructure only, see
the package docstring).

Sources: FP8 training runs in Megatron Core (upppp.jp NeMo RL FP8 article,
«FP8適用の難所：数値のズレ問題»; greentreeone.com article, «Технический
прорыв»: linear layers in FP8 with 128x128 weight blocks and 1x128
activation groups). The pages describe the forward recipe only; for the
backward pass of Y = X W^T the plainest reading keeps the same rule -- each
GEMM operand quantized along its contraction dimension, 1x128 groups for
activations and gradients, 128x128 blocks for weights:

* dgrad  dX[M, K] = dY[M, N] W[N, K]: contraction over N. dY in 1x128
  groups along N (the forward activation quantizer applied to dY); W in its
  128x128 blocks, stored transposed (W^T [K, N] codes, scales
  [K/128, N/128]) so the GEMM reads both operands along the contraction;
* wgrad  dW[N, K] = dY^T[N, M] X[M, K]: contraction over M (tokens). Both
  dY and X in 128x1 groups -- 128 consecutive tokens of one column -- i.e.
  the 1x128 group quantizer applied to dY^T and X^T; the product has a
  per-row scale on both operands:
      dW[n, k] = sum_b SA[n, b] SB[k, b] sum_{m in b} A[n, m] B[k, m]
  with A = Q(dY^T) [N, M], B = Q(X^T) [K, M], b over M/128 blocks.

Mixture-of-experts layers (rows sorted by expert, offsets[E+1]; weights
[E, N, K]) take the same rules per expert:

* grouped dgrad  dX[rows of e] = dY[rows of e] W_e: the activation quantizer
  on dY and W_e's blocks transposed, i.e. the grouped GEMM with [E, K, N]
  weights;
* grouped wgrad  dW_e = dY_e^T X_e over expert e's M_e tokens. Reading (the
  pages are silent): the 128x1 groups start at each expert's first token and
  an expert's last, partial group is completed with zero rows -- zeros
  change neither a group's maximum nor the sums -- so the transposed operands
  live on a padded token axis where expert e owns columns
  pad[e] .. pad[e+1], pad[e] = sum_{e' < e} ceil(M_e' / 128) * 128.

Pins (tests/test_oracle_backward.py): the row-scaled GEMM against the
pinned block-scaled GEMM when each 128-row block of B shares its scales,
against exact Fraction sums on a tiny case, and scale linearity per row; the
transposed quantizers against per-group loops of the pinned group and block
quantizers; dgrad and wgrad equal to the exact products dY W and dY^T X
when every group is exactly representable (lossless quantization). Grouped
forms: the grouped transposed quantizer against the pinned group quantizer
on each zero-completed group; grouped dgrad and wgrad against the exact
per-expert products on lossless inputs (ragged experts, an empty one); one
expert of a multiple of 128 tokens reduces to the dense wgrad.
"""

import numpy as np

from .e4m3 import decode
from .quant import GROUP, bf16_values, quant_act_ref, quant_weight_ref


def quant_act_t_ref(x, pow2=False):
    """128x1 groups of X [M, K] (M % 128 == 0): the 1x128 group quantizer
    applied to X^T. Returns (Q^T uint8 [K, M], S^T float32 [K, M/128])."""
    xv = bf16_values(x)
    if xv.ndim != 2 or xv.shape[0] % GROUP:
        raise ValueError("X must be [M, K] with M % 128 == 0")
    return quant_act_ref(np.ascontiguousarray(xv.T), pow2)


def quant_weight_t_ref(w, pow2=False):
    """The 128x128 block quantization of W [N, K] in transposed layout:
    (QW^T uint8 [K, N], SW^T float32 [K/128, N/128])."""
    q, s = quant_weight_ref(w, pow2)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def gemm_rowscaled_ref(qa, sa, qb, sb):
    """Y[m, n] = sum_b sa[m, b] sb[n, b] sum_{k in b} dec(qa[m, k]) dec(qb[n, k]),
    exact in float64 (each 128-term block sum of E4M3 products is exact).
    qa [M, K], sa [M, K/128], qb [N, K], sb [N, K/128]. Returns float64 [M, N]."""
    qa, qb = np.asarray(qa), np.asarray(qb)
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k or k % GROUP:
        raise ValueError("qa [M, K] and qb [N, K] with K % 128 == 0")
    kb = k // GROUP
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64).reshape(m, kb)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64).reshape(n, kb)
    a = decode(qa).reshape(m, kb, GROUP)
    b = decode(qb).reshape(n, kb, GROUP)
    y = np.zeros((m, n))
    for blk in range(kb):
        part = a[:, blk, :] @ b[:, blk, :].T        # exact: products are multiples of 2^-18 below 2^18
        y += (sa[:, blk][:, None] * sb[:, blk][None, :]) * part
    return y


def dgrad_ref(dy, w, pow2=False):
    """dX = dY W with dY in 1x128 groups along N and W in 128x128 blocks.
    dy [M, N], w [N, K] bf16. Returns float64 [M, K]."""
    from .gemm import gemm_ref
    qa, sa = quant_act_ref(dy, pow2)
    qwt, swt = quant_weight_t_ref(w, pow2)
    return gemm_ref(qa, sa, qwt, swt)


def wgrad_ref(dy, x, pow2=False):
    """dW = dY^T X with both operands in 128x1 groups along M.
    dy [M, N], x [M, K] bf16 (M % 128 == 0). Returns float64 [N, K]."""
    qa, sa = quant_act_t_ref(dy, pow2)
    qb, sb = quant_act_t_ref(x, pow2)
    return gemm_rowscaled_ref(qa, sa, qb, sb)


def padded_offsets(offsets):
    """pad[e] = sum over e' < e of ceil(M_e' / 128) * 128 (int64 [E+1]): where
    expert e's tokens start on the padded token axis of the grouped wgrad."""
    m = np.diff(np.asarray(offsets, dtype=np.int64))
    return np.concatenate([[0], np.cumsum((m + GROUP - 1) // GROUP * GROUP)])


def _expert_padded(x, lo, hi):
    """Rows lo..hi of bf16 values x, completed with zero rows to a multiple of 128."""
    rows = x[lo:hi]
    pad = (-(hi - lo)) % GROUP
    return np.concatenate([rows, np.zeros((pad, x.shape[1]))]) if pad else rows


def quant_act_t_grouped_ref(x, offsets, pow2=False):
    """128x1 groups of X [M, K] (rows sorted by expert) starting at each
    expert's first row, the last group of each expert completed with zeros.
    Returns (Q^T uint8 [K, P], S^T float32 [K, P/128]), P = pad[E]: expert
    e's tokens are columns pad[e] .. pad[e] + M_e, its padding columns up to
    pad[e+1] hold code 0 (and count in their group's scale as zeros)."""
    xv = bf16_values(x)
    off = np.asarray(offsets, dtype=np.int64)
    pad = padded_offsets(off)
    k = xv.shape[1]
    qt = np.zeros((k, int(pad[-1])), np.uint8)
    st = np.zeros((k, int(pad[-1]) // GROUP), np.float32)
    for e in range(len(off) - 1):
        if off[e + 1] == off[e]:
            continue
        xe = _expert_padded(xv, off[e], off[e + 1])
        q, sc = quant_act_ref(np.ascontiguousarray(xe.T), pow2)   # 1x128 groups of X_e^T
        qt[:, pad[e]:pad[e + 1]] = q
        st[:, pad[e] // GROUP:pad[e + 1] // GROUP] = sc
    return qt, st


def grouped_dgrad_ref(dy, w, offsets, pow2=False):
    """dX [M, K] for dY [M, N] (rows sorted by expert) and W [E, N, K]: the
    dense dgrad of each expert's rows against its weights. float64."""
    from .gemm import gemm_ref
    off = np.asarray(offsets, dtype=np.int64)
    qa, sa = quant_act_ref(dy, pow2)
    out = np.zeros((qa.shape[0], w.shape[2]))
    for e in range(len(off) - 1):
        if off[e + 1] == off[e]:
            continue
        qwt, swt = quant_weight_t_ref(w[e], pow2)
        out[off[e]:off[e + 1]] = gemm_ref(qa[off[e]:off[e + 1]], sa[off[e]:off[e + 1]], qwt, swt)
    return out


def grouped_wgrad_ref(dy, x, offsets, pow2=False):
    """dW [E, N, K] = per expert dY_e^T X_e with both operands in 128x1 groups
    along the expert's tokens, the last group completed with zero rows
    (dense wgrad on the zero-completed rows). Empty experts give zeros."""
    dyv, xv = bf16_values(dy), bf16_values(x)
    off = np.asarray(offsets, dtype=np.int64)
    e_count = len(off) - 1
    out = np.zeros((e_count, dyv.shape[1], xv.shape[1]))
    for e in range(e_count):
        if off[e + 1] == off[e]:
            continue
        qa, sa = quant_act_ref(np.ascontiguousarray(_expert_padded(dyv, off[e], off[e + 1]).T), pow2)
        qb, sb = quant_act_ref(np.ascontiguousarray(_expert_padded(xv, off[e], off[e + 1]).T), pow2)
        out[e] = gemm_rowscaled_ref(qa, sa, qb, sb)
    return out
