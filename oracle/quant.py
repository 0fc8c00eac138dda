"""Block quantisation to E4M3 for the oracle (test infrastructure only).

Granularity: the greentreeone.com NeMo RL article, section «Технический
прорыв», gives one scale per 1x128 activation group (one row, 128 consecutive
columns of the reduction dimension K) and one per 128x128 weight block.

Readings taken where the pages are silent:

* scale s = amax / 448 rounded once to fp32, stored as the dequantisation
  multiplier (x ~ dec(q) * s); amax is the largest |x| in the group or block;
* power-of-two option (upppp.jp «設定方法»; greentreeone.com «Почему это
  важно для экономики ИИ»): s = 2**k with k the smallest integer such that
  448 * 2**k >= amax, i.e. rounded up, so nothing saturates;
* an all-zero group or block gets s = 0 and codes +-0 (sign kept);
* the element code is enc(RN32(x / s)): the IEEE fp32 quotient first, then
  round-to-nearest-even into E4M3 with saturation (see ``e4m3.encode``);
* inputs are bf16 values and must be finite.

Pins (tests/test_oracle_quant.py): closed forms of the scale (amax = 448*2**j
gives s = 2**j in both modes; s equals numpy's IEEE fp32 division; pow2
bounds 224*s < amax <= 448*s), the fp32 quotient against an exact rational
rounding built from ``fractions``, and invariants of the whole quantiser
(elements equal to +-amax code to +-448, error bounds, sign symmetry,
power-of-two equivariance, permutation equivariance, zero groups).
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode

GROUP = 128  # 1x128 activation groups, 128x128 weight blocks


def bf16_values(x):
    """Exact float64 values of a bf16 input.

    Accepts a torch bfloat16 tensor, a numpy uint16 array of bf16 bit
    patterns, or a float array whose values are all bf16-representable.
    """
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch  # only for its exact bf16 -> fp32 widening
        return x.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    arr = np.asarray(x)
    if arr.dtype == np.uint16:
        f32 = (arr.astype(np.uint32) << 16).view(np.float32)
        return f32.astype(np.float64)
    f32 = arr.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), arr.astype(np.float64)):
        raise ValueError("oracle input is not exactly representable in fp32")
    if np.any(f32.view(np.uint32) & 0xFFFF):
        raise ValueError("oracle input is not exactly representable in bf16")
    return f32.astype(np.float64)


def _pow2_exponent(amax):
    """Smallest integer k with 448 * 2**k >= amax, for amax > 0 (array)."""
    k = np.ceil(np.log2(amax / E4M3_MAX)).astype(np.int64)
    # the float estimate can be off by one either way; settle it with exact
    # comparisons (448 * 2**k and amax are both exact in float64)
    for _ in range(3):
        lower_ok = np.ldexp(E4M3_MAX, (k - 1).astype(np.int32)) >= amax
        k = np.where(lower_ok, k - 1, k)
    for _ in range(3):
        too_small = np.ldexp(E4M3_MAX, k.astype(np.int32)) < amax
        k = np.where(too_small, k + 1, k)
    return k


def group_scale(amax, pow2=False):
    """fp32 scale for each group/block maximum ``amax`` (float64 array).

    Non-pow2: RN32(amax / 448). The float64 quotient of two exact values,
    rounded to float32, is the correctly rounded fp32 quotient: a double
    rounding through binary64 cannot change a quotient rounded to binary32
    (53 >= 2*24 + 2).
    Pow2: 2**k with k from ``_pow2_exponent``.
    Zero amax gives 0.
    """
    amax = np.asarray(amax, dtype=np.float64)
    s = np.zeros(amax.shape, dtype=np.float32)
    nz = amax > 0
    if pow2:
        k = _pow2_exponent(amax[nz])
        s[nz] = np.ldexp(1.0, k.astype(np.int32)).astype(np.float32)
    else:
        s[nz] = (amax[nz] / E4M3_MAX).astype(np.float32)
    return s


def quantize_values(x, s):
    """E4M3 codes of x under scale s (broadcast), as uint8.

    s == 0 (all-zero group) gives +-0 codes. Otherwise the fp32 quotient
    RN32(x / s) is formed (float64 division of exact operands, rounded once
    to float32 -- the same single-rounding argument as in ``group_scale``)
    and then encoded.
    """
    x = np.asarray(x, dtype=np.float64)
    s64 = np.broadcast_to(np.asarray(s, dtype=np.float32).astype(np.float64), x.shape)
    zero = s64 == 0
    q = np.where(zero, 0.0, x / np.where(zero, 1.0, s64)).astype(np.float32)
    # keep the sign of x on exact zeros of a zero group
    q = np.where(zero, np.copysign(np.float32(0.0), x).astype(np.float32), q)
    return encode(q)


def quant_act_ref(x, pow2=False):
    """1x128 group quantisation of activations X[M, K] (K % 128 == 0).

    Returns (Q uint8 [M, K], S float32 [M, K/128]); group g of row m covers
    columns 128*g .. 128*g+127 and S[m, g] is its scale.
    """
    xv = bf16_values(x)
    if xv.ndim != 2 or xv.shape[1] % GROUP:
        raise ValueError("quant_act_ref: X must be [M, K] with K % 128 == 0")
    m, k = xv.shape
    groups = xv.reshape(m, k // GROUP, GROUP)
    amax = np.abs(groups).max(axis=2) if m else np.zeros((0, k // GROUP))
    s = group_scale(amax, pow2)
    q = quantize_values(groups, s[:, :, None]).reshape(m, k)
    return q, s


def quant_weight_ref(w, pow2=False):
    """128x128 block quantisation of weights W[N, K] (N, K % 128 == 0).

    Returns (Q uint8 [N, K], S float32 [N/128, K/128]); block (i, j) covers
    rows 128*i .. 128*i+127 and columns 128*j .. 128*j+127.
    """
    wv = bf16_values(w)
    if wv.ndim != 2 or wv.shape[0] % GROUP or wv.shape[1] % GROUP:
        raise ValueError("quant_weight_ref: W must be [N, K], N and K multiples of 128")
    n, k = wv.shape
    blocks = wv.reshape(n // GROUP, GROUP, k // GROUP, GROUP)
    amax = np.abs(blocks).max(axis=(1, 3))
    s = group_scale(amax, pow2)
    q = quantize_values(blocks, s[:, None, :, None]).reshape(n, k)
    return q, s
