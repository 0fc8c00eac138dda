"""Producers of the activations the FP8 linears quantize, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The greentreeone.com NeMo RL FP8 article («Технический прорыв») keeps
normalization and nonlinear functions in BF16 around the FP8 linears; the
upppp.jp article («重要度サンプリングで精度を保つ») and the greentreeone.com
article («Реальные прирост производительности») name the quantization
kernels as overhead and kernel fusion as the way past it. The producers
fused with the 1x128 activation quantization here are the two that feed a
transformer block's linears:

* RMSNorm, the input of the qkv and gate_up projections:
      y[k] = x[k] / sqrt(mean_j x[j]^2 + eps) * gamma[k]
* SiLU(gate) * up, the input of the down projection, from the gate_up
  projection's output laid out [gate | up] along the feature axis:
      h[k] = g[k] / (1 + exp(-g[k])) * u[k]

The pages give neither formula; these are the standard definitions (Llama
and Qwen use both). Readings: the producer's output is rounded once to
bf16 (round to nearest, ties to even) and the quantizer then sees exactly
those bf16 values, as it would if the producer had written them; the
arithmetic before that rounding is fp32 on the GPU and exact (fp64) here,
so the two agree except where the exact value lies within the GPU's fp32
error of a bf16 rounding boundary.

Pins (tests/test_oracle_producers.py): closed forms for constant and one-hot
rows, mean(y^2) = 1 with eps = 0 and unit gamma, exact invariance under
power-of-two scaling, the identity silu(g) - silu(-g) = g, the SiLU minimum
-W(1/e) at -(1 + W(1/e)) (Lambert W), the [gate | up] layout, and
round_bf16 against every bf16 neighbour pair.
"""

import numpy as np

from .quant import bf16_values


def rmsnorm_ref(x, gamma, eps):
    """Exact RMSNorm of each row of x (bf16 [M, K]) with weights gamma (bf16
    [K]) and eps (an fp32 value), in float64. Returns float64 [M, K]."""
    xv = bf16_values(x)
    gv = bf16_values(gamma)
    if xv.ndim != 2 or gv.shape != (xv.shape[1],):
        raise ValueError("x must be [M, K] and gamma [K]")
    e = float(np.float32(eps))
    ms = np.mean(xv * xv, axis=1, keepdims=True)
    return xv / np.sqrt(ms + e) * gv[None, :]


def silu_mul_ref(gu):
    """Exact SiLU(gate) * up for gu (bf16 [M, 2F]) laid out [gate | up] along
    the feature axis, in float64. Returns float64 [M, F]."""
    v = bf16_values(gu)
    if v.ndim != 2 or v.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    f = v.shape[1] // 2
    g, u = v[:, :f], v[:, f:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def round_bf16(v):
    """Round float64 values to bf16 (nearest, ties to even; values beyond
    the bf16 range become +-inf). Returns (uint16 bit patterns, float64
    values). Done in two exact steps: float64 -> float32 would round twice,
    so the rounding is applied directly to the float64 significand."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2**e, |m| in [0.5, 1)
    # a normal bf16 has 8 significant bits: scale to an integer significand
    emin = -125                              # smallest normal bf16 exponent (2**-126 = 0.5 * 2**-125)
    shift = np.where(e < emin, 8 - (emin - e), 8)  # subnormals keep fewer bits
    r = np.ldexp(np.round(np.ldexp(m, shift)), e - shift)   # np.round: ties to even
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    r = np.where(v == 0, v, r)               # keep the sign of zero
    bits = (np.asarray(r, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits, r
