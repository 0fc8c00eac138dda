"""FP8 KV cache: per-step Q/K/V scale recalibration and the quantize-and-write
of K and V into the cache (test infrastructure only, see the package
docstring).

Sources: the upppp.jp NeMo RL FP8 article, section «KVキャッシュとAttention
にも拡張»: the KV cache and attention also run in FP8; because the policy's
weights change every training step, the Q, K and V scales are recomputed in
BF16 at the end of each step (with the updated weights, on training prompts
and generated responses) and handed to the rollout engine for the next
rollout, at 2-3% of the step. The greentreeone.com article, section
«Реальные прирост производительности»: FP8 KV cache and attention, with the
quantization scales recalibrated after every training step.

Readings taken where the pages are silent:

* granularity: one scale per tensor -- Q, K and V of one attention layer --
  over all calibration tokens; amax accumulates over every chunk of the
  calibration batch;
* scale rule: as for the linear layers' groups, s = RN32(amax / 448), or the
  power-of-two option (``group_scale``);
* layout: the qkv projection writes each token's row as [Q heads | K heads |
  V heads] = Hq*D, Hkv*D and Hkv*D columns;
* cache entry = enc(RN32(x / s)) as for the linear layers, saturating at
  +-448 (tokens written after calibration may exceed the calibrated range;
  a quotient beyond the fp32 range saturates too); s = 0 gives +-0;
* paged cache layout per tensor: [num_blocks][Hkv][block_size][D] -- each
  page holds block_size tokens, head-major, so one head's rows of a page are
  contiguous; slot = block * block_size + offset, and token t goes to slot
  slot[t]; a negative slot (padding) writes nothing; the slots of one call
  are distinct.

Pins (tests/test_oracle_kv_cache.py): maxima planted at known places and a
brute-force Python scan; the per-tensor quantizer equals the pinned 1x128
group quantizer when the tensor is one group; saturation and zero-scale
cases; the dequantization error bound; the cache write against a per-token
Python loop over tokens and heads, with padding slots left untouched.
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode
from .quant import bf16_values, group_scale


def qkv_amax_ref(qkv, hq, hkv, d):
    """Largest |Q|, |K|, |V| of a qkv projection output [T, (hq + 2*hkv)*d]
    (bf16). Returns float64 [3]; an empty input gives zeros."""
    v = bf16_values(qkv)
    if v.ndim != 2 or v.shape[1] != (hq + 2 * hkv) * d:
        raise ValueError("qkv must be [T, (Hq + 2*Hkv) * D]")
    cuts = (0, hq * d, (hq + hkv) * d, (hq + 2 * hkv) * d)
    return np.array([np.abs(v[:, cuts[i]:cuts[i + 1]]).max(initial=0.0) for i in range(3)])


def kv_scales_ref(amax, pow2=False):
    """Per-tensor scales from the maxima: the linear layers' scale rule."""
    return group_scale(np.asarray(amax, dtype=np.float64), pow2)


def kv_quantize_ref(x, s):
    """E4M3 codes of bf16 x under one fp32 scale s, saturating at +-448.

    The quotient |x| / s is exact in float64 (both operands exact); it is
    clamped at 448 before the single rounding to fp32, which changes no
    quotient below 448 and sends every larger one (including those beyond
    the fp32 range) to the saturated code."""
    xv = bf16_values(x)
    s = float(np.float32(s))
    if s == 0.0:
        return encode(np.copysign(0.0, xv))
    q = np.minimum(np.abs(xv) / s, E4M3_MAX).astype(np.float32).astype(np.float64)
    return encode(np.copysign(q, xv))


def kv_cache_write_ref(k, v, slot, k_cache, v_cache, k_scale, v_scale):
    """Write the quantized rows of k and v ([T, Hkv*D] bf16) into copies of
    the paged caches ([num_blocks, Hkv, block_size, D] uint8): head h of
    token t goes to [slot[t] // block_size, h, slot[t] % block_size] (skipped
    when slot[t] is negative). Returns the two new caches."""
    slot = np.asarray(slot, dtype=np.int64)
    kc = np.array(k_cache, dtype=np.uint8, copy=True)
    vc = np.array(v_cache, dtype=np.uint8, copy=True)
    if kc.ndim != 4 or vc.shape != kc.shape:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D] and alike")
    nblk, hkv, bs, d = kc.shape
    qk = kv_quantize_ref(k, k_scale).reshape(-1, hkv, d)
    qv = kv_quantize_ref(v, v_scale).reshape(-1, hkv, d)
    live = slot >= 0
    if len(np.unique(slot[live])) != int(live.sum()):
        raise ValueError("slots of one call must be distinct")
    if np.any(slot[live] >= nblk * bs):
        raise ValueError("slot out of range")
    blk, off = slot[live] // bs, slot[live] % bs
    kc[blk, :, off] = qk[live]
    vc[blk, :, off] = qv[live]
    return kc, vc
