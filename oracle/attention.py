"""FP8 decode attention over the paged FP8 KV cache (test infrastructure
only, see the package docstring).

Sources: the upppp.jp NeMo RL FP8 article, section «KVキャッシュとAttention
にも拡張»: the longer the outputs, the more the KV cache and attention
dominate rollout time, so the KV cache and attention also run in FP8 with
the recalibrated Q/K/V scales; the greentreeone.com article, section
«Реальные прирост производительности»: FP8 for the KV cache and the
attention operations.

Readings taken where the pages are silent:

* the decode step: each sequence's new query token attends over every token
  cached for it (context_len tokens, the new one included once written);
* Q is quantized like K and V, per tensor with the calibrated Q scale
  (``kv_quantize_ref``); scores are the exact products of the FP8 values,
      s[h, t] = (sum_d dec(q8[h, d]) dec(k8[t, g, d])) * q_scale * k_scale * sm_scale
  with g = h // (Hq / Hkv) (grouped-query attention) and sm_scale given
  (1 / sqrt(D) by default);
* softmax over t in exact arithmetic, the probabilities kept unquantized,
      out[h, d] = sum_t softmax(s[h])_t dec(v8[t, g, d]) * v_scale
  rounded once to bf16 by the caller's comparison; a sequence with no
  cached tokens gives 0;
* paged cache: token t of sequence b is at offset t % block_size of page
  block_table[b, t // block_size] of the [num_blocks, Hkv, block_size, D]
  caches written by the cache write (head-major pages).

Pins (tests/test_oracle_attention.py): one cached token returns its value
row exactly; equal scores give the plain mean of the value rows; a dominant
score selects its token; the softmax weights equal a Python loop with
math.exp; permuting the pages (block table) leaves the output unchanged;
grouped heads read their own KV head. The score scaling
(q_scale * k_scale * sm_scale, default 1/sqrt(D)) is pinned against
torch's scaled_dot_product_attention in float64 on the dequantized Q, K, V
(default and explicit scale, grouped heads expanded, ragged lengths, paged
tables) and against the two-token closed form: the first token's weight is
the logistic function of the score difference. Planted mistakes in the
scaling (k_scale dropped, sm_scale squared, 1/D for the default) fail them.

The prefill step (same sources; readings where they are silent): a sequence's n new
tokens are the last n of its context_len cached tokens, so new token i sits
at position p = context_len - n + i and its query attends causally over the
cached tokens 0..p; scores, softmax and the weighted sum as in the decode
step (exact, probabilities unquantized). Pins: torch's
scaled_dot_product_attention in float64 with the bottom-right causal mask
(and is_causal when the whole context is new), the last new token against
the decode step over the whole context, the first token of a fresh prompt
returning its value row exactly, and planted mistakes in the mask (t < p,
top-left alignment) that these pins catch.
"""

import numpy as np

from .e4m3 import decode
from .kv_cache import kv_quantize_ref
from .quant import bf16_values


def softmax_scale(d, sm_scale):
    """The softmax scale: 1/sqrt(D) for standard attention unless given
    (then the fp32 value the kernels receive)."""
    return 1.0 / np.sqrt(d) if sm_scale is None else float(np.float32(sm_scale))


def scores(dots, qs, ks, sm):
    """Scores from the exact dot products of the E4M3 values: the per-tensor
    Q and K scales and the softmax scale multiply each one."""
    return dots * qs * ks * sm


def decode_attention_ref(q, k_cache, v_cache, block_table, block_size, context_lens, q_scale, k_scale, v_scale,
                         sm_scale=None):
    """q [B, Hq, D] bf16; caches [num_blocks, Hkv, block_size, D] E4M3 codes
    (uint8); block_table [B, max_blocks] int; context_lens [B] int. Returns
    float64 [B, Hq, D]."""
    qv = bf16_values(q)
    b_, hq, d = qv.shape
    k_cache = np.asarray(k_cache, np.uint8)
    v_cache = np.asarray(v_cache, np.uint8)
    if k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D] and alike")
    hkv = k_cache.shape[1]
    if hq % hkv or k_cache.shape[3] != d or k_cache.shape[2] != block_size:
        raise ValueError("shapes: q [B, Hq, D], caches [num_blocks, Hkv, block_size, D], Hq % Hkv == 0")
    group = hq // hkv
    sm = softmax_scale(d, sm_scale)
    qs, ks, vs = (float(np.float32(s)) for s in (q_scale, k_scale, v_scale))
    q8 = decode(kv_quantize_ref(q, qs).reshape(b_, hq, d))
    kd = decode(k_cache)
    vd = decode(v_cache)
    out = np.zeros((b_, hq, d))
    table = np.asarray(block_table, np.int64)
    for b in range(b_):
        n = int(context_lens[b])
        if n == 0:
            continue
        t = np.arange(n)
        blk, off = table[b, t // block_size], t % block_size
        for h in range(hq):
            g = h // group
            s = scores(kd[blk, g, off, :] @ q8[b, h], qs, ks, sm)
            w = np.exp(s - s.max())
            w /= w.sum()
            out[b, h] = (w @ vd[blk, g, off, :]) * vs
    return out


def causal_limit(context_len, n_new, i):
    """Position of new token i of a sequence whose n_new new tokens are the
    last of its context_len cached tokens: its query attends to tokens
    0..limit."""
    return context_len - n_new + i


def prefill_attention_ref(q, cu_seqlens_q, k_cache, v_cache, block_table, block_size, context_lens, q_scale,
                          k_scale, v_scale, sm_scale=None):
    """q [total_q, Hq, D] bf16: the new tokens of every sequence, sequence b's
    rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; caches [num_blocks, Hkv,
    block_size, D] E4M3 codes; block_table [B, max_blocks]; context_lens [B]
    (cached tokens per sequence, the new ones included). Returns float64
    [total_q, Hq, D]."""
    qv = bf16_values(q)
    tq, hq, d = qv.shape
    k_cache = np.asarray(k_cache, np.uint8)
    v_cache = np.asarray(v_cache, np.uint8)
    if k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D] and alike")
    hkv = k_cache.shape[1]
    if hq % hkv or k_cache.shape[3] != d or k_cache.shape[2] != block_size:
        raise ValueError("shapes: q [total_q, Hq, D], caches [num_blocks, Hkv, block_size, D], Hq % Hkv == 0")
    group = hq // hkv
    cu = np.asarray(cu_seqlens_q, np.int64)
    sm = softmax_scale(d, sm_scale)
    qs, ks, vs = (float(np.float32(s)) for s in (q_scale, k_scale, v_scale))
    q8 = decode(kv_quantize_ref(q, qs).reshape(tq, hq, d))
    kd = decode(k_cache)
    vd = decode(v_cache)
    table = np.asarray(block_table, np.int64)
    out = np.zeros((tq, hq, d))
    for b in range(len(cu) - 1):
        n_new = int(cu[b + 1] - cu[b])
        length = int(context_lens[b])
        if n_new == 0 or length == 0:
            continue
        t = np.arange(length)
        blk, off = table[b, t // block_size], t % block_size
        for g in range(hkv):
            keys, vals = kd[blk, g, off, :], vd[blk, g, off, :]        # [L, D] of KV head g
            for i in range(n_new):
                lim = causal_limit(length, n_new, i)
                if lim < 0:
                    continue
                for h in range(g * group, (g + 1) * group):
                    s = scores(keys[:lim + 1] @ q8[cu[b] + i, h], qs, ks, sm)
                    w = np.exp(s - s.max())
                    w /= w.sum()
                    out[cu[b] + i, h] = (w @ vals[:lim + 1]) * vs
    return out
