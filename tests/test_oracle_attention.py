"""Pins of the FP8 decode-attention oracle.

Each check comes from something other than the oracle's own formulas: a
single cached token (softmax of one score is 1), equal scores (the plain
mean), a dominant score, a pure-Python loop with math.exp for the softmax
and the weighted sum, page-permutation invariance of the block table, and
grouped heads reading their own KV head.
"""

import math

import numpy as np
import torch

import oracle
from oracle.attention import decode_attention_ref


def bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x30
    return c


def setup(rng, b=2, hq=4, hkv=2, d=16, bs=4, blocks=6, pages=16):
    """Head-major paged caches [pages, Hkv, bs, D] of random finite codes and
    a block table of distinct pages."""
    q = bf16(rng.standard_normal((b, hq, d)))
    kc, vc = codes(rng, (pages, hkv, bs, d)), codes(rng, (pages, hkv, bs, d))
    table = rng.permutation(pages)[: b * blocks].reshape(b, blocks)
    return q, kc, vc, table, bs


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(30)
    q, kc, vc, table, bs = setup(rng)
    out = decode_attention_ref(q, kc, vc, table, bs, [1, 1], 0.05, 0.1, 0.25)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], oracle.decode(vc[table[b, 0], h // 2, 0]) * float(np.float32(0.25)))


def test_equal_scores_give_the_mean():
    rng = np.random.default_rng(31)
    q, kc, vc, table, bs = setup(rng)
    q0 = bf16(np.zeros((2, 4, 16)))                   # every score 0
    out = decode_attention_ref(q0, kc, vc, table, bs, [7, 13], 0.05, 0.1, 0.5)
    for b, n in ((0, 7), (1, 13)):
        rows = [vc[table[b, t // bs], :, t % bs] for t in range(n)]   # [Hkv, D] per token
        for h in range(4):
            want = oracle.decode(np.stack([r[h // 2] for r in rows])).mean(axis=0) * 0.5
            assert np.allclose(out[b, h], want, rtol=1e-14, atol=1e-300)


def test_dominant_score_selects_its_token():
    rng = np.random.default_rng(32)
    d = 16
    kc = np.zeros((2, 1, 4, d), np.uint8)             # every key 0 except token 5
    vc = codes(rng, (2, 1, 4, d))
    kc[1, 0, 1, :] = 0x7E                             # token 5 = page 1, row 1: 448
    q = bf16(np.full((1, 1, d), 448.0))
    table = np.array([[0, 1]])
    out = decode_attention_ref(q, kc, vc, table, 4, [8], 1.0, 1.0, 1.0, sm_scale=1.0)
    assert np.allclose(out[0, 0], oracle.decode(vc[1, 0, 1]), rtol=0, atol=1e-300)


def test_matches_python_loop_with_math_exp():
    rng = np.random.default_rng(33)
    q, kc, vc, table, bs = setup(rng, b=1, hq=2, hkv=1, d=8, bs=2, blocks=5, pages=6)
    qs, ks, vs, sm = 0.02, 0.07, 0.3, 0.37
    n = 9
    out = decode_attention_ref(q, kc, vc, table, bs, [n], qs, ks, vs, sm_scale=sm)
    q8 = oracle.decode(oracle.kv_quantize_ref(q, qs))
    f = lambda x: float(np.float32(x))
    for h in range(2):
        scores = []
        for t in range(n):
            page, row = int(table[0, t // bs]), t % bs
            dot = sum(float(q8[0, h, i]) * float(oracle.decode(kc[page, 0, row, i])) for i in range(8))
            scores.append(dot * f(qs) * f(ks) * f(sm))
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        for i in range(8):
            acc = 0.0
            for t in range(n):
                page, row = int(table[0, t // bs]), t % bs
                acc += w[t] / tot * float(oracle.decode(vc[page, 0, row, i])) * f(vs)
            assert abs(out[0, h, i] - acc) <= 1e-12 * (abs(acc) + 1e-30)


def test_page_permutation_invariance():
    rng = np.random.default_rng(34)
    q, kc, vc, table, bs = setup(rng)
    out = decode_attention_ref(q, kc, vc, table, bs, [17, 23], 0.05, 0.1, 0.25)
    perm = rng.permutation(kc.shape[0])                # move every page elsewhere
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    for old, new in enumerate(perm):
        kc2[new] = kc[old]
        vc2[new] = vc[old]
    out2 = decode_attention_ref(q, kc2, vc2, perm[table], bs, [17, 23], 0.05, 0.1, 0.25)
    assert np.array_equal(out, out2)


def test_grouped_heads_read_their_kv_head():
    rng = np.random.default_rng(35)
    q, kc, vc, table, bs = setup(rng, hq=4, hkv=2)
    vc[:, 1] = 0                                      # KV head 1 carries no values
    out = decode_attention_ref(q, kc, vc, table, bs, [9, 11], 0.05, 0.1, 0.25)
    assert np.all(out[:, 2:] == 0) and np.any(out[:, :2] != 0)
    assert np.all(decode_attention_ref(q, kc, vc, table, bs, [0, 0], 0.05, 0.1, 0.25) == 0)
