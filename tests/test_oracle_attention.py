"""Pins of the FP8 decode-attention oracle.

Each check comes from something other than the oracle's own formulas: a
single cached token (softmax of one score is 1), equal scores (the plain
mean), a dominant score, a pure-Python loop with math.exp for the softmax
and the weighted sum, page-permutation invariance of the block table,
grouped heads reading their own KV head, torch's
scaled_dot_product_attention in float64 on the dequantized operands (the
score scaling q_scale * k_scale * sm_scale and the default 1/sqrt(D)), and
the two-token closed form (the logistic function of the score difference).
Planted scaling mistakes must fail these pins.
"""

import math

import numpy as np
import pytest
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


# --- score scaling: torch's scaled_dot_product_attention in float64 and the
# two-token closed form ---

def gather_dequantized(kc, vc, table, bs, n, b, hq, ks, vs):
    """K and V of sequence b's first n tokens, read page by page with explicit
    loops, dequantized (code value times the tensor scale) and expanded to
    the Hq query heads (query head h reads KV head h // (Hq / Hkv))."""
    hkv, d = kc.shape[1], kc.shape[3]
    k = np.zeros((hkv, n, d))
    v = np.zeros((hkv, n, d))
    for t in range(n):
        page, row = int(table[b][t // bs]), t % bs
        for g in range(hkv):
            k[g, t] = oracle.decode(kc[page, g, row]) * ks
            v[g, t] = oracle.decode(vc[page, g, row]) * vs
    rep = hq // hkv
    return (torch.from_numpy(k).repeat_interleave(rep, dim=0), torch.from_numpy(v).repeat_interleave(rep, dim=0))


def sdpa_reference(q_deq, kc, vc, table, bs, lens, ks, vs, sm_scale):
    """torch SDPA (float64, CPU) per sequence on dequantized operands."""
    b_, hq, d = q_deq.shape
    out = np.zeros((b_, hq, d))
    for b in range(b_):
        n = int(lens[b])
        if n == 0:
            continue
        k, v = gather_dequantized(kc, vc, table, bs, n, b, hq, ks, vs)
        q = torch.from_numpy(q_deq[b]).unsqueeze(1)                       # [Hq, 1, D]
        kw = {} if sm_scale is None else {"scale": float(np.float32(sm_scale))}
        out[b] = torch.nn.functional.scaled_dot_product_attention(q, k, v, **kw).squeeze(1).numpy()
    return out


def lossless_query(rng, b, hq, d, qs_pow2):
    """A bf16 query whose per-tensor quantization is exact: each value is a
    finite E4M3 value times a power-of-two scale, so q / q_scale is that E4M3
    value and the dequantized query equals q itself."""
    c = codes(rng, (b, hq, d))
    vals = oracle.decode(c) * qs_pow2
    return bf16(vals), vals


@pytest.mark.parametrize("sm_scale", [None, 0.37, 2.0 ** -3])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (2, 2)])
def test_matches_torch_sdpa_float64(sm_scale, hq, hkv):
    rng = np.random.default_rng(40 + hq + hkv)
    d, bs, pages = 16, 4, 40
    b_ = 3
    qs, ks, vs = 2.0 ** -7, 0.043, 0.29        # non-unit scales on every tensor
    q, q_deq = lossless_query(rng, b_, hq, d, qs)
    kc, vc = codes(rng, (pages, hkv, bs, d)), codes(rng, (pages, hkv, bs, d))
    table = rng.permutation(pages)[: b_ * 9].reshape(b_, 9)
    lens = [1, 17, 33]                          # ragged, partial last pages
    out = decode_attention_ref(q, kc, vc, table, bs, lens, qs, ks, vs, sm_scale=sm_scale)
    ref = sdpa_reference(q_deq, kc, vc, table, bs, lens, float(np.float32(ks)), float(np.float32(vs)), sm_scale)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_matches_torch_sdpa_with_quantized_query():
    """Any bf16 query: the oracle's scores use its per-tensor quantization of
    Q (pinned in test_oracle_kv_cache.py); SDPA gets that dequantized Q."""
    rng = np.random.default_rng(47)
    b_, hq, hkv, d, bs, pages = 2, 4, 2, 32, 8, 12
    q = bf16(rng.standard_normal((b_, hq, d)) * 3)
    qs = float(np.float32(np.abs(oracle.bf16_values(q)).max() / 448))
    ks, vs = 0.011, 0.7
    kc, vc = codes(rng, (pages, hkv, bs, d)), codes(rng, (pages, hkv, bs, d))
    table = rng.permutation(pages)[:10].reshape(b_, 5)
    lens = [40, 9]
    q_deq = oracle.decode(oracle.kv_quantize_ref(q, qs)).reshape(b_, hq, d) * qs
    out = decode_attention_ref(q, kc, vc, table, bs, lens, qs, ks, vs)
    ref = sdpa_reference(q_deq, kc, vc, table, bs, lens, float(np.float32(ks)), float(np.float32(vs)), None)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def two_token_case(sm_scale, d=16):
    """One query head over two cached tokens whose E4M3 dot products with the
    query are 4 and 0 exactly: the query is 1.0 (code 0x38) times q_scale in
    every dimension, the first key is 1.0 in four dimensions and 0 elsewhere,
    the second key is 0."""
    qs, ks, vs = 2.0 ** -4, 0.37, 1.5
    q = bf16(np.full((1, 1, d), qs))
    kc = np.zeros((1, 1, 2, d), np.uint8)
    kc[0, 0, 0, :4] = 0x38
    vc = np.zeros((1, 1, 2, d), np.uint8)
    vc[0, 0, 0, :] = 0x40                       # 2.0
    vc[0, 0, 1, :] = 0xB0                       # -0.5
    out = decode_attention_ref(q, kc, vc, np.array([[0]]), 2, [2], qs, ks, vs, sm_scale=sm_scale)
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(np.float32(sm_scale))
    delta = 4.0 * qs * float(np.float32(ks)) * sm
    w = 1.0 / (1.0 + math.exp(-delta))          # logistic weight of the first token
    want = (w * 2.0 + (1.0 - w) * -0.5) * vs
    return out[0, 0], want


@pytest.mark.parametrize("sm_scale", [None, 0.7, 3.0])
def test_two_token_closed_form(sm_scale):
    got, want = two_token_case(sm_scale)
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_scaling_mutations_are_caught(monkeypatch):
    """Plant each plausible scaling mistake; a pin above must fail."""
    import oracle.attention as oatt

    def pins_hold():
        ok = all(np.allclose(*two_token_case(s), rtol=1e-14, atol=0) for s in (None, 0.7))
        try:
            test_matches_torch_sdpa_float64(None, 4, 2)
            test_matches_torch_sdpa_float64(0.37, 4, 2)
        except AssertionError:
            ok = False
        return ok

    assert pins_hold()
    real_scores, real_sm = oatt.scores, oatt.softmax_scale
    mutations = {
        "k_scale dropped": ("scores", lambda dots, qs, ks, sm: real_scores(dots, qs, 1.0, sm)),
        "q_scale dropped": ("scores", lambda dots, qs, ks, sm: real_scores(dots, 1.0, ks, sm)),
        "sm_scale squared": ("scores", lambda dots, qs, ks, sm: real_scores(dots, qs, ks, sm * sm)),
        "default 1/D": ("softmax_scale", lambda d, s: 1.0 / d if s is None else real_sm(d, s)),
        "default 1": ("softmax_scale", lambda d, s: 1.0 if s is None else real_sm(d, s)),
    }
    for name, (attr, fn) in mutations.items():
        with monkeypatch.context() as m:
            m.setattr(oatt, attr, fn)
            assert not pins_hold(), "planted mistake not caught: " + name
