"""Pins of the FP8 prefill-attention oracle (a sequence's new tokens are
the last of its cached tokens; new token i sits at position
context_len - n_new + i and attends causally to tokens 0..position).

Each pin comes from something other than the oracle's own loops:
torch's scaled_dot_product_attention in float64 on the dequantized operands
with an explicit bottom-right causal mask (and with is_causal when the
whole context is new, where both alignments agree), the last new token
against the decode-step oracle over the whole context (pinned in
test_oracle_attention.py), the first token of a fresh prompt returning its
value row exactly, grouped query heads reading their own KV head, and
planted mask mistakes (strict inequality, top-left alignment) that fail.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
from oracle.attention import decode_attention_ref, prefill_attention_ref
from tests.test_oracle_attention import bf16, codes, lossless_query


def paged_setup(rng, lens, hkv, d=16, bs=4, spare=3):
    """Head-major caches holding every sequence's context on shuffled pages."""
    blocks = [(n + bs - 1) // bs for n in lens]
    pages = sum(blocks) + spare
    kc, vc = codes(rng, (pages, hkv, bs, d)), codes(rng, (pages, hkv, bs, d))
    perm = rng.permutation(pages)
    mb = max(1, max(blocks))
    table = np.full((len(lens), mb), -1, np.int64)
    used = 0
    for b, nb in enumerate(blocks):
        table[b, :nb] = perm[used:used + nb]
        used += nb
    return kc, vc, table, bs


def sdpa_prefill(q_deq, cu, kc, vc, table, bs, lens, ks, vs, sm_scale, use_is_causal=False):
    """torch SDPA (float64, CPU) per sequence with the bottom-right causal
    mask: new token i of n attends to cached tokens t <= L - n + i."""
    tq, hq, d = q_deq.shape
    hkv = kc.shape[1]
    out = np.zeros((tq, hq, d))
    for b in range(len(lens)):
        n, L = int(cu[b + 1] - cu[b]), int(lens[b])
        if n == 0 or L == 0:
            continue
        k = np.zeros((hkv, L, d))
        v = np.zeros((hkv, L, d))
        for t in range(L):
            page, row = int(table[b][t // bs]), t % bs
            for g in range(hkv):
                k[g, t] = oracle.decode(kc[page, g, row]) * ks
                v[g, t] = oracle.decode(vc[page, g, row]) * vs
        rep = hq // hkv
        kt = torch.from_numpy(k).repeat_interleave(rep, dim=0)            # [Hq, L, D]
        vt = torch.from_numpy(v).repeat_interleave(rep, dim=0)
        qt = torch.from_numpy(q_deq[cu[b]:cu[b + 1]]).transpose(0, 1)      # [Hq, n, D]
        kw = {} if sm_scale is None else {"scale": float(np.float32(sm_scale))}
        if use_is_causal:
            o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, **kw)
        else:
            pos = torch.arange(n)[:, None] + (L - n)
            mask = torch.arange(L)[None, :] <= pos                          # [n, L], True = attend
            o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, **kw)
        out[cu[b]:cu[b + 1]] = o.transpose(0, 1).numpy()
    return out


CASES = [  # (new tokens, context length) per sequence
    [(5, 5), (3, 20), (1, 17), (0, 9), (12, 12)],
    [(7, 30), (16, 16)],
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (2, 2)])
@pytest.mark.parametrize("sm_scale", [None, 0.29])
def test_matches_torch_sdpa_float64(case, hq, hkv, sm_scale):
    rng = np.random.default_rng(60 + case + hq)
    seqs = CASES[case]
    news, lens = [n for n, _ in seqs], [L for _, L in seqs]
    cu = np.concatenate([[0], np.cumsum(news)])
    d = 16
    qs, ks, vs = 2.0 ** -6, 0.031, 0.43
    q, q_deq = lossless_query(rng, int(cu[-1]), hq, d, qs)
    kc, vc, table, bs = paged_setup(rng, lens, hkv, d)
    out = prefill_attention_ref(q, cu, kc, vc, table, bs, lens, qs, ks, vs, sm_scale)
    ref = sdpa_prefill(q_deq, cu, kc, vc, table, bs, lens, float(np.float32(ks)), float(np.float32(vs)), sm_scale)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_whole_new_context_matches_is_causal():
    """When every cached token is new (a fresh prompt), the bottom-right mask
    is torch's is_causal."""
    rng = np.random.default_rng(70)
    lens, news = [9, 14], [9, 14]
    cu = np.concatenate([[0], np.cumsum(news)])
    q, q_deq = lossless_query(rng, int(cu[-1]), 4, 16, 2.0 ** -5)
    kc, vc, table, bs = paged_setup(rng, lens, 2)
    out = prefill_attention_ref(q, cu, kc, vc, table, bs, lens, 2.0 ** -5, 0.05, 0.5)
    ref = sdpa_prefill(q_deq, cu, kc, vc, table, bs, lens, float(np.float32(0.05)), 0.5, None, use_is_causal=True)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_last_new_token_is_the_decode_step():
    rng = np.random.default_rng(71)
    lens, news = [23, 8, 40], [6, 8, 1]
    cu = np.concatenate([[0], np.cumsum(news)])
    q = bf16(rng.standard_normal((int(cu[-1]), 4, 16)) * 2)
    kc, vc, table, bs = paged_setup(rng, lens, 2)
    out = prefill_attention_ref(q, cu, kc, vc, table, bs, lens, 0.02, 0.07, 0.3, 0.41)
    last = q[torch.tensor(cu[1:] - 1)]
    dec = decode_attention_ref(last, kc, vc, table, bs, lens, 0.02, 0.07, 0.3, 0.41)
    assert np.array_equal(out[cu[1:] - 1], dec)


def test_first_token_of_a_fresh_prompt_returns_its_value_row():
    rng = np.random.default_rng(72)
    lens, news = [6, 11], [6, 11]
    cu = np.concatenate([[0], np.cumsum(news)])
    q = bf16(rng.standard_normal((int(cu[-1]), 2, 16)))
    kc, vc, table, bs = paged_setup(rng, lens, 1)
    out = prefill_attention_ref(q, cu, kc, vc, table, bs, lens, 0.05, 0.1, 0.25)
    for b in range(2):
        want = oracle.decode(vc[table[b, 0], 0, 0]) * float(np.float32(0.25))
        assert np.array_equal(out[cu[b], 0], want) and np.array_equal(out[cu[b], 1], want)


def test_grouped_heads_read_their_kv_head():
    rng = np.random.default_rng(73)
    lens, news = [13], [5]
    cu = np.array([0, 5])
    q = bf16(rng.standard_normal((5, 4, 16)))
    kc, vc, table, bs = paged_setup(rng, lens, 2)
    vc[:, 0] = 0                                  # KV head 0 carries no values
    out = prefill_attention_ref(q, cu, kc, vc, table, bs, lens, 0.05, 0.1, 0.25)
    assert np.all(out[:, :2] == 0) and np.all(np.any(out[:, 2:] != 0, axis=-1))


def test_mask_mutations_are_caught(monkeypatch):
    def pins_hold():
        try:
            test_matches_torch_sdpa_float64(0, 4, 2, None)
            test_first_token_of_a_fresh_prompt_returns_its_value_row()
            test_last_new_token_is_the_decode_step()
        except (AssertionError, ValueError, IndexError):
            return False
        return True

    assert pins_hold()
    real = oatt.causal_limit
    for name, fn in {"strict t < p": lambda L, n, i: real(L, n, i) - 1,
                     "top-left alignment": lambda L, n, i: i,
                     "no mask": lambda L, n, i: L - 1}.items():
        with monkeypatch.context() as m:
            m.setattr(oatt, "causal_limit", fn)
            assert not pins_hold(), "planted mistake not caught: " + name
