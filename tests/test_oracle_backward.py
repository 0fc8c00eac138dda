"""Pins of the backward-GEMM oracle (dgrad, wgrad, the transposed quantizers
and the GEMM with per-row scales on both operands).

Each check comes from something other than the oracle's own formulas: the
already pinned block-scaled GEMM and group/block quantizers applied group by
group, exact Fraction sums, per-row linearity, and exact products of inputs
whose quantization is lossless.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import (dgrad_ref, gemm_rowscaled_ref, grouped_dgrad_ref, grouped_wgrad_ref, padded_offsets,
                             quant_act_t_grouped_ref, quant_act_t_ref, quant_weight_t_ref, wgrad_ref)


def bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    return c


def test_rowscaled_equals_block_gemm_when_rows_share_scales():
    rng = np.random.default_rng(20)
    m, n, k = 5, 256, 384
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa = rng.uniform(0.5, 2, (m, k // 128)).astype(np.float32)
    s_blk = rng.uniform(0.5, 2, (n // 128, k // 128)).astype(np.float32)
    sb = np.repeat(s_blk, 128, axis=0)       # every row of a 128-row block has its block's scale
    assert np.array_equal(gemm_rowscaled_ref(qa, sa, qb, sb), oracle.gemm_ref(qa, sa, qb, s_blk))


def test_rowscaled_exact_fraction_sum():
    rng = np.random.default_rng(21)
    m, n, k = 2, 3, 256
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa = np.float32(rng.uniform(0.1, 3, (m, 2)))
    sb = np.float32(rng.uniform(0.1, 3, (n, 2)))
    da, db = oracle.decode(qa), oracle.decode(qb)
    y = gemm_rowscaled_ref(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for b in range(2):
                blk = sum(Fraction(float(da[i, kk])) * Fraction(float(db[j, kk])) for kk in range(128 * b, 128 * b + 128))
                tot += Fraction(float(sa[i, b])) * Fraction(float(sb[j, b])) * blk
            assert abs(y[i, j] - float(tot)) <= 1e-15 * abs(float(tot)) + 1e-300


def test_rowscaled_is_linear_in_each_row_scale():
    rng = np.random.default_rng(22)
    qa, qb = random_codes(rng, (4, 256)), random_codes(rng, (6, 256))
    sa = np.ones((4, 2), np.float32)
    sb = np.ones((6, 2), np.float32)
    y = gemm_rowscaled_ref(qa, sa, qb, sb)
    sb2 = sb.copy()
    sb2[3] *= 4.0                            # a power of two: exact
    y2 = gemm_rowscaled_ref(qa, sa, qb, sb2)
    assert np.array_equal(y2[:, 3], 4 * y[:, 3]) and np.array_equal(np.delete(y2, 3, 1), np.delete(y, 3, 1))


@pytest.mark.parametrize("pow2", [False, True])
def test_transposed_act_quantizer_group_by_group(pow2):
    """Each 128-token run of one column is quantized exactly as a 1x128
    group of the pinned quantizer would be."""
    rng = np.random.default_rng(23)
    x = bf16(rng.standard_normal((256, 5)) * np.array([1, 100, 1e-3, 7, 0.5]))
    q, s = quant_act_t_ref(x, pow2)
    assert q.shape == (5, 256) and s.shape == (5, 2)
    xv = oracle.bf16_values(x)
    for col in range(5):
        for b in range(2):
            g = bf16(xv[128 * b:128 * b + 128, col][None, :])
            qg, sg = oracle.quant_act_ref(g, pow2)
            assert np.array_equal(q[col, 128 * b:128 * b + 128], qg[0])
            assert s[col, b] == sg[0, 0]


def test_transposed_weight_quantizer_is_the_same_blocks():
    rng = np.random.default_rng(24)
    w = bf16(rng.standard_normal((256, 384)) * 0.02)
    qt, st = quant_weight_t_ref(w)
    q, s = oracle.quant_weight_ref(w)
    assert qt.shape == (384, 256) and st.shape == (3, 2)
    for i in range(2):
        for j in range(3):
            assert st[j, i] == s[i, j]
            assert np.array_equal(qt[128 * j:128 * j + 128, 128 * i:128 * i + 128],
                                  q[128 * i:128 * i + 128, 128 * j:128 * j + 128].T)


def lossless(rng, shape, groups_axis):
    """Values that quantize exactly: E4M3-representable magnitudes times a
    power of two, each group/block holding +-448 * 2^e so its scale is 2^e."""
    vals = oracle.decode(np.arange(0, 0x7F, dtype=np.uint8))          # non-negative finite codes
    v = rng.choice(vals, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    return v


def test_dgrad_and_wgrad_equal_exact_products_when_lossless():
    rng = np.random.default_rng(25)
    m, n, k = 256, 256, 384
    dy = lossless(rng, (m, n), 1)
    w = lossless(rng, (n, k), None)
    x = lossless(rng, (m, k), 0)
    # plant the group maxima: every 1x128 group of dY along N, every 128x1
    # group of dY and X along M, every 128x128 block of W contains 448 * 2^e
    dy[:, ::128] = 448.0
    dy[::128, :] = 448.0
    x[::128, :] = -448.0
    w[::128, ::128] = 448.0
    sdy, sw, sx = 2.0 ** -3, 2.0 ** -10, 2.0 ** 2
    dy, w, x = dy * sdy, w * sw, x * sx
    for pow2 in (False, True):
        assert np.array_equal(dgrad_ref(bf16(dy), bf16(w), pow2), dy @ w)
        assert np.array_equal(wgrad_ref(bf16(dy), bf16(x), pow2), dy.T @ x)


# ------------------------------------------------------------ grouped (MoE)

OFFSETS = np.array([0, 100, 100, 356, 357, 557])        # 100, 0, 256, 1, 200 rows


def test_padded_offsets():
    assert np.array_equal(padded_offsets(OFFSETS), [0, 128, 128, 384, 512, 768])


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_transposed_quantizer_group_by_group(pow2):
    """Each expert's 128-token groups (the last completed with zeros) are
    quantized as 1x128 groups of the pinned quantizer would be; padding
    columns hold code 0."""
    rng = np.random.default_rng(26)
    x = bf16(rng.standard_normal((557, 3)) * np.array([1, 50, 1e-2]))
    q, s = quant_act_t_grouped_ref(x, OFFSETS, pow2)
    pad = padded_offsets(OFFSETS)
    assert q.shape == (3, 768) and s.shape == (3, 6)
    xv = oracle.bf16_values(x)
    for e in range(5):
        lo, hi = OFFSETS[e], OFFSETS[e + 1]
        for j in range((hi - lo + 127) // 128):
            rows = xv[lo + 128 * j:min(hi, lo + 128 * j + 128)]
            for col in range(3):
                g = np.zeros(128)
                g[:len(rows)] = rows[:, col]
                qg, sg = oracle.quant_act_ref(bf16(g[None, :]), pow2)
                c0 = pad[e] + 128 * j
                assert np.array_equal(q[col, c0:c0 + 128], qg[0])
                assert s[col, c0 // 128] == sg[0, 0]
                assert np.all(q[col, c0 + len(rows):c0 + 128] == 0)


def test_grouped_dgrad_and_wgrad_exact_when_lossless():
    """Per expert, dX = dY_e W_e and dW_e = dY_e^T X_e exactly when every
    group and block is exactly representable (maxima planted at the start of
    every expert's 128-token groups); the empty expert gets zeros."""
    rng = np.random.default_rng(27)
    m, n, k, e_count = OFFSETS[-1], 256, 384, 5
    dy = lossless(rng, (m, n), 1)
    x = lossless(rng, (m, k), 0)
    w = lossless(rng, (e_count, n, k), None)
    dy[:, ::128] = 448.0                       # 1x128 groups of dY along N (dgrad)
    for e in range(e_count):
        for r in range(OFFSETS[e], OFFSETS[e + 1], 128):
            dy[r, :] = 448.0                   # 128x1 groups along each expert's tokens (wgrad)
            x[r, :] = -448.0
    w[:, ::128, ::128] = 448.0
    sdy, sw, sx = 2.0 ** -3, 2.0 ** -10, 2.0 ** 2
    dy, w, x = dy * sdy, w * sw, x * sx
    for pow2 in (False, True):
        dx = grouped_dgrad_ref(bf16(dy), bf16(w), OFFSETS, pow2)
        dw = grouped_wgrad_ref(bf16(dy), bf16(x), OFFSETS, pow2)
        for e in range(e_count):
            lo, hi = OFFSETS[e], OFFSETS[e + 1]
            assert np.array_equal(dx[lo:hi], dy[lo:hi] @ w[e])
            assert np.array_equal(dw[e], dy[lo:hi].T @ x[lo:hi])
        assert np.all(dw[1] == 0)


def test_grouped_wgrad_one_expert_is_dense_wgrad():
    rng = np.random.default_rng(28)
    dy = bf16(rng.standard_normal((256, 128)))
    x = bf16(rng.standard_normal((256, 256)) * 3)
    assert np.array_equal(grouped_wgrad_ref(dy, x, [0, 256])[0], wgrad_ref(dy, x))
