"""Pins of the oracle's block-scaled GEMM and grouped GEMM (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (
    decode, decode_table, encode, gemm_ref, gemm_ref_blas, grouped_gemm_ref,
    quant_act_ref, quant_weight_ref, tolerance_ok,
)


def _random_operands(rng, m, n, k, scale_range=(-12, 4)):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    qa = rng.choice(finite, size=(m, k)).astype(np.uint8)
    qw = rng.choice(finite, size=(n, k)).astype(np.uint8)
    sa = np.exp2(rng.uniform(*scale_range, size=(m, k // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(*scale_range, size=(n // 128, k // 128))).astype(np.float32)
    return qa, sa, qw, sw


def _fraction_gemm(qa, sa, qw, sw):
    """Exact rational Y[m, n] straight from the block-scaled definition."""
    tab = decode_table()
    fa = [[Fraction(float(tab[c])) for c in row] for row in qa]
    fw = [[Fraction(float(tab[c])) for c in row] for row in qw]
    m, k = qa.shape
    n = qw.shape[0]
    y = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for b in range(k // 128):
                dot = sum(fa[i][kk] * fw[j][kk] for kk in range(128 * b, 128 * b + 128))
                tot += Fraction(float(sa[i, b])) * Fraction(float(sw[j // 128, b])) * dot
            y[i][j] = tot
    return y


@pytest.mark.parametrize("k", [128, 256, 384])
def test_gemm_matches_exact_fractions(k):
    rng = np.random.default_rng(k)
    qa, sa, qw, sw = _random_operands(rng, 3, 128, k)
    y = gemm_ref(qa, sa, qw, sw)
    yb = gemm_ref_blas(qa, sa, qw, sw)
    exact = _fraction_gemm(qa, sa, qw[:128], sw)
    for i in range(3):
        for j in range(0, 128, 7):
            e = float(exact[i][j])
            assert abs(y[i, j] - e) <= 1e-12 * max(1.0, abs(e)) * 64
            assert abs(yb[i, j] - e) <= 1e-12 * max(1.0, abs(e)) * 64


def test_gemm_two_block_rows_use_their_own_weight_scale():
    # N = 256: the second 128-row weight block must use SW[1, :]
    rng = np.random.default_rng(11)
    qa, sa, qw, sw = _random_operands(rng, 2, 256, 256)
    sw[1] *= 4
    y = gemm_ref(qa, sa, qw, sw)
    exact = _fraction_gemm(qa, sa, qw, sw)
    for i in range(2):
        for j in (0, 127, 128, 200, 255):
            assert abs(y[i, j] - float(exact[i][j])) <= 1e-12 * max(1.0, abs(float(exact[i][j]))) * 64


def test_gemm_integer_closed_form_is_exact():
    rng = np.random.default_rng(5)
    a_int = rng.integers(-1, 2, size=(16, 256))
    w_int = rng.integers(-1, 2, size=(128, 256))
    qa, qw = encode(a_int.astype(np.float64)), encode(w_int.astype(np.float64))
    sa = np.ones((16, 2), np.float32)
    sw = np.ones((1, 2), np.float32)
    want = a_int @ w_int.T                      # integer matmul, a library routine
    assert np.array_equal(gemm_ref(qa, sa, qw, sw), want.astype(np.float64))
    # |y| <= 256 and bf16 holds every integer up to 256 exactly, so a GPU
    # must reproduce these bitwise
    assert np.all(np.abs(want) <= 256)


def test_blockwise_and_blas_forms_agree_on_tiny_workload():
    x, w = synth.linear_inputs("tiny", 0)
    qa, sa = quant_act_ref(x)
    qw, sw = quant_weight_ref(w)
    y = gemm_ref(qa, sa, qw, sw)
    yb = gemm_ref_blas(qa, sa, qw, sw)
    assert np.max(np.abs(y - yb)) <= 1e-12 * np.max(np.abs(y))


def test_zero_block_contributes_nothing():
    rng = np.random.default_rng(9)
    qa, sa, qw, sw = _random_operands(rng, 8, 128, 384)
    y_drop = gemm_ref(np.delete(qa, np.s_[128:256], 1), np.delete(sa, 1, 1),
                      np.delete(qw, np.s_[128:256], 1), np.delete(sw, 1, 1))
    qa0 = qa.copy()
    qa0[:, 128:256] = 0
    y0 = gemm_ref(qa0, sa, qw, sw)
    assert np.allclose(y0, y_drop, rtol=1e-13, atol=0)
    # a zero scale (all-zero group) also contributes exactly zero
    sa0 = sa.copy()
    sa0[:, 1] = 0
    assert np.allclose(gemm_ref(qa, sa0, qw, sw), y_drop, rtol=1e-13, atol=0)


def test_doubling_row_scales_doubles_row():
    rng = np.random.default_rng(10)
    qa, sa, qw, sw = _random_operands(rng, 4, 128, 256)
    y = gemm_ref(qa, sa, qw, sw)
    sa2 = sa.copy()
    sa2[2] *= 2
    y2 = gemm_ref(qa, sa2, qw, sw)
    assert np.array_equal(y2[2], 2 * y[2])
    assert np.array_equal(np.delete(y2, 2, 0), np.delete(y, 2, 0))


def test_gemm_matches_unquantised_product_within_quantisation_error():
    """Y_ref approximates X W^T of the unquantised bf16 inputs (fidelity of
    the method, not a parity gate): a few percent relative Frobenius error."""
    x, w = synth.linear_inputs("tiny", 0)
    qa, sa = quant_act_ref(x)
    qw, sw = quant_weight_ref(w)
    y = gemm_ref(qa, sa, qw, sw)
    yt = x.double().numpy() @ w.double().numpy().T
    rel = np.linalg.norm(y - yt) / np.linalg.norm(yt)
    assert rel < 0.06


def test_grouped_single_expert_reduces_to_gemm():
    x, w = synth.linear_inputs("tiny", 0)
    qa, sa = quant_act_ref(x)
    qw, sw = quant_weight_ref(w)
    off = np.array([0, x.shape[0]])
    assert np.array_equal(grouped_gemm_ref(qa, sa, qw[None], sw[None], off), gemm_ref(qa, sa, qw, sw))


def test_grouped_matches_exact_fractions_with_empty_experts():
    rng = np.random.default_rng(12)
    e_count, n, k = 4, 128, 256
    counts = [2, 0, 3, 0]
    off = np.concatenate([[0], np.cumsum(counts)])
    qa, sa, _, _ = _random_operands(rng, int(off[-1]), n, k)
    qw = np.stack([_random_operands(rng, 1, n, k)[2] for _ in range(e_count)])
    sw = np.exp2(rng.uniform(-8, 0, size=(e_count, 1, 2))).astype(np.float32)
    y = grouped_gemm_ref(qa, sa, qw, sw, off)
    for e in range(e_count):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        exact = _fraction_gemm(qa[lo:hi], sa[lo:hi], qw[e], sw[e])
        for i in range(hi - lo):
            for j in range(0, n, 9):
                assert abs(y[lo + i, j] - float(exact[i][j])) <= 1e-12 * max(1.0, abs(float(exact[i][j]))) * 64


def test_grouped_offsets_validation():
    qa = np.zeros((3, 128), np.uint8)
    sa = np.zeros((3, 1), np.float32)
    qw = np.zeros((2, 128, 128), np.uint8)
    sw = np.zeros((2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        grouped_gemm_ref(qa, sa, qw, sw, [0, 2, 2])   # does not end at 3
    with pytest.raises(ValueError):
        grouped_gemm_ref(qa, sa, qw, sw, [0, 3])      # wrong length


def test_tolerance_rule():
    rng = np.random.default_rng(13)
    y_ref = rng.standard_normal(10000) * 10
    y_bf16 = torch.tensor(y_ref, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert tolerance_ok(y_bf16, y_ref)[0]          # bf16 rounding alone passes
    big = np.argmax(np.abs(y_ref))
    y_bad = y_ref.copy()
    y_bad[big] *= 1 + 2.0 ** -5
    assert not tolerance_ok(y_bad, y_ref)[0]       # a 2**-5 relative error fails
    y_nan = y_ref.copy()
    y_nan[0] = np.nan
    assert not tolerance_ok(y_nan, y_ref)[0]
