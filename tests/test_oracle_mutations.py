"""Plant plausible mistakes in the oracle (CPU only) and check that a pin
catches each one: evidence that the pins discriminate."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.e4m3 as e4m3
import oracle.gemm as ogemm
import oracle.quant as oquant
import synth
from tests.test_oracle_gemm import _fraction_gemm, _random_operands
from tests.test_oracle_quant import _bruteforce_group, bf16_positive_finite


def _midpoint_pin_holds():
    t = oracle.decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    return np.array_equal(e4m3.encode(mids), oracle.encode_bruteforce(mids))


def test_round_half_up_is_caught(monkeypatch):
    assert _midpoint_pin_holds()
    monkeypatch.setattr(e4m3.np, "rint", lambda a: np.floor(np.asarray(a) + 0.5))
    assert not _midpoint_pin_holds()


def test_wrong_exponent_bias_is_caught(monkeypatch):
    good = e4m3.encode

    def shifted(values):
        c = good(values).astype(np.int64)
        mag = c & 0x7F
        mag = np.where((mag >= 8) & (mag < 0x7E), mag + 8, mag)   # off-by-one binade
        return ((c & 0x80) | np.minimum(mag, 0x7E)).astype(np.uint8)

    monkeypatch.setattr(oquant, "encode", shifted)
    x, _ = synth.linear_inputs("tiny", 0)
    q, s = oracle.quant_act_ref(x[:1])
    codes, sc = _bruteforce_group(list(x[0, :128].double().numpy()), False)
    assert list(q[0, :128]) != codes


def test_reciprocal_shortcut_is_caught(monkeypatch):
    real = oquant.quantize_values

    def via_reciprocal(x, s):
        s32 = np.asarray(s, np.float32)
        inv = np.where(s32 == 0, 0, np.float32(1) / np.where(s32 == 0, 1, s32)).astype(np.float32)
        return e4m3.encode((np.asarray(x, np.float32) * inv).astype(np.float64))

    from tests.test_oracle_quant import divide_vs_reciprocal_pairs
    x, amax = divide_vs_reciprocal_pairs(20)
    s = oracle.group_scale(amax, False)
    monkeypatch.setattr(oquant, "quantize_values", via_reciprocal)
    exact = [oracle.encode_bruteforce(np.array([float(Fraction(float(a)) / Fraction(float(b)))]))[0]
             for a, b in zip(x, s)]
    assert not np.array_equal(oquant.quantize_values(x, s), real(x, s))
    assert not np.array_equal(oquant.quantize_values(x, s), np.array(exact, np.uint8))


def test_pow2_rounded_down_is_caught(monkeypatch):
    monkeypatch.setattr(oquant, "_pow2_exponent",
                        lambda amax: np.floor(np.log2(amax / 448.0)).astype(np.int64))
    amax = bf16_positive_finite()
    s = oracle.group_scale(amax, True).astype(np.float64)
    assert not np.all(448.0 * s >= amax)


def test_wrong_weight_scale_index_is_caught(monkeypatch):
    rng = np.random.default_rng(11)
    qa, sa, qw, sw = _random_operands(rng, 2, 256, 256)
    sw[1] *= 4
    exact = _fraction_gemm(qa, sa, qw, sw)
    monkeypatch.setattr(ogemm.np, "repeat",
                        lambda a, r, axis=None: np.tile(a, (r, 1)) if axis == 0 else np.repeat(a, r, axis))
    y = ogemm.gemm_ref(qa, sa, qw, sw)
    assert any(abs(y[i, j] - float(exact[i][j])) > 1e-9 * abs(float(exact[i][j]))
               for i in range(2) for j in (0, 127, 128, 255))


def test_dropped_block_is_caught(monkeypatch):
    rng = np.random.default_rng(3)
    qa, sa, qw, sw = _random_operands(rng, 2, 128, 384)
    exact = _fraction_gemm(qa, sa, qw, sw)
    real_range = range

    def short_range(*a):
        r = real_range(*a)
        return r[:-1] if len(a) == 1 and a[0] == 3 else r

    monkeypatch.setattr(ogemm, "range", short_range, raising=False)
    y = ogemm.gemm_ref(qa, sa, qw, sw)
    assert any(abs(y[0, j] - float(exact[0][j])) > 1e-9 * max(1, abs(float(exact[0][j]))) for j in (0, 5, 9))
