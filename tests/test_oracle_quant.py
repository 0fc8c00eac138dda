"""Pins of the oracle's block quantiser (CPU only).

Scales are pinned to closed forms and to numpy's IEEE fp32 division; the fp32
quotient x/s to an exact rational rounding written here with ``fractions``;
whole-tensor results to pure-Python brute force on small blocks and to
invariants that any correct quantiser has.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (
    E4M3_MAX, decode, encode_bruteforce, group_scale, quant_act_ref,
    quant_weight_ref, quantize_values,
)


# ---------------------------------------------------------------- helpers

def rn32_exact(fr):
    """Round a rational to the nearest fp32 value, ties to even, with the
    fp32 subnormal grid below 2**-126. Independent of numpy's float32."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    n0 = n.numerator // n.denominator
    rem = n - n0
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n0 % 2 == 1):
        n0 += 1
    r = float(n0 * quantum)
    return -r if neg else r


def bf16_positive_finite():
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16   # +min subnormal .. +max finite
    return bits.view(np.float32).astype(np.float64)


def bf16_round(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).float().numpy().astype(np.float64)


# ---------------------------------------------------------------- scales

def test_scale_closed_form_powers_of_two():
    j = np.arange(-40, 40)
    amax = np.ldexp(E4M3_MAX, j)
    for pow2 in (False, True):
        s = group_scale(amax, pow2)
        assert np.array_equal(s.astype(np.float64), np.ldexp(1.0, j))


def test_scale_matches_ieee_fp32_division_on_all_bf16():
    amax = bf16_positive_finite()
    s = group_scale(amax, pow2=False)
    ref = np.float32(amax.astype(np.float32)) / np.float32(448.0)   # numpy IEEE fp32 divide
    assert np.array_equal(s.view(np.uint32), ref.view(np.uint32))


def test_scale_matches_exact_rational_rounding():
    amax = bf16_positive_finite()[::37]
    s = group_scale(amax, pow2=False)
    for a, got in zip(amax, s):
        assert float(got) == rn32_exact(Fraction(a) / 448)


def test_scale_pow2_bounds_on_all_bf16():
    amax = bf16_positive_finite()
    s = group_scale(amax, pow2=True).astype(np.float64)
    mant, _ = np.frexp(s)
    assert np.all(mant == 0.5)                       # a power of two
    assert np.all(448.0 * s >= amax)                 # nothing saturates
    assert np.all(224.0 * s < amax)                  # and it is the smallest such


def test_scale_zero_group():
    assert group_scale(np.array([0.0]), False)[0] == 0
    assert group_scale(np.array([0.0]), True)[0] == 0


def test_pow2_worked_example():
    # amax = 1 -> s = 2**-8; x = 1 -> 256 exactly -> code 0x78; x = -0.5 -> -128 -> 0xF0
    s = group_scale(np.array([1.0]), pow2=True)
    assert s[0] == 2.0 ** -8
    assert list(quantize_values(np.array([1.0, -0.5]), s[0])) == [0x78, 0xF0]


# ---------------------------------------------------------------- quotient

def divide_vs_reciprocal_pairs(count, seed=7):
    """(x, amax) pairs, x and amax bf16 with |x| <= amax, for which the E4M3
    code of the fp32 quotient x/s differs from the code of x * fp32(1/s)."""
    rng = np.random.default_rng(seed)
    xs, am = [], []
    while len(xs) < count:
        amax = bf16_round(np.exp2(rng.uniform(-20, 20, 200000)))
        x = bf16_round(amax * rng.uniform(-1, 1, amax.size))
        s = (amax / 448.0).astype(np.float32)
        q_div = x.astype(np.float32) / s
        q_rcp = x.astype(np.float32) * (np.float32(1.0) / s)
        ok = (q_div != q_rcp) & (np.abs(x) <= amax)
        ok &= encode_bruteforce(q_div.astype(np.float64)) != encode_bruteforce(q_rcp.astype(np.float64))
        xs.extend(x[ok][: count - len(xs)])
        am.extend(amax[ok][: count - len(am)])
    return np.array(xs), np.array(am)


def test_quotient_matches_exact_rational_rounding():
    rng = np.random.default_rng(3)
    amax = bf16_round(np.exp2(rng.uniform(-30, 30, 3000)))
    x = bf16_round(amax * rng.uniform(-1, 1, amax.size))
    dx, da = divide_vs_reciprocal_pairs(300)
    x = np.concatenate([x, dx, [0.0, -0.0, 1e-40, -1e-40]])
    amax = np.concatenate([amax, da, [1.0, 1.0, 1.0, 1.0]])
    for pow2 in (False, True):
        s = group_scale(amax, pow2)
        got = quantize_values(x, s)
        exact = np.array([rn32_exact(Fraction(float(xi)) / Fraction(float(si)))
                          for xi, si in zip(x, s)])
        # keep the sign of exact zeros
        exact = np.where(exact == 0, np.copysign(0.0, x), exact)
        assert np.array_equal(got, encode_bruteforce(exact))


def test_divide_and_reciprocal_really_differ():
    """The discriminating pairs exist: a reciprocal shortcut changes codes."""
    x, amax = divide_vs_reciprocal_pairs(50)
    s = group_scale(amax, False)
    via_rcp = encode_bruteforce((x.astype(np.float32) * (np.float32(1) / s)).astype(np.float64))
    assert np.all(quantize_values(x, s) != via_rcp)


# ---------------------------------------------------------------- brute force

def _bruteforce_group(vals, pow2):
    """Pure-Python quantisation of one group/block (list of floats)."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        return [0x80 if np.signbit(v) else 0x00 for v in vals], 0.0
    if pow2:
        k = 0
        while Fraction(448) * Fraction(2) ** k < Fraction(amax):
            k += 1
        while Fraction(448) * Fraction(2) ** (k - 1) >= Fraction(amax):
            k -= 1
        s = float(Fraction(2) ** k)
    else:
        s = rn32_exact(Fraction(amax) / 448)
    qv = [rn32_exact(Fraction(v) / Fraction(s)) for v in vals]
    qv = [np.copysign(0.0, v) if q == 0 else q for q, v in zip(qv, vals)]
    return list(encode_bruteforce(np.array(qv))), s


@pytest.mark.parametrize("pow2", [False, True])
def test_act_quant_matches_bruteforce(pow2):
    x, _ = synth.linear_inputs("tiny", 0)
    x = x[:3]
    q, s = quant_act_ref(x, pow2)
    xv = x.float().numpy().astype(np.float64)
    for m in range(xv.shape[0]):
        for g in range(xv.shape[1] // 128):
            codes, sc = _bruteforce_group(list(xv[m, 128 * g:128 * g + 128]), pow2)
            assert float(s[m, g]) == sc
            assert list(q[m, 128 * g:128 * g + 128]) == codes


@pytest.mark.parametrize("pow2", [False, True])
def test_weight_quant_matches_bruteforce(pow2):
    _, w = synth.linear_inputs("tiny", 0)
    w = w[:128]                     # one block row: blocks (0,0) and (0,1)
    q, s = quant_weight_ref(w, pow2)
    wv = w.float().numpy().astype(np.float64)
    for j in range(2):
        blk = wv[:, 128 * j:128 * j + 128]
        codes, sc = _bruteforce_group(list(blk.ravel()), pow2)
        assert float(s[0, j]) == sc
        assert list(q[:, 128 * j:128 * j + 128].ravel()) == codes


# ---------------------------------------------------------------- invariants

def _varied_activations():
    x, _ = synth.linear_inputs("tiny", 0)
    g = synth.generator(1)
    wild = (torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-60, 60, (64, 1), generator=g).float()))
    return torch.cat([x, wild.to(torch.bfloat16)])


@pytest.mark.parametrize("pow2", [False, True])
def test_no_nan_codes_and_error_bound(pow2):
    x = _varied_activations()
    q, s = quant_act_ref(x, pow2)
    assert not np.any((q == 0x7F) | (q == 0xFF))
    xv = x.float().numpy().astype(np.float64)
    s_el = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = decode(q) * s_el
    v = np.where(s_el > 0, xv / np.where(s_el > 0, s_el, 1), 0)
    err = np.abs(deq - xv)
    normal = np.abs(v) >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(xv[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * s_el[~normal] + 2.0 ** -24 * np.abs(xv[~normal]))


def test_amax_elements_code_to_448():
    x = _varied_activations()
    q, s = quant_act_ref(x, pow2=False)
    xv = x.float().numpy().astype(np.float64).reshape(x.shape[0], -1, 128)
    amax = np.abs(xv).max(axis=2, keepdims=True)
    qg = q.reshape(xv.shape)
    hit = (np.abs(xv) == amax) & (amax > 0)
    assert np.all(qg[hit & (xv > 0)] == 0x7E)
    assert np.all(qg[hit & (xv < 0)] == 0xFE)


@pytest.mark.parametrize("pow2", [False, True])
def test_sign_symmetry(pow2):
    x = _varied_activations()
    q, s = quant_act_ref(x, pow2)
    qn, sn = quant_act_ref(-x, pow2)
    assert np.array_equal(qn, q ^ 0x80)
    assert np.array_equal(sn.view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("pow2", [False, True])
def test_power_of_two_equivariance(pow2):
    x, _ = synth.linear_inputs("tiny", 0)
    q, s = quant_act_ref(x, pow2)
    for j in (-7, -1, 1, 5, 20):
        qj, sj = quant_act_ref((x.float() * 2.0 ** j).to(torch.bfloat16), pow2)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj.astype(np.float64), s.astype(np.float64) * 2.0 ** j)


def test_permutation_equivariance():
    x, w = synth.linear_inputs("tiny", 0)
    g = synth.generator(2)
    pc = torch.randperm(128, generator=g)
    pr = torch.randperm(x.shape[0], generator=g)
    q, s = quant_act_ref(x)
    xp = x.clone()
    xp[:, :128] = x[:, pc]
    xp = xp[pr]
    qp, sp = quant_act_ref(xp)
    qe = q.copy()
    qe[:, :128] = q[:, pc.numpy()]
    assert np.array_equal(qp, qe[pr.numpy()])
    assert np.array_equal(sp, s[pr.numpy()])
    # weights: permuting rows inside a 128-row block and whole blocks
    qw, sw = quant_weight_ref(w)
    pw = torch.cat([torch.randperm(128, generator=g) + 128 * b for b in (2, 0, 1)])
    qwp, swp = quant_weight_ref(w[pw])
    assert np.array_equal(qwp, qw[pw.numpy()])
    assert np.array_equal(swp, sw[[2, 0, 1]])


def test_zero_group_and_signed_zeros():
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    x[0, :128] = -0.0
    x[1, 128:] = torch.randn(128).to(torch.bfloat16)
    q, s = quant_act_ref(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] > 0
    assert np.all(q[0, :128] == 0x80) and np.all(q[0, 128:] == 0x00) and np.all(q[1, :128] == 0x00)


def test_subnormal_scale():
    # amax so small that s = amax/448 is an fp32 subnormal
    x = torch.zeros(1, 128, dtype=torch.float32)
    x[0, 0] = 2.0 ** -130
    x[0, 1] = -(2.0 ** -133)
    x[0, 2] = 3 * 2.0 ** -133
    q, s = quant_act_ref(x.to(torch.bfloat16))
    assert 0 < s[0, 0] < np.float32(2.0 ** -126)
    assert float(s[0, 0]) == rn32_exact(Fraction(2) ** -130 / 448)
    assert q[0, 0] == 0x7E
    # pow2: 448 * 2**-138 >= 2**-130 > 448 * 2**-139, and 2**-130 / 2**-138 = 256
    q2, s2 = quant_act_ref(x.to(torch.bfloat16), pow2=True)
    assert float(s2[0, 0]) == 2.0 ** -138 and q2[0, 0] == 0x78
