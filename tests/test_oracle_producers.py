"""Pins of the fp64 producers (RMSNorm, SiLU(gate)*up) and bf16 rounding.

Each check comes from the mathematics, not from re-typing the oracle's
formula: closed forms for constant and one-hot rows, the mean-square
invariant, exact power-of-two scale invariance, the SiLU identity and its
minimum (Lambert W), the [gate | up] layout, and bf16 rounding at every
midpoint between neighbouring bf16 values.
"""

import numpy as np
import pytest
import torch
from scipy.special import lambertw

import oracle
from oracle.producers import rmsnorm_ref, round_bf16, silu_mul_ref


def bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_rmsnorm_constant_row_closed_form():
    eps = 1e-5
    for c in (1.0, -3.0, 0.0625, 448.0):
        x = bf16(np.full((1, 256), c))
        y = rmsnorm_ref(x, bf16(np.ones(256)), eps)
        e = float(np.float32(eps))
        assert np.allclose(y, c / np.sqrt(c * c + e), rtol=1e-14, atol=0)


def test_rmsnorm_one_hot_row():
    k, v, eps = 512, 7.5, 1e-6
    xv = np.zeros((1, k)); xv[0, 37] = v
    g = np.linspace(0.5, 2.0, k).astype(np.float32)
    y = rmsnorm_ref(bf16(xv), bf16(g), eps)
    gv = oracle.bf16_values(bf16(g))
    e = float(np.float32(eps))
    assert y[0, 37] == pytest.approx(v / np.sqrt(v * v / k + e) * gv[37], rel=1e-14)
    assert np.all(np.delete(y[0], 37) == 0)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = bf16(rng.standard_normal((8, 384)))
    ones = bf16(np.ones(384))
    y = rmsnorm_ref(x, ones, 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-13)
    # scaling x by a power of two scales the mean square exactly: y unchanged bit for bit
    y2 = rmsnorm_ref(bf16(oracle.bf16_values(x) * 2.0 ** -20), ones, 0.0)
    assert np.array_equal(y, y2)
    # gamma enters linearly
    g = bf16(rng.uniform(0.5, 2, 384))
    assert np.allclose(rmsnorm_ref(x, g, 1e-5), rmsnorm_ref(x, ones, 1e-5) * oracle.bf16_values(g)[None],
                       rtol=1e-15, atol=0)


def test_silu_identities():
    rng = np.random.default_rng(4)
    g = rng.uniform(-30, 30, (4, 256))
    ones = np.ones_like(g)
    sp = silu_mul_ref(bf16(np.concatenate([g, ones], axis=1)))
    sm = silu_mul_ref(bf16(np.concatenate([-g, ones], axis=1)))
    gv = oracle.bf16_values(bf16(g))
    # sigma(g) + sigma(-g) = 1  =>  silu(g) - silu(-g) = g
    assert np.allclose(sp - sm, gv, rtol=0, atol=1e-13 * np.abs(gv).max())
    z = silu_mul_ref(bf16(np.concatenate([np.zeros((1, 128)), np.ones((1, 128))], axis=1)))
    assert np.all(z == 0)
    big = silu_mul_ref(bf16(np.concatenate([np.full((1, 128), 40.0), np.ones((1, 128))], axis=1)))
    assert np.allclose(big, 40.0, rtol=1e-15, atol=0)


def test_silu_minimum_is_minus_lambert_w():
    w = float(lambertw(np.exp(-1.0)).real)        # W(1/e)
    xstar, fmin = -(1.0 + w), -w
    # the oracle on an fp64 grid around the minimiser (through the bf16 input
    # path, so evaluate the formula's float64 core on bf16-exact points)
    xs = oracle.bf16_values(bf16(np.linspace(xstar - 0.05, xstar + 0.05, 201)))
    vals = silu_mul_ref(bf16(np.concatenate([xs[None], np.ones((1, xs.size))], axis=1)))[0]
    assert vals.min() >= fmin - 1e-15
    assert vals.min() == pytest.approx(fmin, abs=2e-5)   # bf16 grid spacing near 1.28 is 2**-7


def test_silu_layout_gate_then_up():
    rng = np.random.default_rng(5)
    g = rng.standard_normal((3, 128)); u = rng.standard_normal((3, 128))
    h = silu_mul_ref(bf16(np.concatenate([g, u], axis=1)))
    gv, uv = oracle.bf16_values(bf16(g)), oracle.bf16_values(bf16(u))
    # swapping the halves changes the result unless u == g
    hs = silu_mul_ref(bf16(np.concatenate([u, g], axis=1)))
    assert not np.allclose(h, hs)
    # with u == 1 the result is silu(g), with u == 2 exactly twice that
    h1 = silu_mul_ref(bf16(np.concatenate([g, np.ones_like(g)], axis=1)))
    h2 = silu_mul_ref(bf16(np.concatenate([g, 2 * np.ones_like(g)], axis=1)))
    assert np.array_equal(h2, 2 * h1)
    assert np.allclose(h, h1 * uv, rtol=1e-15, atol=0)
    assert np.all(np.sign(h1) == np.sign(gv))


def test_round_bf16_at_every_midpoint():
    """Between each pair of neighbouring positive finite bf16 values, the
    midpoint rounds to the one with an even last bit, points just below /
    above it to the lower / upper value; the bit patterns are those of the
    rounded values."""
    lo_bits = np.arange(0, 0x7F7F, dtype=np.uint32)          # up to the largest finite - 1
    lo = (lo_bits << 16).view(np.float32).astype(np.float64)
    hi = ((lo_bits + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2                                      # exact in float64
    bits, vals = round_bf16(mid)
    even_lo = (lo_bits & 1) == 0
    assert np.array_equal(vals, np.where(even_lo, lo, hi))
    assert np.array_equal(bits.astype(np.uint32), np.where(even_lo, lo_bits, lo_bits + 1))
    below = mid - (hi - lo) * 2.0 ** -20
    above = mid + (hi - lo) * 2.0 ** -20
    assert np.array_equal(round_bf16(below)[1], lo)
    assert np.array_equal(round_bf16(above)[1], hi)
    # signs and zeros
    b, v = round_bf16(np.array([-0.0, 0.0, -mid[1000]]))
    assert list(b) == [0x8000, 0x0000, 0x8000 | int(np.where(even_lo, lo_bits, lo_bits + 1)[1000])]
    # overflow: the largest finite bf16 (odd last bit) and the midpoint to 2**128:
    # the midpoint ties to the even neighbour, infinity; just below it stays finite
    big = 3.3895313892515355e38
    half_ulp = 2.0 ** 119
    assert round_bf16(np.array([big + half_ulp]))[1][0] == np.inf
    assert round_bf16(np.array([big + half_ulp * 0.999]))[1][0] == big
