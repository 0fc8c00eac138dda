"""Pins of the oracle's E4M3 codec (CPU only).

The codec is pinned to (a) torch's own float8_e4m3fn implementation, a
library routine independent of the oracle, (b) landmarks that follow from
the OCP E4M3 format definition, and (c) the exhaustive nearest-code search.
"""

import numpy as np
import pytest
import torch

from oracle import E4M3_MAX, decode, decode_table, encode, encode_bruteforce


def _bf16_all_finite():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)].astype(np.float64)


def test_decode_table_matches_torch_float8_e4m3fn():
    ours = decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], theirs[fin])
    # sign of zero too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(theirs[fin]))


def test_decode_landmarks():
    t = decode_table()
    assert t[0x38] == 1.0
    assert t[0x40] == 2.0
    assert t[0x78] == 256.0
    assert t[0x7E] == 448.0 == E4M3_MAX
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2      # no other NaN, no infinities
    assert not np.any(np.isinf(t))
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)      # strictly increasing magnitudes


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode(decode(codes)), codes)


def test_encode_matches_bruteforce_on_all_bf16():
    v = _bf16_all_finite()
    assert np.array_equal(encode(v), encode_bruteforce(v))


def _midpoints_pm_ulp():
    t = decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)   # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (t[:-1] + t[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    extra = np.array([448, 448.00003, 460, 463.99997, 464, 464.00003, 480, 1e30, 3.4e38,
                      2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45], dtype=np.float32)
    v = np.concatenate([mids, up, dn, extra])
    return np.concatenate([v, -v]).astype(np.float64), mids


def test_encode_matches_bruteforce_at_midpoints():
    v, mids = _midpoints_pm_ulp()
    assert np.array_equal(encode(v), encode_bruteforce(v))
    # ties go to the even code, one ulp either side goes to the neighbour
    codes = encode(mids.astype(np.float64))
    assert np.all(codes % 2 == 0)
    lo = np.arange(0x7E, dtype=np.uint8)
    assert np.array_equal(encode(np.nextafter(mids, np.float32(0)).astype(np.float64)), lo)
    assert np.array_equal(encode(np.nextafter(mids, np.float32(np.inf)).astype(np.float64)), lo + 1)


def test_encode_saturates_and_never_emits_nan():
    big = np.array([448.0, 449.0, 464.0, 500.0, 1e10, 3e38])
    assert np.all(encode(big) == 0x7E)
    assert np.all(encode(-big) == 0xFE)
    v = _bf16_all_finite()
    c = encode(v)
    assert not np.any((c == 0x7F) | (c == 0xFF))


def test_encode_sign_of_zero():
    v = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10)])
    assert list(encode(v)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        encode(np.array([np.nan]))
    with pytest.raises(ValueError):
        encode(np.array([np.inf]))


def test_encode_matches_torch_cast_in_range():
    """torch's fp32 -> float8_e4m3fn cast is round-to-nearest-even within
    range; values are clamped to +-448 first because torch does not saturate.
    Exact zeros are left out (their sign is pinned above)."""
    g = torch.Generator().manual_seed(1234)
    mag = torch.exp2(torch.empty(200000).uniform_(-14, 9.5, generator=g))
    sgn = torch.where(torch.rand(200000, generator=g) < 0.5, -1.0, 1.0)
    x = (mag * sgn).to(torch.float32)
    mids, _ = _midpoints_pm_ulp()
    x = torch.cat([x, torch.from_numpy(mids.astype(np.float32))])
    x = x[x != 0]
    theirs = x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = encode(x.numpy().astype(np.float64))
    nz = decode(theirs) != 0
    assert np.array_equal(ours[nz], theirs[nz])
    # where torch gives zero, ours gives a zero of the input's sign
    assert np.all(decode(ours[~nz]) == 0)
