"""Pins of the FP8 KV-cache oracle: Q/K/V maxima, per-tensor quantization,
the cache write.

Each check comes from something other than the oracle's own formulas: maxima
planted at known places and a plain Python scan, the already pinned 1x128
group quantizer (a tensor that is one group must quantize identically), the
saturation and zero-scale cases of the format, the dequantization error
bound of E4M3, and a per-token loop for the cache write.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.kv_cache import kv_cache_write_ref, kv_quantize_ref, kv_scales_ref, qkv_amax_ref


def bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_amax_planted_maxima():
    hq, hkv, d, t = 4, 2, 16, 5
    c = (hq + 2 * hkv) * d
    x = np.zeros((t, c))
    x[2, 5] = -3.5                     # Q section
    x[4, hq * d + 7] = 1000.0          # K section
    x[0, (hq + hkv) * d + 31] = -2.0 ** -100   # V section (tiny, negative)
    x[1, hq * d - 1] = 2.0             # last Q column
    a = qkv_amax_ref(bf16(x), hq, hkv, d)
    assert list(a) == [3.5, 1000.0, 2.0 ** -100]


def test_amax_matches_python_scan():
    rng = np.random.default_rng(7)
    hq, hkv, d, t = 3, 1, 8, 6
    x = bf16(rng.standard_normal((t, (hq + 2 * hkv) * d)) * 5)
    vals = oracle.bf16_values(x)
    best = [0.0, 0.0, 0.0]
    for r in range(t):
        for col in range(vals.shape[1]):
            sec = 0 if col < hq * d else (1 if col < (hq + hkv) * d else 2)
            best[sec] = max(best[sec], abs(float(vals[r, col])))
    assert list(qkv_amax_ref(x, hq, hkv, d)) == best
    assert list(qkv_amax_ref(bf16(np.zeros((0, (hq + 2 * hkv) * d))), hq, hkv, d)) == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("pow2", [False, True])
def test_one_group_tensor_equals_group_quantizer(pow2):
    """A [1, 128] tensor is one 1x128 group: per-tensor scale and codes must
    equal the pinned group quantizer's."""
    rng = np.random.default_rng(8)
    for scale in (1.0, 1e-20, 3e15):
        x = bf16(rng.standard_normal((1, 128)) * scale)
        q_ref, s_ref = oracle.quant_act_ref(x, pow2)
        s = kv_scales_ref([np.abs(oracle.bf16_values(x)).max()], pow2)
        assert s[0] == s_ref[0, 0]
        assert np.array_equal(kv_quantize_ref(x, s[0])[0], q_ref[0])


def test_saturation_and_zero_scale():
    s = np.float32(0.25)
    x = bf16([448 * 0.25, 464 * 0.25, 1e30, -1e30, -0.0, 0.0, 3e38])
    q = kv_quantize_ref(x, s)
    assert list(q) == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x7E]
    # a tiny scale: quotients beyond the fp32 range still saturate
    assert list(kv_quantize_ref(bf16([1e30, -2.0]), np.float32(1e-40))) == [0x7E, 0xFE]
    assert list(kv_quantize_ref(bf16([1.0, -1.0, 0.0, -0.0]), 0.0)) == [0x00, 0x80, 0x00, 0x80]


def test_dequantization_error_bound():
    """In range, dec(code) * s is within half an E4M3 step of x: relative
    2^-4 for normal codes, absolute 2^-10 * s for subnormal ones."""
    rng = np.random.default_rng(9)
    x = bf16(rng.standard_normal(4096) * 3)
    xv = oracle.bf16_values(x)
    s = kv_scales_ref([np.abs(xv).max()])[0]
    dq = oracle.decode(kv_quantize_ref(x, s)) * float(s)
    tol = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)
    assert np.all(np.abs(dq - xv) <= tol)


def test_cache_write_matches_token_loop():
    """Head h of token i lands at page slot // 4, head h, row slot % 4 of the
    head-major paged caches; every other row keeps its old bytes."""
    rng = np.random.default_rng(10)
    t, hkv, d, bs, nblk = 9, 2, 8, 4, 5
    k = bf16(rng.standard_normal((t, hkv * d)))
    v = bf16(rng.standard_normal((t, hkv * d)) * 7)
    slot = np.array([3, -1, 0, 19, 7, -1, 11, 4, 15])
    kc0 = np.full((nblk, hkv, bs, d), 0xA5, np.uint8)
    vc0 = np.full((nblk, hkv, bs, d), 0x5A, np.uint8)
    ks, vs = np.float32(0.01), np.float32(0.02)
    kc, vc = kv_cache_write_ref(k, v, slot, kc0, vc0, ks, vs)
    kv_, vv_ = oracle.bf16_values(k), oracle.bf16_values(v)
    for i in range(t):
        if slot[i] < 0:
            continue
        page, row = divmod(int(slot[i]), bs)
        for h in range(hkv):
            for j in range(d):
                assert kc[page, h, row, j] == kv_quantize_ref(bf16([kv_[i, h * d + j]]), ks)[0]
                assert vc[page, h, row, j] == kv_quantize_ref(bf16([vv_[i, h * d + j]]), vs)[0]
    for sl in np.setdiff1d(np.arange(nblk * bs), slot[slot >= 0]):
        page, row = divmod(int(sl), bs)
        assert np.all(kc[page, :, row] == 0xA5) and np.all(vc[page, :, row] == 0x5A)
    with pytest.raises(ValueError):
        kv_cache_write_ref(k, v, np.array([1, 1, 2, 3, 4, 5, 6, 7, 8]), kc0, vc0, ks, vs)
    with pytest.raises(ValueError):
        kv_cache_write_ref(k, v, np.array([20, -1, 0, 1, 2, 3, 4, 5, 6]), kc0, vc0, ks, vs)
