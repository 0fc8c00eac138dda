"""GPU parity of the FP8 KV-cache path (Q/K/V recalibration maxima, scales,
quantize-and-write) against the oracle, through the C ABI: maxima, scales
and cache codes must match bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_codes_equal, assert_scales_equal, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def qkv_input(t, hq, hkv, d, gen, scales=(1.0, 2.0, 0.5)):
    """[T, (hq + 2 hkv) d] bf16 with Q, K, V drawn at different scales."""
    q = torch.randn(t, hq * d, generator=gen) * scales[0]
    k = torch.randn(t, hkv * d, generator=gen) * scales[1]
    v = torch.randn(t, hkv * d, generator=gen) * scales[2]
    return torch.cat([q, k, v], dim=1).to(torch.bfloat16)


def amax_of(fb, qkv, hq, hkv, d):
    amax, check = guarded((3,), torch.float32, DEV)
    fb.qkv_amax(qkv.to(DEV), hq, hkv, d, amax=amax, reset=True)
    check()
    return amax.cpu().numpy()


# T spans one row, fewer rows than workgroups, more rows than workgroups
# (2048: the grid-stride loop), and rows wider than one 1024-unit pass
# (Hq = 64: 1280 units per row); D = 8 is the smallest head.
@pytest.mark.parametrize("t,hq,hkv,d", [(1, 1, 1, 8), (37, 32, 8, 128), (5, 4, 2, 64), (4100, 8, 2, 128),
                                        (3, 64, 8, 128), (19, 7, 3, 24)])
def test_qkv_amax(fp8blk_lib, t, hq, hkv, d):
    qkv = qkv_input(t, hq, hkv, d, synth.generator(60, t + hq))
    got = amax_of(fp8blk_lib, qkv, hq, hkv, d)
    assert_scales_equal(got, oracle.qkv_amax_ref(qkv, hq, hkv, d).astype(np.float32), "qkv amax")


def test_qkv_amax_planted_and_chunked(fp8blk_lib):
    """Maxima planted at section edges; the batch fed in chunks (reset on
    the first) equals the whole batch; an all-zero chunk changes nothing."""
    fb = fp8blk_lib
    hq, hkv, d, t = 32, 8, 128, 600
    x = qkv_input(t, hq, hkv, d, synth.generator(61)).float()
    x[123, hq * d - 1] = -900.0            # last Q column
    x[7, hq * d] = 2.0 ** 18               # first K column
    x[599, (hq + 2 * hkv) * d - 1] = -2e-3 # V stays small
    x[:, (hq + hkv) * d:] *= 1e-3
    qkv = x.to(torch.bfloat16)
    ref = oracle.qkv_amax_ref(qkv, hq, hkv, d).astype(np.float32)
    assert list(ref[:2]) == [900.0, 2.0 ** 18]
    amax = torch.empty(3, dtype=torch.float32, device=DEV)
    dq = qkv.to(DEV)
    for i, (a, b) in enumerate([(0, 100), (100, 101), (101, 450), (450, 600)]):
        fb.qkv_amax(dq[a:b], hq, hkv, d, amax=amax, reset=(i == 0))
    fb.qkv_amax(torch.zeros(50, (hq + 2 * hkv) * d, dtype=torch.bfloat16, device=DEV), hq, hkv, d,
                amax=amax, reset=False)
    torch.cuda.synchronize()
    assert_scales_equal(amax.cpu().numpy(), ref, "chunked amax")
    # reset with no rows zeroes the maxima
    fb.fp8blk_qkv_amax(None, 0, hq, hkv, d, amax.data_ptr(), 1, fb._stream(amax.device))
    torch.cuda.synchronize()
    assert amax.cpu().tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("pow2", [False, True])
def test_kv_scales(fp8blk_lib, pow2):
    """Every positive finite bf16 value as a maximum, plus zero."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    got = fp8blk_lib.kv_scales(torch.from_numpy(amax.copy()).to(DEV), pow2)
    torch.cuda.synchronize()
    assert_scales_equal(got.cpu().numpy(), oracle.kv_scales_ref(amax.astype(np.float64), pow2), "kv scales")


def slot_rows(cache):
    """[num_blocks, Hkv, bs, D] paged cache -> [num_slots, Hkv*D] rows by slot (a copy)."""
    nblk, hkv, bs, d = cache.shape
    return cache.permute(0, 2, 1, 3).reshape(nblk * bs, hkv * d)


def run_write(fb, k, v, slot, num_slots, ks, vs, hkv, bs, canary=(0xA5, 0x5A)):
    """k, v: [T, Hkv*D] bf16 device views (row stride may exceed the width);
    caches of num_slots / bs head-major pages of bs tokens."""
    t, w = k.shape
    shape = (num_slots // bs, hkv, bs, w // hkv)
    kc, ckk = guarded(shape, torch.uint8, DEV)
    vc, cvv = guarded(shape, torch.uint8, DEV)
    kc.fill_(canary[0])
    vc.fill_(canary[1])
    fb.kv_cache_write(k, v, torch.as_tensor(slot, dtype=torch.int64).to(DEV),
                      torch.tensor([ks], dtype=torch.float32, device=DEV),
                      torch.tensor([vs], dtype=torch.float32, device=DEV), kc, vc)
    ckk()
    cvv()
    return kc.cpu().numpy(), vc.cpu().numpy()


def check_write(fb, qkv, hq, hkv, d, slot, num_slots, ks, vs, bs):
    """K and V read straight out of the qkv buffer (row stride > width)."""
    dq = qkv.to(DEV)
    k = dq[:, hq * d:(hq + hkv) * d]
    v = dq[:, (hq + hkv) * d:]
    kc, vc = run_write(fb, k, v, slot, num_slots, ks, vs, hkv, bs)
    canary_k = np.full((num_slots // bs, hkv, bs, d), 0xA5, np.uint8)
    canary_v = np.full((num_slots // bs, hkv, bs, d), 0x5A, np.uint8)
    live = np.where(np.asarray(slot) < num_slots, np.asarray(slot), -1)
    rk, rv = oracle.kv_cache_write_ref(qkv[:, hq * d:(hq + hkv) * d], qkv[:, (hq + hkv) * d:], live,
                                       canary_k, canary_v, ks, vs)
    assert_codes_equal(kc, rk, "k cache")
    assert_codes_equal(vc, rv, "v cache")


@pytest.mark.parametrize("t,hq,hkv,d,bs", [(1, 1, 1, 8, 1), (13, 32, 8, 128, 16), (70, 4, 2, 64, 8),
                                           (9, 2, 1, 1032, 3), (40, 8, 3, 24, 5)])
def test_kv_cache_write(fp8blk_lib, t, hq, hkv, d, bs):
    """Scales calibrated on the first half of the tokens (the rest may
    saturate), slots a shuffled subset with padding (-1) and slots past the
    cache (skipped); pages of bs tokens, powers of two and not. d = 1032
    gives rows of 129 units: a partial second pass; hkv = 3 with d = 24 puts
    several heads in one pass."""
    gen = synth.generator(62, t + d)
    qkv = qkv_input(t, hq, hkv, d, gen)
    half = max(1, t // 2)
    amax = oracle.qkv_amax_ref(qkv[:half], hq, hkv, d)
    ks, vs = (float(s) for s in oracle.kv_scales_ref(amax[1:]))
    num_slots = (2 * t + 3 + bs - 1) // bs * bs
    slot = torch.randperm(num_slots, generator=gen)[:t].numpy().astype(np.int64)
    slot[::5] = -1
    if t > 3:
        slot[3] = num_slots + 7              # past the cache: skipped
    check_write(fp8blk_lib, qkv, hq, hkv, d, slot, num_slots, ks, vs, bs)


def test_kv_cache_write_special_scales(fp8blk_lib):
    """Zero scale (codes +-0), tiny scales (every quotient saturates, many
    beyond the fp32 range), huge scales (above 2^126, where the kernel
    divides) and a scale that puts values exactly on E4M3 rounding
    midpoints."""
    hq, hkv, d, t = 2, 1, 128, 6
    qkv = qkv_input(t, hq, hkv, d, synth.generator(63))
    slot = np.arange(t, dtype=np.int64)[::-1].copy()
    check_write(fp8blk_lib, qkv, hq, hkv, d, slot, t, 0.0, 0.0, 3)
    check_write(fp8blk_lib, qkv, hq, hkv, d, slot, t, float(np.float32(1e-40)), float(np.float32(2.0 ** -100)), 3)
    big = qkv_input(t, hq, hkv, d, synth.generator(68), scales=(1e37, 1e37, 3e36))
    check_write(fp8blk_lib, big, hq, hkv, d, slot, t, float(np.float32(2.0 ** 127)), float(np.float32(3e35)), 2)
    mids = (oracle.decode_table()[:0x7E] + oracle.decode_table()[1:0x7F]) / 2
    vals = np.resize(np.concatenate([mids, -mids]), (t, (hq + 2 * hkv) * d))
    qkv2 = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    check_write(fp8blk_lib, qkv2, hq, hkv, d, slot, t, 1.0, 0.5, 6)


def test_recalibrate_then_write_end_to_end(fp8blk_lib):
    """qkv_amax over chunks -> kv_scales -> kv_cache_write, all on the
    device, against the oracle chain."""
    fb = fp8blk_lib
    hq, hkv, d, t = 32, 8, 128, 300
    qkv = qkv_input(t, hq, hkv, d, synth.generator(64), scales=(3.0, 1.5, 0.25))
    dq = qkv.to(DEV)
    amax = fb.qkv_amax(dq[:128], hq, hkv, d)
    fb.qkv_amax(dq[128:], hq, hkv, d, amax=amax, reset=False)
    scales = fb.kv_scales(amax)
    slot = torch.randperm(4 * t, generator=synth.generator(65))[:t].to(DEV)
    kc = torch.full((4 * t // 16, hkv, 16, d), 0xA5, dtype=torch.uint8, device=DEV)
    vc = torch.full((4 * t // 16, hkv, 16, d), 0xA5, dtype=torch.uint8, device=DEV)
    fb.kv_cache_write(dq[:, hq * d:(hq + hkv) * d], dq[:, (hq + hkv) * d:], slot, scales[1:2], scales[2:3], kc, vc)
    torch.cuda.synchronize()
    ref_amax = oracle.qkv_amax_ref(qkv, hq, hkv, d)
    ref_s = oracle.kv_scales_ref(ref_amax)
    assert_scales_equal(scales.cpu().numpy(), ref_s, "end-to-end scales")
    c0 = np.full((4 * t // 16, hkv, 16, d), 0xA5, np.uint8)
    rk, rv = oracle.kv_cache_write_ref(qkv[:, hq * d:(hq + hkv) * d], qkv[:, (hq + hkv) * d:],
                                       slot.cpu().numpy(), c0, c0, ref_s[1], ref_s[2])
    assert_codes_equal(kc.cpu().numpy(), rk, "end-to-end k cache")
    assert_codes_equal(vc.cpu().numpy(), rv, "end-to-end v cache")


def test_full_size_prefill(fp8blk_lib):
    """Llama-3.1-8B attention shapes at the prefill batch (T = 16384,
    Hq = 32, Hkv = 8, D = 128): maxima exactly, the cache on sampled tokens,
    untouched slots keep their canary."""
    fb = fp8blk_lib
    qkv, (hq, hkv, d) = synth.kv_inputs("llama8b_prefill")
    t = qkv.shape[0]
    dq = qkv.to(DEV)
    amax = fb.qkv_amax(dq, hq, hkv, d)
    scales = fb.kv_scales(amax)
    num_slots = 2 * t
    slot = torch.randperm(num_slots, generator=synth.generator(66))[:t]
    kc = torch.full((num_slots // 16, hkv, 16, d), 0xA5, dtype=torch.uint8, device=DEV)
    vc = torch.full((num_slots // 16, hkv, 16, d), 0xA5, dtype=torch.uint8, device=DEV)
    fb.kv_cache_write(dq[:, hq * d:(hq + hkv) * d], dq[:, (hq + hkv) * d:], slot.to(DEV), scales[1:2],
                      scales[2:3], kc, vc)
    torch.cuda.synchronize()
    ref_amax = oracle.qkv_amax_ref(qkv, hq, hkv, d)
    assert_scales_equal(amax.cpu().numpy(), ref_amax.astype(np.float32), "full-size amax")
    ref_s = oracle.kv_scales_ref(ref_amax)
    rows = np.unique(np.concatenate([[0, 1, t - 1, t // 2],
                                     torch.randint(0, t, (64,), generator=synth.generator(67)).numpy()]))
    r = torch.from_numpy(rows)
    sl = slot[r].to(DEV)
    krows, vrows = slot_rows(kc), slot_rows(vc)   # by slot: page sl // 16, row sl % 16, every head
    assert_codes_equal(krows[sl].cpu().numpy(), oracle.kv_quantize_ref(qkv[r, hq * d:(hq + hkv) * d], ref_s[1]),
                       "sampled k cache")
    assert_codes_equal(vrows[sl].cpu().numpy(), oracle.kv_quantize_ref(qkv[r, (hq + hkv) * d:], ref_s[2]),
                       "sampled v cache")
    untouched = torch.ones(num_slots, dtype=torch.bool)
    untouched[slot] = False
    assert bool(torch.all(krows[untouched.to(DEV)] == 0xA5)) and bool(torch.all(vrows[untouched.to(DEV)] == 0xA5))
