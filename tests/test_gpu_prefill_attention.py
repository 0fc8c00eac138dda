"""GPU parity of the FP8 prefill attention over the paged FP8 KV cache
against the oracle, through the C ABI. The caches are written by the
library's own cache write from seeded bf16 K and V (scales calibrated on
the data); the oracle reads the same cache bytes. Outputs within
|y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref), rms over the call's output."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_quant_amd as fb
import oracle
import synth
from tests.gpu_util import assert_within_tolerance, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def build(seqs, hq, hkv, seed=0, bs=16, k_ramp=None):
    """Inputs and the FP8 cache; with ``k_ramp`` each cached token t of a
    sequence has its key scaled by 1 + t / k_ramp (row maxima that keep
    rising along the sequence)."""
    a = synth.prefill_inputs(seqs, hq, hkv, D, bs, seed)
    if k_ramp is not None:
        t = torch.cat([torch.arange(int(n), dtype=torch.float32) for n in a["context_lens"].tolist()])
        a["k"] = (a["k"].float() * (1.0 + t / k_ramp)[:, None]).to(torch.bfloat16)
    k, v = a["k"].to(DEV), a["v"].to(DEV)
    num_slots = a["num_slots"]
    kc = torch.zeros(num_slots // bs, hkv, bs, D, dtype=torch.uint8, device=DEV)
    vc = torch.zeros(num_slots // bs, hkv, bs, D, dtype=torch.uint8, device=DEV)
    amax = torch.stack([a["q"].float().abs().max(), a["k"].float().abs().max(), a["v"].float().abs().max()])
    scales = fb.kv_scales(amax.to(DEV))
    if k.shape[0]:
        fb.kv_cache_write(k, v, a["slot"].to(DEV), scales[1:2], scales[2:3], kc, vc)
    torch.cuda.synchronize()
    return a, kc, vc, scales


def run(a, kc, vc, scales, sm=None, max_seqlen=None, q=None):
    tq, hq = a["q"].shape[0], a["q"].shape[1]
    out, check = guarded((tq, hq, D), torch.bfloat16, DEV)
    out.fill_(0)
    fb.prefill_attention(a["q"].to(DEV) if q is None else q, a["cu_seqlens_q"].to(DEV),
                         a["max_seqlen_q"] if max_seqlen is None else max_seqlen, kc, vc,
                         a["block_table"].to(DEV), a["block_size"], a["context_lens"].to(DEV), scales[0:1],
                         scales[1:2], scales[2:3], sm_scale=sm, out=out)
    check()
    return out


def reference(a, kc, vc, scales, sm=None):
    s = scales.cpu().numpy()
    return oracle.prefill_attention_ref(a["q"], a["cu_seqlens_q"].numpy(), kc.cpu().numpy(), vc.cpu().numpy(),
                                        a["block_table"].numpy(), a["block_size"], a["context_lens"].numpy(),
                                        s[0], s[1], s[2], sm)


# (new tokens, context length) per sequence: one token, a fresh prompt inside
# one 64-token tile, exactly one tile, one past it, a chunk of new tokens
# after cached ones (chunked prefill), several token blocks of a workgroup,
# a sequence with no new tokens, a decode-like single token over a long
# context, and more new tokens than one workgroup block for every head group
SEQS = [(1, 1), (5, 5), (64, 64), (65, 65), (130, 300), (200, 200), (0, 50), (1, 777), (17, 1000), (129, 129)]


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (32, 8), (32, 4)])
def test_prefill_sequences_and_groups(fp8blk_lib, hq, hkv):
    a, kc, vc, sc = build(SEQS, hq, hkv, seed=hq + hkv)
    print("prefill attention hq=%d hkv=%d total_q=%d" % (hq, hkv, a["q"].shape[0]), flush=True)
    out = run(a, kc, vc, sc)
    ref = reference(a, kc, vc, sc)
    worst = assert_within_tolerance(out.float().cpu().numpy().reshape(-1), ref.reshape(-1), what="prefill attention")
    print("worst error / tolerance: %.3f" % worst, flush=True)


def test_explicit_scale_and_strided_queries(fp8blk_lib):
    """sm_scale given; q read through a row stride (a view into a wider
    projection output, as the qkv linear produces)."""
    seqs = [(40, 90), (70, 70)]
    a, kc, vc, sc = build(seqs, 32, 8, seed=3)
    tq = a["q"].shape[0]
    wide = torch.zeros(tq, 48 * D, dtype=torch.bfloat16, device=DEV)
    wide[:, :32 * D] = a["q"].reshape(tq, -1).to(DEV)
    out = run(a, kc, vc, sc, sm=0.05, q=wide[:, :32 * D])
    ref = reference(a, kc, vc, sc, sm=0.05)
    assert_within_tolerance(out.float().cpu().numpy().reshape(-1), ref.reshape(-1), what="prefill attention sm")


@pytest.mark.parametrize("sm,ramp", [(1.0, None), (0.3, 64.0), (1.0, 16.0)])
def test_large_score_jumps(fp8blk_lib, sm, ramp):
    """Row maxima that rise by far more than 2^8 (8 in log2 units) between
    KV tiles, where the kernel moves its reference maximum and rescales the
    accumulators: a large sm_scale (scores of standard deviation ~23, i.e.
    ~33 in log2 units) and keys growing along the sequence."""
    seqs = [(130, 300), (200, 200), (64, 64), (1, 777)]
    a, kc, vc, sc = build(seqs, 32, 8, seed=7, k_ramp=ramp)
    out = run(a, kc, vc, sc, sm=sm)
    ref = reference(a, kc, vc, sc, sm=sm)
    worst = assert_within_tolerance(out.float().cpu().numpy().reshape(-1), ref.reshape(-1),
                                    what="prefill attention (score jumps)")
    print("sm %.2f ramp %s: worst error / tolerance %.3f" % (sm, ramp, worst), flush=True)


@pytest.mark.parametrize("sm", [-0.2, 0.0])
def test_negative_and_zero_softmax_scale(fp8blk_lib, sm):
    """A negative scale (the largest products get the smallest weights) and
    a zero scale (uniform weights over each token's context); these take
    the path that scales every score, as masked tiles do."""
    seqs = [(130, 300), (64, 64), (5, 5)]
    a, kc, vc, sc = build(seqs, 32, 8, seed=8)
    out = run(a, kc, vc, sc, sm=sm)
    ref = reference(a, kc, vc, sc, sm=sm)
    assert_within_tolerance(out.float().cpu().numpy().reshape(-1), ref.reshape(-1), what="prefill attention sm %g" % sm)


@pytest.mark.parametrize("bs", [12, 48])
def test_block_size_not_a_power_of_two(fp8blk_lib, bs):
    """Pages of 12 or 48 tokens: the kernel divides token positions by the
    block size instead of shifting (a power of two takes the shift)."""
    seqs = [(130, 300), (64, 64), (1, 777), (17, 1000)]
    a, kc, vc, sc = build(seqs, 16, 4, seed=9, bs=bs)
    out = run(a, kc, vc, sc)
    ref = reference(a, kc, vc, sc)
    assert_within_tolerance(out.float().cpu().numpy().reshape(-1), ref.reshape(-1), what="block size %d" % bs)


def test_tokens_past_max_seqlen_are_left_alone(fp8blk_lib):
    """max_seqlen_q below a sequence's new tokens: the tokens past it are not
    computed (their rows keep what the caller put there); the others match."""
    seqs = [(300, 300), (20, 40)]
    a, kc, vc, sc = build(seqs, 8, 4, seed=4)
    out = run(a, kc, vc, sc, max_seqlen=256)
    ref = reference(a, kc, vc, sc)
    o = out.float().cpu().numpy()
    assert np.all(o[256:300] == 0)
    keep = np.r_[0:256, 300:320]
    assert_within_tolerance(o[keep].reshape(-1), ref[keep].reshape(-1), what="prefill attention (max_seqlen)")


def test_deterministic(fp8blk_lib):
    a, kc, vc, sc = build([(150, 400), (90, 90)], 32, 8, seed=5)
    o1, o2 = run(a, kc, vc, sc), run(a, kc, vc, sc)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_full_size_sampled(fp8blk_lib):
    """The Llama-3.1-8B prefill step (8 sequences x 2048 new tokens, 32 query
    and 8 KV heads): sampled new tokens against the oracle, each on the
    context it attends to (one new token at position p over p + 1 cached
    tokens is exactly that token's prefill row)."""
    seqs = [(2048, 2048)] * 8
    a, kc, vc, sc = build(seqs, 32, 8, seed=6)
    out = run(a, kc, vc, sc)
    o = out.float().cpu().numpy()
    s = sc.cpu().numpy()
    kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()
    gen = synth.generator(0x62)
    picks = [(0, 0), (0, 63), (0, 64), (3, 2047), (7, 1000)] + [
        (int(b), int(p)) for b, p in zip(torch.randint(0, 8, (15,), generator=gen),
                                         torch.randint(0, 2048, (15,), generator=gen))]
    got, want = [], []
    for b, p in picks:
        row = int(a["cu_seqlens_q"][b]) + p
        ref = oracle.prefill_attention_ref(a["q"][row:row + 1], np.array([0, 1]), kcn, vcn,
                                           a["block_table"][b:b + 1].numpy(), 16, np.array([p + 1]), s[0], s[1], s[2])
        got.append(o[row])
        want.append(ref[0])
    rms = float(np.sqrt(np.mean(np.square(np.stack(want)))))
    worst = assert_within_tolerance(np.stack(got).reshape(-1), np.stack(want).reshape(-1), rms=rms,
                                    what="prefill attention full size (sampled)")
    print("worst error / tolerance: %.3f" % worst, flush=True)
