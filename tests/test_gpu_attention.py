"""GPU parity of the FP8 decode attention over the paged FP8 KV cache
against the oracle, through the C ABI. The caches are written by the
library's own cache write from seeded bf16 K and V; the oracle reads the same
cache bytes. Outputs within |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref)."""

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


def build(lens, hq, hkv, seed=0, bs=16, k_ramp=None):
    """Inputs on the device, caches filled by the cache write with scales
    calibrated on the data; with ``k_ramp`` each cached token t of a
    sequence has its key scaled by 1 + t / k_ramp."""
    a = synth.attention_inputs(lens, hq, hkv, D, bs, seed)
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


MODES = {"direct": dict(split=False), "split_auto": dict(split=True),
         "split_256": dict(split=True, split_tokens=256), "split_512": dict(split=True, split_tokens=512)}


def run(a, kc, vc, scales, sm=None, mode="split_auto"):
    b, hq = a["q"].shape[0], a["q"].shape[1]
    out, check = guarded((b, hq, D), torch.bfloat16, DEV)
    fb.decode_attention(a["q"].to(DEV), kc, vc, a["block_table"].to(DEV), a["block_size"],
                        a["context_lens"].to(DEV), scales[0:1], scales[1:2], scales[2:3], sm_scale=sm, out=out,
                        **MODES[mode])
    check()
    return out


def reference(a, kc, vc, scales, sm=None):
    s = scales.cpu().numpy()
    return oracle.decode_attention_ref(a["q"], kc.cpu().numpy(), vc.cpu().numpy(), a["block_table"].numpy(),
                                       a["block_size"], a["context_lens"].numpy(), s[0], s[1], s[2], sm)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (32, 8), (32, 4)])
def test_context_lengths_and_groups(fp8blk_lib, hq, hkv, mode):
    """Context lengths 0, 1, a partial 16-token subtile, one and two 64-token
    tiles, more tiles than waves, ragged tails, both sides of the 256- and
    512-token chunk edges; every head-group size; the direct path and the
    split path with the automatic and two explicit chunk sizes."""
    lens = [0, 1, 15, 64, 65, 300, 1000, 257, 255, 256, 511, 512, 513]
    a, kc, vc, sc = build(lens, hq, hkv, seed=hq + hkv)
    out = run(a, kc, vc, sc, mode=mode)
    ref = reference(a, kc, vc, sc)
    assert torch.all(out[0].float() == 0)
    assert_within_tolerance(out.float().cpu().numpy().reshape(len(lens), -1), ref.reshape(len(lens), -1),
                            what="decode attention (%s)" % mode)


def test_split_workspace_reuse_and_size(fp8blk_lib):
    """One workspace serves calls of different shapes in a row; the size
    query matches the chunking (partials of 130 floats per head and chunk)."""
    a, kc, vc, sc = build([700, 20, 1300], 32, 8, seed=11)
    b, mb = 3, a["block_table"].shape[1]
    need = fb.fp8blk_decode_attention_workspace_size(b, 32, 8, D, mb, 16, 256)
    assert need == b * 32 * ((mb * 16 + 255) // 256) * 130 * 4
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = reference(a, kc, vc, sc)
    for _ in range(2):
        out = torch.empty(b, 32, D, dtype=torch.bfloat16, device=DEV)
        fb.decode_attention(a["q"].to(DEV), kc, vc, a["block_table"].to(DEV), 16, a["context_lens"].to(DEV),
                            sc[0:1], sc[1:2], sc[2:3], out=out, split_tokens=256, workspace=ws)
        torch.cuda.synchronize()
        assert_within_tolerance(out.float().cpu().numpy().reshape(b, -1), ref.reshape(b, -1), what="reuse")
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(fb.Fp8BlkError):
        fb.decode_attention(a["q"].to(DEV), kc, vc, a["block_table"].to(DEV), 16, a["context_lens"].to(DEV),
                            sc[0:1], sc[1:2], sc[2:3], split_tokens=256, workspace=small)


def test_softmax_scale_and_block_size(fp8blk_lib):
    a, kc, vc, sc = build([33, 130, 7], 16, 4, seed=5, bs=8)
    for sm in (0.01, 0.3, -0.2, 0.0):
        out = run(a, kc, vc, sc, sm)
        assert_within_tolerance(out.float().cpu().numpy().reshape(3, -1), reference(a, kc, vc, sc, sm).reshape(3, -1),
                                what="sm_scale %g" % sm)


@pytest.mark.parametrize("bs", [12, 48])
@pytest.mark.parametrize("mode", ["direct", "split_256"])
def test_block_size_not_a_power_of_two(fp8blk_lib, bs, mode):
    """Pages of 12 or 48 tokens: the kernel divides token positions by the
    block size instead of shifting (a power of two takes the shift)."""
    a, kc, vc, sc = build([33, 130, 700, 1], 16, 4, seed=8, bs=bs)
    out = run(a, kc, vc, sc, mode=mode)
    assert_within_tolerance(out.float().cpu().numpy().reshape(4, -1), reference(a, kc, vc, sc).reshape(4, -1),
                            what="block size %d" % bs)


@pytest.mark.parametrize("mode", ["direct", "split_256"])
@pytest.mark.parametrize("sm,ramp", [(1.0, None), (0.3, 64.0), (1.0, 16.0)])
def test_large_score_jumps(fp8blk_lib, sm, ramp, mode):
    """Scores with a large spread and row maxima that keep rising along the
    context (a large sm_scale, keys growing with the token index): the
    scores must be exact products, or the softmax moves with their errors."""
    a, kc, vc, sc = build([1, 63, 300, 777, 1024], 32, 8, seed=9, k_ramp=ramp)
    out = run(a, kc, vc, sc, sm=sm, mode=mode)
    worst = assert_within_tolerance(out.float().cpu().numpy().reshape(-1), reference(a, kc, vc, sc, sm=sm).reshape(-1),
                                    what="decode attention (score jumps)")
    print("sm %.2f ramp %s %s: worst error / tolerance %.3f" % (sm, ramp, mode, worst), flush=True)


def test_single_token_is_its_value_row(fp8blk_lib):
    """One cached token: softmax weight 1, out = v8 * v_scale to a bf16 ulp."""
    a, kc, vc, sc = build([1, 1, 1], 8, 2, seed=6)
    out = run(a, kc, vc, sc).float().cpu().numpy()
    ref = reference(a, kc, vc, sc)
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("mode", ["direct", "split_256"])
def test_masked_tokens_are_skipped(fp8blk_lib, mode):
    """A negative block id, a block past the cache and a context longer than
    the block table: those tokens are left out, as if never cached."""
    a, kc, vc, sc = build([40, 50, 300], 8, 4, seed=7)
    table = a["block_table"].clone()
    table[0, 1] = -1                                   # tokens 16..31 of sequence 0
    table[1, 2] = a["num_slots"] // 16 + 5             # tokens 32..47 of sequence 1
    lens = a["context_lens"].clone()
    lens[2] = 300 + 16 * table.shape[1]                # past max_blocks * block_size
    b2 = dict(a, block_table=table, context_lens=lens)
    out = run(b2, kc, vc, sc, mode=mode).float().cpu().numpy()
    # the same attention on a cache holding only the kept tokens, repacked
    keep = {0: [t for t in range(40) if not 16 <= t < 32], 1: [t for t in range(50) if not 32 <= t < 48],
            2: list(range(16 * table.shape[1]))}
    assert table.shape[1] == 19                        # sequence 2's 300 tokens fill its whole table row
    kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()      # [pages, Hkv, 16, D]
    rows_k, rows_v, new_table, new_lens, nxt = [], [], [], [], 0
    width = max(len(v) for v in keep.values())
    for bi in range(3):
        ids = []
        for t in keep[bi]:
            blk = int(a["block_table"][bi, t // 16]) if t // 16 < table.shape[1] else -1
            if blk < 0:
                continue
            rows_k.append(kcn[blk, :, t % 16])
            rows_v.append(vcn[blk, :, t % 16])
            ids.append(nxt)
            nxt += 1
        new_lens.append(len(ids))
        new_table.append(ids + [0] * (width - len(ids)))
    # pages of one token each: [tokens, Hkv, 1, D]
    ref = oracle.decode_attention_ref(a["q"], np.stack(rows_k)[:, :, None], np.stack(rows_v)[:, :, None],
                                      np.array(new_table), 1,
                                      np.array(new_lens), *sc.cpu().numpy())
    assert_within_tolerance(out.reshape(3, -1), ref.reshape(3, -1), what="masked tokens")


def test_end_to_end_recalibrate_write_attend(fp8blk_lib):
    """A qkv projection output for the cached tokens: maxima -> scales ->
    cache write -> attention of each sequence's last token, all on the
    device; the oracle reads the caches the device wrote."""
    hq, hkv = 32, 8
    lens = [100, 37, 256, 1]
    qkv, _ = synth.kv_inputs("llama8b_decode", t=sum(lens))
    dq = qkv.to(DEV)
    scales = fb.kv_scales(fb.qkv_amax(dq, hq, hkv, D))
    a = synth.attention_inputs(lens, hq, hkv, D, 16, seed=8)
    kc = torch.zeros(a["num_slots"] // 16, hkv, 16, D, dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    fb.kv_cache_write(dq[:, hq * D:(hq + hkv) * D], dq[:, (hq + hkv) * D:], a["slot"].to(DEV), scales[1:2],
                      scales[2:3], kc, vc)
    b = len(lens)
    q_rows = dq[-b:, :hq * D]                          # read in place: row stride (Hq + 2 Hkv) D
    assert q_rows.stride(0) == (hq + 2 * hkv) * D
    out = torch.empty(b, hq, D, dtype=torch.bfloat16, device=DEV)
    fb.decode_attention(q_rows, kc, vc, a["block_table"].to(DEV), 16, a["context_lens"].to(DEV), scales[0:1],
                        scales[1:2], scales[2:3], out=out)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()
    ref = oracle.decode_attention_ref(qkv[-b:, :hq * D].reshape(b, hq, D), kc.cpu().numpy(), vc.cpu().numpy(),
                                      a["block_table"].numpy(), 16, np.array(lens), s[0], s[1], s[2])
    assert_within_tolerance(out.float().cpu().numpy().reshape(b, -1), ref.reshape(b, -1), what="end to end")


def test_full_size_decode_sampled(fp8blk_lib):
    """The Llama-3.1-8B decode batch (256 sequences, 32/8 heads) at 2048
    cached tokens each, caches of random codes; sampled sequences checked."""
    b, hq, hkv, ctx, bs = 256, 32, 8, 2048, 16
    blocks = ctx // bs
    g = synth.generator(90)
    perm = torch.randperm(b * blocks + 7, generator=g)[: b * blocks].to(torch.int32).reshape(b, blocks)
    kc = synth.random_cache_codes((b * blocks + 7, hkv, bs, D), 1, DEV)
    vc = synth.random_cache_codes((b * blocks + 7, hkv, bs, D), 2, DEV)
    q = torch.randn(b, hq, D, generator=g).to(torch.bfloat16)
    lens = torch.full((b,), ctx, dtype=torch.int32)
    scales = torch.tensor([4.0 / 448, 0.004, 0.01], dtype=torch.float32, device=DEV)
    out = fb.decode_attention(q.to(DEV), kc, vc, perm.to(DEV), bs, lens.to(DEV), scales[0:1], scales[1:2],
                              scales[2:3])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255], torch.randint(0, b, (4,), generator=g).numpy()]))
    # the oracle reads only the sampled sequences' pages, gathered into a
    # small cache with the block table renumbered (page order is immaterial)
    pages = perm[torch.from_numpy(rows)].reshape(-1).long().to(DEV)
    small_k = kc[pages].cpu().numpy()
    small_v = vc[pages].cpu().numpy()
    table = np.arange(len(rows) * blocks).reshape(len(rows), blocks)
    ref = oracle.decode_attention_ref(q[torch.from_numpy(rows)], small_k, small_v, table, bs, lens.numpy()[rows],
                                      *scales.cpu().numpy())
    got = out[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    assert_within_tolerance(got.reshape(len(rows), -1), ref.reshape(len(rows), -1), what="full-size decode")
