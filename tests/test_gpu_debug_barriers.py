"""Race detection on the GPU: the kernels that stage operands through LDS
(every GEMM tile configuration, the split-K, grouped and row-scaled GEMMs,
the prefill and decode attention) built with an extra barrier at every LDS stage
transition (libfp8blk_debug_barriers.so, -DFP8BLK_DEBUG_BARRIERS=1) must give
the normal build's outputs bit for bit: the arithmetic is identical, so any
difference would come from a stage read while being refilled or refilled
while still read."""

import ctypes
import os

import pytest
import torch

import block_scaled_fp8_quant_amd as fb
from block_scaled_fp8_quant_amd import build as fbuild
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dbg(fp8blk_lib):
    if not os.path.exists(fbuild.DEBUG_LIB):
        raise RuntimeError("the race-detection build is missing: run __graft_entry__.build()")
    return fb.declare(ctypes.CDLL(fbuild.DEBUG_LIB))


def stream():
    return torch.cuda.current_stream().cuda_stream


def same(a, b, what):
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what + ": debug-barrier build differs"


def operands(m, n, k, seed, pow2=False):
    g = synth.generator(0x63, seed)
    qa, sa = fb.quant_act(synth.activation(m, k, g, 0.005, 30.0).to(DEV), pow2)
    qw, sw = fb.quant_weight(synth.weight(n, k, g).to(DEV), pow2)
    return qa, sa, qw, sw


# (M, N, K): the 256x256, 128x128, 64x64 and 256x128 tiles, the pow2
# in-MFMA path of the 256x256 tile, partial tiles on every edge, and the
# persistent walk of 256x256 tiles (at least three per CU, K <= 64 blocks)
# in both scale paths, with a partial row and column tile
GEMMS = [(4096, 4096, 1024, False), (4096, 2048, 1024, False), (300, 512, 1024, False),
         (256, 28672, 1024, False), (4096, 4096, 1024, True), (4000, 3968, 640, False),
         (6144, 8192, 512, False), (6144, 8192, 512, True), (6000, 8320, 384, False)]


@pytest.mark.parametrize("m,n,k,pow2", GEMMS)
def test_gemm_tiles(dbg, m, n, k, pow2):
    qa, sa, qw, sw = operands(m, n, k, m + n + k, pow2)
    y0 = fb.gemm(qa, sa, qw, sw, split=False)
    y1 = torch.empty_like(y0)
    assert dbg.fp8blk_gemm(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k, y1.data_ptr(),
                           stream()) == 0
    same(y0, y1, "gemm %dx%dx%d" % (m, n, k))


def test_split_k(dbg):
    m, n, k = 256, 4096, 8192
    qa, sa, qw, sw = operands(m, n, k, 7)
    need = fb.fp8blk_gemm_workspace_size(m, n, k)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y0 = fb.gemm(qa, sa, qw, sw, workspace=ws)
    y1 = torch.empty_like(y0)
    assert dbg.fp8blk_gemm_ws(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k, y1.data_ptr(),
                              ws.data_ptr(), need, stream()) == 0
    same(y0, y1, "split-K gemm")


# the last two run the persistent kernel (more tiles than the CUs hold at
# once): 128x128 tiles at K = 512, 256x256 tiles at K = 2048
@pytest.mark.parametrize("tokens,experts,topk,hidden,n", [(64, 8, 2, 256, 512), (600, 4, 2, 2048, 512),
                                                          (300, 16, 4, 512, 256), (2048, 16, 2, 512, 2048),
                                                          (2048, 8, 2, 2048, 4096)])
def test_grouped(dbg, tokens, experts, topk, hidden, n):
    x, w, off = synth.small_moe_inputs(1, tokens=tokens, hidden=hidden, experts=experts, topk=topk, n=n)
    qa, sa = fb.quant_act(x.to(DEV))
    qw, sw = fb.quant_weight(w.to(DEV))
    offd = off.to(DEV)
    y0 = fb.grouped_gemm(qa, sa, qw, sw, offd)
    y1 = torch.empty_like(y0)
    m, k = qa.shape
    assert dbg.fp8blk_grouped_gemm(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), offd.data_ptr(),
                                   experts, m, n, k, y1.data_ptr(), stream()) == 0
    same(y0, y1, "grouped gemm")


@pytest.mark.parametrize("m,n,k", [(4096, 4096, 512), (2048, 4096, 512), (512, 384, 640)])
def test_rowscaled(dbg, m, n, k):
    g = synth.generator(0x64, m + n)
    qa, sa = fb.quant_act_t(synth.activation(k, m, g).to(DEV))   # [m, k] with per-row scales
    qb, sb = fb.quant_act_t(synth.activation(k, n, g).to(DEV))
    y0 = fb.gemm_rowscaled(qa, sa, qb, sb)
    y1 = torch.empty_like(y0)
    assert dbg.fp8blk_gemm_rowscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), m, n, k,
                                     y1.data_ptr(), stream()) == 0
    same(y0, y1, "row-scaled gemm")


def test_grouped_rowscaled(dbg):
    x, w, off = synth.small_moe_inputs(2, tokens=300, hidden=512, experts=8, topk=2, n=256)
    g = synth.generator(0x65)
    dy = synth.activation(x.shape[0], 256, g).to(DEV)
    offd = off.to(DEV)
    qa, sa = fb.quant_act_t_grouped(dy, offd)
    qb, sb = fb.quant_act_t_grouped(x.to(DEV), offd)
    y0 = fb.grouped_gemm_rowscaled(qa, sa, qb, sb, offd)
    y1 = torch.empty_like(y0)
    e, nn, kk = y0.shape
    assert dbg.fp8blk_grouped_gemm_rowscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                             offd.data_ptr(), e, qa.shape[1], nn, kk, y1.data_ptr(), stream()) == 0
    same(y0, y1, "grouped row-scaled gemm")


def test_prefill_attention(dbg):
    a = synth.prefill_inputs([(150, 300), (64, 64), (1, 90)], 32, 8, seed=9)
    nslots = a["num_slots"]
    kc = synth.random_cache_codes((nslots // 16, 8, 16, 128), 31, DEV)
    vc = synth.random_cache_codes((nslots // 16, 8, 16, 128), 32, DEV)
    sc = torch.tensor([4.0 / 448, 0.004, 0.01], dtype=torch.float32, device=DEV)
    q, cu = a["q"].to(DEV), a["cu_seqlens_q"].to(DEV)
    table, lens = a["block_table"].to(DEV), a["context_lens"].to(DEV)
    o0 = fb.prefill_attention(q, cu, a["max_seqlen_q"], kc, vc, table, 16, lens, sc[0:1], sc[1:2], sc[2:3])
    o1 = torch.empty_like(o0)
    tq = q.shape[0]
    assert dbg.fp8blk_prefill_attention(q.data_ptr(), 32 * 128, tq, 3, 32, 8, 128, cu.data_ptr(), a["max_seqlen_q"],
                                        kc.data_ptr(), vc.data_ptr(), nslots, table.data_ptr(), table.shape[1], 16,
                                        lens.data_ptr(), sc[0:1].data_ptr(), sc[1:2].data_ptr(), sc[2:3].data_ptr(),
                                        128 ** -0.5, o1.data_ptr(), 32 * 128, stream()) == 0
    same(o0, o1, "prefill attention")


@pytest.mark.parametrize("split", [0, 256])
def test_decode_attention(dbg, split):
    a = synth.attention_inputs([700, 33, 2048, 1], 32, 8, 128, 16, 11)
    nslots = a["num_slots"]
    kc = synth.random_cache_codes((nslots // 16, 8, 16, 128), 33, DEV)
    vc = synth.random_cache_codes((nslots // 16, 8, 16, 128), 34, DEV)
    sc = torch.tensor([4.0 / 448, 0.004, 0.01], dtype=torch.float32, device=DEV)
    q, table, lens = a["q"].to(DEV), a["block_table"].to(DEV), a["context_lens"].to(DEV)
    b = q.shape[0]
    need = fb.fp8blk_decode_attention_workspace_size(b, 32, 8, 128, table.shape[1], 16, split) if split else 0
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    outs = []
    for lib in (fb.load(), dbg):
        o = torch.empty(b, 32, 128, dtype=torch.bfloat16, device=DEV)
        assert lib.fp8blk_decode_attention(q.data_ptr(), 32 * 128, b, 32, 8, 128, kc.data_ptr(), vc.data_ptr(), nslots,
                                           table.data_ptr(), table.shape[1], 16, lens.data_ptr(), sc[0:1].data_ptr(),
                                           sc[1:2].data_ptr(), sc[2:3].data_ptr(), 128 ** -0.5, o.data_ptr(), 32 * 128,
                                           split, ws.data_ptr() if need else None, need, stream()) == 0
        outs.append(o)
    same(outs[0], outs[1], "decode attention split=%d" % split)
