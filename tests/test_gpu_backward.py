"""GPU parity of the backward GEMMs (dgrad, wgrad) and their pieces -- the
transposed quantizers and the GEMM with per-row scales on both operands --
against the oracle, through the C ABI. Codes and scales bit for bit; GEMM
outputs within |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref)."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_quant_amd as fb
import oracle
import synth
from tests.gpu_util import assert_codes_equal, assert_scales_equal, assert_within_tolerance, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16_from_bits(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def check_act_t(x, pow2):
    m, k = x.shape
    qt, cq = guarded((k, m), torch.uint8, DEV)
    st, cs = guarded((k, m // 128), torch.float32, DEV)
    fb.quant_act_t(x.to(DEV), pow2, qt=qt, st=st)
    cq()
    cs()
    q_r, s_r = oracle.quant_act_t_ref(x, pow2)
    assert_codes_equal(qt.cpu().numpy(), q_r, "transposed codes")
    assert_scales_equal(st.cpu().numpy(), s_r, "transposed scales")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,k", [(128, 64), (256, 192), (384, 4096), (1280, 640)])
def test_quant_act_t(fp8blk_lib, m, k, pow2):
    """Columns at magnitudes from 2^-40 to 2^40 and a zero column."""
    g = synth.generator(80, m + k)
    x = synth.activation(m, k, g, 0.005, 30.0).float()
    x *= torch.pow(2.0, torch.randint(-40, 41, (1, k), generator=g).float())
    x[:, k // 2] = 0
    check_act_t(x.to(torch.bfloat16), pow2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_quant_act_t_every_finite_bf16_value(fp8blk_lib, order, pow2):
    """All 65280 finite bf16 values as 510 columns of 128 tokens (plus two
    zero columns): sorted, every group holds neighbouring magnitudes down to
    the subnormals; shuffled, every value under many scales."""
    b = np.arange(1 << 16, dtype=np.uint32)
    bits = b[(b & 0x7F80) != 0x7F80].astype(np.uint16)
    if order == "shuffled":
        bits = bits[torch.randperm(bits.size, generator=synth.generator(81)).numpy()]
    else:
        bits = np.sort(bits)
    cols = np.zeros((512, 128), np.uint16)
    cols[:510] = bits.reshape(510, 128)
    x = _bf16_from_bits(cols.T.copy())            # [128 tokens, 512 columns]
    check_act_t(x, pow2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (384, 256), (1024, 2048)])
def test_quant_weight_t(fp8blk_lib, n, k, pow2):
    g = synth.generator(82, n + k)
    w = synth.weight(n, k, g).float()
    w[:128, :128] *= 1e-30                        # a block far below the others
    w = w.to(torch.bfloat16)
    qt, cq = guarded((k, n), torch.uint8, DEV)
    st, cs = guarded((k // 128, n // 128), torch.float32, DEV)
    fb.quant_weight_t(w.to(DEV), pow2, qt=qt, st=st)
    cq()
    cs()
    q_r, s_r = oracle.quant_weight_t_ref(w, pow2)
    assert_codes_equal(qt.cpu().numpy(), q_r, "transposed weight codes")
    assert_scales_equal(st.cpu().numpy(), s_r, "transposed weight scales")
    q, s = fb.quant_weight(w.to(DEV), pow2)       # the forward layout, transposed, is the same
    assert torch.equal(q.t().contiguous(), qt) and torch.equal(s.t().contiguous(), st)


def rowscaled_check(x, b, pow2=False):
    """x [M, K], b [N, K] bf16, both quantized in 1x128 groups along K."""
    qa, sa = fb.quant_act(x.to(DEV), pow2)
    qb, sb = fb.quant_act(b.to(DEV), pow2)
    y, check = guarded((x.shape[0], b.shape[0]), torch.bfloat16, DEV)
    fb.gemm_rowscaled(qa, sa, qb, sb, y=y)
    check()
    qa_r, sa_r = oracle.quant_act_ref(x, pow2)
    qb_r, sb_r = oracle.quant_act_ref(b, pow2)
    return assert_within_tolerance(y.float().cpu().numpy(), oracle.gemm_rowscaled_ref(qa_r, sa_r, qb_r, sb_r),
                                   what="rowscaled gemm")


@pytest.mark.parametrize("m,k,n", [
    (1, 128, 128), (130, 1152, 256),
    (300, 256, 640),      # 64x64 tiles
    (2048, 256, 4096),    # 128x128 tiles
    (2100, 384, 8320),    # 256x256 tiles, with an M tail and a half-width N tail
])
def test_gemm_rowscaled_tiles(fp8blk_lib, m, k, n):
    g = synth.generator(83, m + k + n)
    rowscaled_check(synth.activation(m, k, g, 0.005, 30.0), synth.activation(n, k, g, 0.005, 30.0))


def test_gemm_rowscaled_scale_extremes(fp8blk_lib):
    """Row scales spread over 2^-60 .. 2^0 on one side and 2^0 .. 2^40 on
    the other (outputs stay inside the bf16 range), zero rows, and one K
    block per operand far from the others."""
    g = synth.generator(84)
    x = synth.activation(300, 512, g).float() * torch.pow(2.0, torch.randint(-60, 1, (300, 1), generator=g).float())
    b = synth.activation(384, 512, g).float() * torch.pow(2.0, torch.randint(0, 41, (384, 1), generator=g).float())
    x[5] = 0
    b[17] = 0
    x[:, 128:256] *= 2.0 ** 20
    b[:, 384:] *= 2.0 ** -20
    rowscaled_check(x.to(torch.bfloat16), b.to(torch.bfloat16))


def test_gemm_rowscaled_deterministic(fp8blk_lib):
    g = synth.generator(85)
    qa, sa = fb.quant_act(synth.activation(1024, 1024, g).to(DEV))
    qb, sb = fb.quant_act(synth.activation(2048, 1024, g).to(DEV))
    y1 = fb.gemm_rowscaled(qa, sa, qb, sb)
    y2 = fb.gemm_rowscaled(qa, sa, qb, sb)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("pow2", [False, True])
def test_dgrad(fp8blk_lib, pow2):
    dy, x, w = synth.backward_inputs("llama8b_decode", "o_proj", m=300)
    w = w[:640, :384].contiguous()
    dy = dy[:, :640].contiguous()
    qwt, swt = fb.quant_weight_t(w.to(DEV), pow2)
    dx = fb.dgrad(dy.to(DEV), qwt, swt, pow2)
    torch.cuda.synchronize()
    assert_within_tolerance(dx.float().cpu().numpy(), oracle.dgrad_ref(dy, w, pow2), what="dgrad")


@pytest.mark.parametrize("pow2", [False, True])
def test_wgrad(fp8blk_lib, pow2):
    dy, x, w = synth.backward_inputs("llama8b_decode", "qkv", m=512)
    dy = dy[:, :384].contiguous()
    x = x[:, :256].contiguous()
    dw = fb.wgrad(dy.to(DEV), x.to(DEV), pow2)
    torch.cuda.synchronize()
    assert_within_tolerance(dw.float().cpu().numpy(), oracle.wgrad_ref(dy, x, pow2), what="wgrad")


def test_wgrad_full_size_sampled(fp8blk_lib):
    """Llama-3.1-8B qkv at the prefill batch: dW [6144, 4096] = dY^T X over
    16384 tokens, checked on sampled output rows and columns."""
    dy, x, _ = synth.backward_inputs("llama8b_prefill", "qkv")
    dw = fb.wgrad(dy.to(DEV), x.to(DEV))
    torch.cuda.synchronize()
    g = synth.generator(86)
    rows = np.unique(np.concatenate([[0, 6143], torch.randint(0, 6144, (14,), generator=g).numpy()]))
    cols = np.unique(np.concatenate([[0, 4095], torch.randint(0, 4096, (14,), generator=g).numpy()]))
    qa, sa = oracle.quant_act_t_ref(dy[:, torch.from_numpy(rows)].contiguous())
    qb, sb = oracle.quant_act_t_ref(x[:, torch.from_numpy(cols)].contiguous())
    y_ref = oracle.gemm_rowscaled_ref(qa, sa, qb, sb)
    got = dw[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
    assert_within_tolerance(got, y_ref, what="sampled wgrad")


def test_dgrad_full_size_sampled(fp8blk_lib):
    """Llama-3.1-8B qkv at the prefill batch: dX [16384, 4096] = dY W,
    checked on sampled rows and whole 128-column blocks."""
    dy, _, w = synth.backward_inputs("llama8b_prefill", "qkv")
    qwt, swt = fb.quant_weight_t(w.to(DEV))
    dx = fb.dgrad(dy.to(DEV), qwt, swt)
    torch.cuda.synchronize()
    g = synth.generator(87)
    rows = np.unique(np.concatenate([[0, 16383], torch.randint(0, 16384, (22,), generator=g).numpy()]))
    blocks = sorted({0, 31} | set(torch.randint(0, 32, (2,), generator=g).tolist()))
    kcols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    qa, sa = oracle.quant_act_ref(dy[torch.from_numpy(rows)])
    qwt_r, swt_r = oracle.quant_weight_t_ref(w)
    y_ref = oracle.gemm_ref(qa, sa, qwt_r[kcols], swt_r[blocks])
    got = dx[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(kcols).to(DEV)].float().cpu().numpy()
    assert_within_tolerance(got, y_ref, what="sampled dgrad")


# ------------------------------------------------------------ expert-grouped backward

MOE_OFFSETS = [0, 100, 100, 356, 357, 557, 813]   # 100, 0, 256, 1, 200, 256 rows


def _moe_case(seed, n, k, offsets=MOE_OFFSETS):
    g = synth.generator(84, seed)
    m = offsets[-1]
    dy = (synth.activation(m, n, g, 0.005, 30.0).float() * 2.0 ** -10).to(torch.bfloat16)
    x = synth.activation(m, k, g, 0.005, 30.0)
    w = synth.weight((len(offsets) - 1) * n, k, g).reshape(len(offsets) - 1, n, k)
    return dy, x, w, torch.tensor(offsets, dtype=torch.int32)


@pytest.mark.parametrize("pow2", [False, True])
def test_quant_weight_t_grouped(fp8blk_lib, pow2):
    _, _, w, _ = _moe_case(1, 256, 384)
    e = w.shape[0]
    qt, cq = guarded((e, 384, 256), torch.uint8, DEV)
    st, cs = guarded((e, 3, 2), torch.float32, DEV)
    fb.quant_weight_t(w.to(DEV), pow2, qt=qt, st=st)
    cq()
    cs()
    for i in range(e):
        q_r, s_r = oracle.quant_weight_t_ref(w[i], pow2)
        assert_codes_equal(qt[i].cpu().numpy(), q_r, "expert %d transposed weight codes" % i)
        assert_scales_equal(st[i].cpu().numpy(), s_r, "expert %d transposed weight scales" % i)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("k", [64, 192])
def test_quant_act_t_grouped(fp8blk_lib, k, pow2):
    """Ragged experts (an empty one, a one-row one): codes and scales of
    every expert group bit for bit, padding columns 0, and nothing written
    past the padded axis' used part."""
    _, x, _, off = _moe_case(2, 128, k)
    m, e = x.shape[0], off.shape[0] - 1
    ld = fb.padded_tokens(m, e)
    qt, cq = guarded((k, ld), torch.uint8, DEV)
    st, cs = guarded((k, ld // 128), torch.float32, DEV)
    qt.fill_(0xA5)
    st.fill_(-1.0)
    fb.quant_act_t_grouped(x.to(DEV), off.to(DEV), pow2, qt=qt, st=st)
    cq()
    cs()
    q_r, s_r = oracle.quant_act_t_grouped_ref(x, off.numpy(), pow2)
    used = q_r.shape[1]
    assert_codes_equal(qt[:, :used].cpu().numpy(), q_r, "grouped transposed codes")
    assert_scales_equal(st[:, :used // 128].cpu().numpy(), s_r, "grouped transposed scales")
    assert bool(torch.all(qt[:, used:] == 0xA5)) and bool(torch.all(st[:, used // 128:] == -1.0))


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_dgrad(fp8blk_lib, pow2):
    dy, _, w, off = _moe_case(3, 256, 384)
    qwt, swt = fb.quant_weight_t(w.to(DEV), pow2)
    dx = fb.grouped_dgrad(dy.to(DEV), qwt, swt, off.to(DEV), pow2)
    torch.cuda.synchronize()
    ref = oracle.grouped_dgrad_ref(dy, w, off.numpy(), pow2)
    assert_within_tolerance(dx.float().cpu().numpy(), ref, what="grouped dgrad")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("n,k", [(256, 384), (128, 640)])
def test_grouped_wgrad(fp8blk_lib, n, k, pow2):
    """Every expert's dW within tolerance (rms per expert); the empty
    expert's dW is exactly zero."""
    dy, x, _, off = _moe_case(4 + n, n, k)
    dw = fb.grouped_wgrad(dy.to(DEV), x.to(DEV), off.to(DEV), pow2)
    torch.cuda.synchronize()
    ref = oracle.grouped_wgrad_ref(dy, x, off.numpy(), pow2)
    got = dw.float().cpu().numpy()
    for i in range(ref.shape[0]):
        if MOE_OFFSETS[i + 1] == MOE_OFFSETS[i]:
            assert np.all(got[i] == 0)
        else:
            assert_within_tolerance(got[i], ref[i], what="grouped wgrad expert %d" % i)


def test_grouped_backward_full_size_sampled(fp8blk_lib):
    """Qwen3-30B-A3B gate_up (4096 tokens, top-8 of 128 experts, hidden 2048,
    2 x 768 outputs): grouped dgrad on sampled rows and grouped wgrad on a
    128 x 128 corner of sampled experts (largest, median, smallest). The
    128x1 groups run along tokens within one column, so a column subset of
    dY and X gives exactly that subset of dW."""
    x, w, off = synth.moe_inputs(0, "gate_up")
    m, (e, n, k) = x.shape[0], w.shape
    g = synth.generator(85)
    dy = (synth.activation(m, n, g, 0.005, 30.0).float() * 2.0 ** -10).to(torch.bfloat16)
    offs = off.numpy().astype(np.int64)
    od = off.to(DEV)
    qwt, swt = fb.quant_weight_t(w.to(DEV))
    dx = fb.grouped_dgrad(dy.to(DEV), qwt, swt, od)
    dw = fb.grouped_wgrad(dy.to(DEV), x.to(DEV), od)
    torch.cuda.synchronize()
    sizes = np.diff(offs)
    picks = sorted({int(np.argmax(sizes)), int(np.argsort(sizes)[len(sizes) // 2]), int(np.argmin(sizes))})
    for ex in picks:
        lo, hi = int(offs[ex]), int(offs[ex + 1])
        rows = np.unique(np.array([lo, hi - 1, (lo + hi) // 2]))
        ref = oracle.dgrad_ref(dy[torch.from_numpy(rows)], w[ex])
        assert_within_tolerance(dx[torch.from_numpy(rows).to(DEV)].float().cpu().numpy(), ref,
                                what="full-size grouped dgrad, expert %d" % ex)
        cols_n, cols_k = slice(1408, 1536), slice(0, 128)
        ref = oracle.grouped_wgrad_ref(dy[lo:hi, cols_n], x[lo:hi, cols_k], [0, hi - lo])[0]
        assert_within_tolerance(dw[ex, cols_n, cols_k].float().cpu().numpy(), ref,
                                what="full-size grouped wgrad, expert %d (%d tokens)" % (ex, hi - lo))
