"""Helpers for the GPU parity tests: guarded output buffers and sampled
full-size comparisons against the oracle."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import block_scaled_fp8_quant_amd as fb
import oracle
from tests.mfma_window import window_bound

GUARD = 4096          # bytes of canary before and after every output
CANARY = 0xA5


def guarded(shape, dtype, dev):
    """An output tensor of ``shape`` inside a buffer whose GUARD bytes on
    each side hold a canary pattern. Returns (tensor, check) where check()
    asserts the canaries are intact."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=dev)
    t = buf[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def check():
        torch.cuda.synchronize()
        head = buf[:GUARD].cpu().numpy()
        tail = buf[GUARD + nbytes:].cpu().numpy()
        assert np.all(head == CANARY), "write before the output buffer"
        assert np.all(tail == CANARY), "write past the output buffer"
    return t, check


def quant_act_guarded(x_dev, pow2):
    m, k = x_dev.shape
    q, cq = guarded((m, k), torch.uint8, x_dev.device)
    s, cs = guarded((m, k // 128), torch.float32, x_dev.device)
    fb.quant_act(x_dev, pow2, q=q, s=s)
    cq()
    cs()
    return q, s


def assert_codes_equal(q_gpu, q_ref, what="codes"):
    q_gpu = np.asarray(q_gpu)
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, "%s: %d mismatches, first at %s: gpu %#x oracle %#x" % (
        what, len(bad), tuple(bad[0]), q_gpu[tuple(bad[0])], q_ref[tuple(bad[0])])


def assert_scales_equal(s_gpu, s_ref, what="scales"):
    a = np.asarray(s_gpu, np.float32).view(np.uint32)
    b = np.asarray(s_ref, np.float32).view(np.uint32)
    bad = np.argwhere(a != b)
    assert bad.size == 0, "%s: %d mismatches, first at %s: gpu %r oracle %r" % (
        what, len(bad), tuple(bad[0]), a.view(np.float32)[tuple(bad[0])], b.view(np.float32)[tuple(bad[0])])


def assert_within_tolerance(y_gpu, y_ref, rms=None, what="gemm"):
    ok, worst = oracle.tolerance_ok(np.asarray(y_gpu, np.float64), y_ref, rms)
    assert ok, "%s outside |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms: worst ratio %.3g" % (what, worst)
    return worst


def assert_within_tolerance_or_window(y_gpu, y_ref, qa, sa, qw, sw, what="gemm", max_share=1e-5):
    """The tolerance above, except that an element outside it may miss it by
    no more than the FP8 matrix instruction's summation window allows for
    that element (tests/mfma_window.py, computed from the oracle's codes and
    scales), and such elements must be rare (at most ``max_share`` of the
    output). Returns (worst ratio to the tolerance, number of elements that
    needed the window)."""
    y = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    tol = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rms
    err = np.abs(y - y_ref)
    out = np.argwhere(err > tol)
    dec = oracle.decode_table()
    for i, j in out:
        w = window_bound(qa[i], sa[i], qw[j], sw[j // 128], dec)
        assert err[i, j] <= tol[i, j] + w, (
            "%s at (%d, %d): |y - y_ref| = %.4g exceeds the tolerance %.4g plus the summation window %.4g"
            % (what, i, j, err[i, j], tol[i, j], w))
    assert len(out) <= max(1, max_share * y.size), "%s: %d elements outside the tolerance" % (what, len(out))
    with np.errstate(divide="ignore", invalid="ignore"):
        worst = float(np.max(np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0)))) if y.size else 0.0
    return worst, len(out)


def sample_rows(m, count, gen, tile=128):
    """Rows to check at full size: the first and last, both sides of tile
    boundaries, and random ones."""
    fixed = {0, m - 1, min(tile - 1, m - 1), min(tile, m - 1), m // 2}
    rnd = torch.randint(0, m, (count,), generator=gen).tolist()
    return np.array(sorted(fixed | set(rnd)), dtype=np.int64)


def check_linear_sampled(x, w, pow2, dev, gen, rows=24, wblocks=2):
    """Full-size layer on the GPU; the oracle recomputes sampled activation
    rows and whole 128-row weight blocks from the same bf16 inputs and
    compares codes, scales (bit-exact) and the sampled outputs (tolerance)."""
    m, k = x.shape
    n = w.shape[0]
    xd, wd = x.to(dev), w.to(dev)
    qa, sa = fb.quant_act(xd, pow2)
    qw, sw = fb.quant_weight(wd, pow2)
    y = fb.gemm(qa, sa, qw, sw)
    torch.cuda.synchronize()

    r = sample_rows(m, rows, gen)
    qa_r, sa_r = oracle.quant_act_ref(x[torch.from_numpy(r)], pow2)
    assert_codes_equal(qa[torch.from_numpy(r).to(dev)].cpu().numpy(), qa_r, "activation codes")
    assert_scales_equal(sa[torch.from_numpy(r).to(dev)].cpu().numpy(), sa_r, "activation scales")

    nb = n // 128
    blocks = sorted({0, nb - 1} | set(torch.randint(0, nb, (wblocks,), generator=gen).tolist()))
    wrows = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    qw_r, sw_r = oracle.quant_weight_ref(w[torch.from_numpy(wrows)], pow2)
    assert_codes_equal(qw[torch.from_numpy(wrows).to(dev)].cpu().numpy(), qw_r, "weight codes")
    assert_scales_equal(sw[torch.tensor(blocks, device=dev)].cpu().numpy(), sw_r, "weight scales")

    y_ref = oracle.gemm_ref(qa_r, sa_r, qw_r, sw_r)
    y_s = y[torch.from_numpy(r).to(dev)][:, torch.from_numpy(wrows).to(dev)].float().cpu().numpy()
    return assert_within_tolerance(y_s, y_ref, what="sampled gemm")


def oracle_quant_whole(t, pow2, weight=False, rows_per_job=1024):
    """The oracle's quantisation of a whole [rows, K] bf16 tensor, its row
    chunks (whole 128-row blocks for weights) run on a thread pool: numpy
    releases the interpreter lock in the heavy steps, and threads need no
    new process next to the one holding the GPU."""
    f = oracle.quant_weight_ref if weight else oracle.quant_act_ref
    chunks = [t[i:i + rows_per_job] for i in range(0, t.shape[0], rows_per_job)]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda c: f(c, pow2), chunks))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
