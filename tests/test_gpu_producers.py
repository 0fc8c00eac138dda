"""GPU parity of the fused producers (RMSNorm -> 1x128 quantisation and
SiLU(gate) * up -> 1x128 quantisation), through the C ABI.

Two checks per call:
  * the bf16 values the kernel produced (written to y) against the exact
    fp64 producer of the oracle: equal to its bf16 rounding, except where
    the exact value lies so close to a bf16 rounding midpoint that the
    kernel's fp32 arithmetic may fall on the other side (then the other
    neighbour is accepted);
  * codes and scales bit for bit against the oracle's quantiser applied to
    those same bf16 values (the decision is taken on the same bf16 inputs
    on both sides), and bit for bit equal to a call without y.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_codes_equal, assert_scales_equal, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# fp32 producer error bound used for the midpoint window, relative to |y|:
# RMSNorm's sum of K squares in fp32 (K/64 sequential fmas per lane plus a
# 64-lane tree), halved by the square root, plus five roundings, stays below
# 2^-17 for K <= 16384; SiLU * up: exp (a few ulp), one add, one division,
# two products. 2^-14 leaves a wide margin while still being 64x finer than
# a bf16 ulp.
MID_WINDOW = 2.0 ** -14
# No allowance for flushing: the kernels keep IEEE fp32 subnormals (no
# flush-to-zero build option), so subnormal results, e.g. SiLU of a large
# negative gate, are compared like any other value.


def bits_of(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_bf16_matches_exact(y_gpu, y_ref, what):
    """y_gpu (bf16 tensor) against the exact values y_ref (float64)."""
    g = oracle.bf16_values(y_gpu.cpu())
    bits_r, r = oracle.round_bf16(y_ref)
    bits_g = bits_of(y_gpu)
    diff = g != r
    neighbours = np.abs(bits_g.astype(np.int64) - bits_r.astype(np.int64)) == 1
    near_mid = np.abs(y_ref - (g + r) / 2) <= MID_WINDOW * np.abs(y_ref)
    bad = diff & ~(neighbours & near_mid)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d values off the exact producer's bf16 rounding; first at %s: "
                             "gpu %r exact %r (rounds to %r)" % (what, bad.sum(), i, g[i], y_ref[i], r[i]))
    assert diff.mean() < 0.01, "%s: %.4f of the values on the far side of a midpoint" % (what, diff.mean())


def run_rmsnorm(x, gamma, eps, pow2, with_y=True):
    import block_scaled_fp8_quant_amd as fb
    m, k = x.shape
    q, cq = guarded((m, k), torch.uint8, DEV)
    s, cs = guarded((m, k // 128), torch.float32, DEV)
    y, cy = guarded((m, k), torch.bfloat16, DEV) if with_y else (None, lambda: None)
    fb.rmsnorm_quant_act(x.to(DEV), gamma.to(DEV), eps, pow2, q=q, s=s, y=y)
    cq(); cs(); cy()
    return q, s, y


def run_silu(gu, pow2, with_y=True):
    import block_scaled_fp8_quant_amd as fb
    m, f = gu.shape[0], gu.shape[1] // 2
    q, cq = guarded((m, f), torch.uint8, DEV)
    s, cs = guarded((m, f // 128), torch.float32, DEV)
    y, cy = guarded((m, f), torch.bfloat16, DEV) if with_y else (None, lambda: None)
    fb.silu_mul_quant_act(gu.to(DEV), pow2, q=q, s=s, y=y)
    cq(); cs(); cy()
    return q, s, y


def check_quant_of_own_values(q, s, y, pow2, what):
    q_r, s_r = oracle.quant_act_ref(y.cpu(), pow2)
    assert_codes_equal(q.cpu().numpy(), q_r, what + " codes")
    assert_scales_equal(s.cpu().numpy(), s_r, what + " scales")


def check_rmsnorm(x, gamma, eps, pow2, what="rmsnorm"):
    q, s, y = run_rmsnorm(x, gamma, eps, pow2)
    assert_bf16_matches_exact(y, oracle.rmsnorm_ref(x, gamma, eps), what + " values")
    check_quant_of_own_values(q, s, y, pow2, what)
    q2, s2, _ = run_rmsnorm(x, gamma, eps, pow2, with_y=False)
    assert torch.equal(q2, q) and torch.equal(s2.view(torch.int32), s.view(torch.int32)), \
        what + ": codes/scales differ when y is not written"
    return q, s, y


def check_silu(gu, pow2, what="silu_mul"):
    q, s, y = run_silu(gu, pow2)
    assert_bf16_matches_exact(y, oracle.silu_mul_ref(gu), what + " values")
    check_quant_of_own_values(q, s, y, pow2, what)
    q2, s2, _ = run_silu(gu, pow2, with_y=False)
    assert torch.equal(q2, q) and torch.equal(s2.view(torch.int32), s.view(torch.int32)), \
        what + ": codes/scales differ when y is not written"
    return q, s, y


# ------------------------------------------------------------------ RMSNorm

# Shapes over every kernel variant (16-byte units per row U = K/8):
# U <= 128: one wave per row (K = 128, 384, 1024); U <= 256: two waves per
# row (1152, 2048); U <= 512: four waves, two units per lane (2176, 4096);
# U <= 1024: four waves, four units per lane (4224, 8192); longer rows: the
# one-wave kernel that reads the row twice (8832, 16384). The row counts
# leave ragged last workgroups (a workgroup takes 16, 8 or 4 rows) and
# lanes past the row end.
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,k", [(1, 128), (37, 128), (5, 384), (37, 1024), (19, 1152), (11, 2048), (9, 2176),
                                 (13, 4096), (6, 4224), (6, 8192), (3, 8832), (2, 16384)])
def test_rmsnorm_shapes(fp8blk_lib, m, k, pow2):
    x, gamma = synth.rmsnorm_inputs(m, k, synth.generator(40, k + m))
    print("rmsnorm m=%d k=%d pow2=%d" % (m, k, pow2), flush=True)
    check_rmsnorm(x, gamma, 1e-5, pow2)


def test_rmsnorm_eps_and_special_rows(fp8blk_lib):
    """A zero row (y = 0, s = 0), a row where eps dominates the mean square
    (eps enters under the root, after the mean), rows 2^-10 and 2^+20 times
    another (with eps = 0 the output is the same bit for bit), a one-hot row
    and a constant row."""
    k = 1024
    gen = synth.generator(41)
    x, gamma = synth.rmsnorm_inputs(8, k, gen)
    xv = x.float()
    xv[0] = 0
    xv[1] = xv[1] * 2.0 ** -6                       # mean square ~2^-12, eps = 0.25 dominates
    xv[3] = xv[2] * 2.0 ** -10
    xv[4] = xv[2] * 2.0 ** 20
    xv[5] = 0
    xv[5, 700] = 3.5
    xv[6] = -2.0
    x = xv.to(torch.bfloat16)
    q, s, y = check_rmsnorm(x, gamma, 0.25, False, "rmsnorm eps=0.25")
    assert torch.all(y[0].float() == 0) and torch.all(s[0] == 0) and torch.all(q[0] == 0)
    # eps = 0 with no zero row: power-of-two scaled rows give identical outputs
    x0 = x.clone()
    x0[0] = x0[7]
    q, s, y = check_rmsnorm(x0, gamma, 0.0, False, "rmsnorm eps=0")
    assert torch.equal(y[2].view(torch.int16), y[3].view(torch.int16))
    assert torch.equal(y[2].view(torch.int16), y[4].view(torch.int16))
    assert torch.equal(q[2], q[3]) and torch.equal(q[2], q[4])


def test_rmsnorm_empty(fp8blk_lib):
    import block_scaled_fp8_quant_amd as fb
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s, y = fb.rmsnorm_quant_act(x, torch.ones(256, dtype=torch.bfloat16, device=DEV), 1e-6, want_y=True)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and s.shape == (0, 2) and y.shape == (0, 256)


@pytest.mark.parametrize("workload", ["llama8b_prefill", "qwen8b_pow2"])
def test_rmsnorm_full_size_sampled(fp8blk_lib, workload):
    """The full-size producer input of the workload (its M and hidden size),
    the oracle on sampled rows (RMSNorm is row-local)."""
    x, gamma = synth.producer_inputs(workload, "rmsnorm")
    pow2 = synth.WORKLOADS[workload].pow2
    import block_scaled_fp8_quant_amd as fb
    q, s, y = fb.rmsnorm_quant_act(x.to(DEV), gamma.to(DEV), 1e-5, pow2, want_y=True)
    torch.cuda.synchronize()
    m = x.shape[0]
    rows = np.unique(np.concatenate([[0, 1, 2, 3, m - 1, m - 4, m // 2],
                                     torch.randint(0, m, (40,), generator=synth.generator(42)).numpy()]))
    r = torch.from_numpy(rows)
    rd = r.to(DEV)
    assert_bf16_matches_exact(y[rd], oracle.rmsnorm_ref(x[r], gamma, 1e-5), "sampled rmsnorm values")
    check_quant_of_own_values(q[rd], s[rd], y[rd], pow2, "sampled rmsnorm")


# ------------------------------------------------------------------ SiLU * up

@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,f", [(1, 128), (3, 384), (17, 1024), (33, 14336)])
def test_silu_mul_shapes(fp8blk_lib, m, f, pow2):
    gu = synth.gate_up_output(m, f, synth.generator(43, f + m))
    print("silu_mul m=%d f=%d pow2=%d" % (m, f, pow2), flush=True)
    check_silu(gu, pow2)


def test_silu_mul_special_values(fp8blk_lib):
    """Gate values across the whole sigmoid: zero (h = 0), large positive
    (h = g * u), large negative (h -> 0 through the bf16 subnormals), a
    zero up half, and every finite bf16 gate value in [-128, 128]."""
    f = 1024
    gen = synth.generator(44)
    g = torch.randn(6, f, generator=gen) * 3
    u = torch.randn(6, f, generator=gen)
    g[0] = 0
    g[1] = torch.linspace(20, 200, f)
    g[2] = torch.linspace(-120, -20, f)
    u[3] = 0
    vals = torch.from_numpy(np.arange(1 << 16, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals) & (vals.abs() <= 128)]
    vals = vals[torch.randperm(vals.numel(), generator=gen)]
    n = (vals.numel() // f) * f
    g_all = torch.cat([g, vals[:n].reshape(-1, f)])
    u_all = torch.cat([u, torch.randn(n // f, f, generator=gen)])
    gu = torch.cat([g_all, u_all], dim=1).to(torch.bfloat16)
    q, s, y = check_silu(gu, False, "silu_mul special")
    check_silu(gu, True, "silu_mul special pow2")
    assert torch.all(y[0].float() == 0) and torch.all(s[0] == 0)
    assert torch.all(y[3].float() == 0) and torch.all(s[3] == 0)


def test_silu_mul_empty(fp8blk_lib):
    import block_scaled_fp8_quant_amd as fb
    gu = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    q, s, y = fb.silu_mul_quant_act(gu)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and s.shape == (0, 2) and y is None


@pytest.mark.parametrize("workload", ["llama8b_prefill", "qwen8b_pow2"])
def test_silu_mul_full_size_sampled(fp8blk_lib, workload):
    """The full-size down-projection input (M x F, F = 14336 or 12288), the
    oracle on sampled rows."""
    gu = synth.producer_inputs(workload, "silu_mul")
    pow2 = synth.WORKLOADS[workload].pow2
    import block_scaled_fp8_quant_amd as fb
    q, s, y = fb.silu_mul_quant_act(gu.to(DEV), pow2, want_y=True)
    torch.cuda.synchronize()
    m = gu.shape[0]
    rows = np.unique(np.concatenate([[0, 1, m - 1, m // 2],
                                     torch.randint(0, m, (24,), generator=synth.generator(45)).numpy()]))
    r = torch.from_numpy(rows)
    rd = r.to(DEV)
    assert_bf16_matches_exact(y[rd], oracle.silu_mul_ref(gu[r]), "sampled silu_mul values")
    check_quant_of_own_values(q[rd], s[rd], y[rd], pow2, "sampled silu_mul")


# ------------------------------------------------------------------ with the GEMM

def test_fused_producer_feeds_gemm(fp8blk_lib):
    """RMSNorm -> quant -> GEMM equals quant_act of the kernel's own bf16
    values -> GEMM, bit for bit (the fused codes are the unfused ones)."""
    import block_scaled_fp8_quant_amd as fb
    x, gamma = synth.rmsnorm_inputs(300, 1024, synth.generator(46))
    w = synth.weight(512, 1024, synth.generator(47))
    qw, sw = fb.quant_weight(w.to(DEV))
    qa, sa, y = fb.rmsnorm_quant_act(x.to(DEV), gamma.to(DEV), 1e-5, want_y=True)
    qa2, sa2 = fb.quant_act(y)
    assert torch.equal(qa, qa2) and torch.equal(sa.view(torch.int32), sa2.view(torch.int32))
    assert torch.equal(fb.gemm(qa, sa, qw, sw).view(torch.int16), fb.gemm(qa2, sa2, qw, sw).view(torch.int16))
