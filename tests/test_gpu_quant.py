"""GPU parity of the quantisation kernels: bit-exact E4M3 codes and fp32
scales against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (
    assert_codes_equal, assert_scales_equal, check_linear_sampled, guarded, oracle_quant_whole, quant_act_guarded,
)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16_from_bits(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def _all_finite_bf16_bits():
    b = np.arange(1 << 16, dtype=np.uint32)
    exp_all_ones = (b & 0x7F80) == 0x7F80
    return b[~exp_all_ones].astype(np.uint16)       # 65280 finite patterns


def _check_act(x, pow2):
    q, s = quant_act_guarded(x.to(DEV), pow2)
    q_r, s_r = oracle.quant_act_ref(x, pow2)
    assert_codes_equal(q.cpu().numpy(), q_r)
    assert_scales_equal(s.cpu().numpy(), s_r)


def _check_weight(w, pow2):
    import block_scaled_fp8_quant_amd as fb
    n, k = w.shape
    q, cq = guarded((n, k), torch.uint8, DEV)
    s, cs = guarded((n // 128, k // 128), torch.float32, DEV)
    fb.quant_weight(w.to(DEV), pow2, q=q, s=s)
    cq()
    cs()
    q_r, s_r = oracle.quant_weight_ref(w, pow2)
    assert_codes_equal(q.cpu().numpy(), q_r, "weight codes")
    assert_scales_equal(s.cpu().numpy(), s_r, "weight scales")


@pytest.mark.parametrize("pow2", [False, True])
def test_tiny_workload(fp8blk_lib, pow2):
    x, w = synth.linear_inputs("tiny", 0)
    _check_act(x, pow2)
    _check_weight(w, pow2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("order", ["shuffled", "sorted"])
def test_every_finite_bf16_value(fp8blk_lib, pow2, order):
    """All 65280 finite bf16 values, either shuffled (every element under
    many different scales) or sorted (groups of similar magnitude: fp32
    subnormal scales, huge scales, all-subnormal groups)."""
    bits = _all_finite_bf16_bits()
    if order == "shuffled":
        bits = bits[torch.randperm(bits.size, generator=synth.generator(3)).numpy()]
    else:
        bits = np.sort(bits)
    x = _bf16_from_bits(bits).reshape(-1, 256)
    _check_act(x, pow2)
    _check_weight(x[: (x.shape[0] // 128) * 128], pow2)


def _tie_rows():
    """Groups with amax = 448 (s = 1 exactly) holding every E4M3 midpoint
    and its bf16 neighbours, so the hardware conversion's tie rule shows."""
    t = oracle.decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    vals = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), t])
    vals = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).float().numpy()
    vals = vals[np.abs(vals) <= 448]
    pad = (-len(vals)) % 127
    vals = np.concatenate([vals, np.zeros(pad)])
    groups = vals.reshape(-1, 127)
    groups = np.concatenate([np.full((groups.shape[0], 1), 448.0), groups], axis=1)
    sign = np.where(np.arange(groups.size).reshape(groups.shape) % 3 == 0, -1.0, 1.0)
    return torch.tensor(groups * sign, dtype=torch.float32).to(torch.bfloat16)


def _divide_vs_reciprocal_rows():
    from tests.test_oracle_quant import divide_vs_reciprocal_pairs
    x, amax = divide_vs_reciprocal_pairs(256, seed=11)
    g = np.zeros((len(x), 128))
    g[:, 0] = amax
    g[:, 1] = x
    g[:, 2] = -x
    return torch.tensor(g, dtype=torch.float32).to(torch.bfloat16)


def _special_rows():
    rows = []
    z = np.zeros(128)
    rows.append(z)                                   # all +0
    rows.append(-z - 0.0)                            # all -0
    r = np.zeros(128); r[::2] = -0.0; rows.append(r)
    for e in (-133, -130, -126, -120, -100, -91, -90, -89, 0, 60, 120, 127):
        r = np.linspace(-1, 1, 128) * 2.0 ** e
        r[5] = 2.0 ** e
        rows.append(r)
    r = np.full(128, 3.3895313892515355e38); r[1::2] *= -1; rows.append(r)   # max bf16
    r = np.zeros(128); r[7] = -(2.0 ** -133); rows.append(r)                # lone min subnormal
    x = np.stack(rows)
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _scale_rounded_down_rows():
    """Groups whose fp32 scale amax/448 rounds down, so the largest
    elements' quotients land just above 448 (they must still encode to
    +-448): every such bf16 amax with exponent in [-80, 100), 512 of them
    evenly spaced, each with -amax and its lower bf16 neighbour."""
    b = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    amax = (b << 16).view(np.float32).astype(np.float64)
    s32 = (amax / 448.0).astype(np.float32).astype(np.float64)
    pick = amax[(s32 * 448.0 < amax) & (amax >= 2.0 ** -80) & (amax < 2.0 ** 100)]
    pick = pick[np.linspace(0, len(pick) - 1, 512).astype(np.int64)]
    g = np.zeros((len(pick), 128))
    g[:, 0] = pick
    g[:, 1] = -pick
    g[:, 2] = pick * (1 - 2.0 ** -8)
    return torch.tensor(g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("pow2", [False, True])
def test_adversarial_groups(fp8blk_lib, pow2):
    x = torch.cat([_tie_rows(), _divide_vs_reciprocal_rows(), _special_rows(), _scale_rounded_down_rows()])
    x = x.reshape(-1, 128)
    pad = (-x.shape[0]) % 4
    x = torch.cat([x, torch.zeros(pad, 128, dtype=torch.bfloat16)]).reshape(-1, 512)
    _check_act(x, pow2)
    w = x.reshape(-1, 128)
    w = w[: (w.shape[0] // 128) * 128]
    _check_weight(w, pow2)


@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (5, 128), (17, 256), (33, 1152), (64, 4096)])
def test_ragged_shapes(fp8blk_lib, m, k):
    g = synth.generator(4, seed=m * 7 + k)
    x = synth.activation(m, k, g, 0.01, 50.0)
    _check_act(x, False)
    _check_act(x, True)


def test_empty_is_noop(fp8blk_lib):
    import block_scaled_fp8_quant_amd as fb
    q, s = fb.quant_act(torch.zeros(0, 256, dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_deterministic(fp8blk_lib):
    import block_scaled_fp8_quant_amd as fb
    x, w = synth.linear_inputs("llama8b_decode", "down")
    xd = x.to(DEV)
    runs = [fb.quant_act(xd) for _ in range(3)]
    for q, s in runs[1:]:
        assert torch.equal(q, runs[0][0]) and torch.equal(s, runs[0][1])


def test_expert_stack_as_one_matrix(fp8blk_lib):
    import block_scaled_fp8_quant_amd as fb
    w = synth.weight(4 * 256, 384, synth.generator(5)).reshape(4, 256, 384)
    q, s = fb.quant_weight(w.to(DEV))
    q_r, s_r = oracle.quant_weight_ref(w.reshape(-1, 384))
    assert_codes_equal(q.reshape(-1, 384).cpu().numpy(), q_r)
    assert_scales_equal(s.reshape(-1, 3).cpu().numpy(), s_r)


@pytest.mark.parametrize("workload", ["llama8b_prefill", "llama8b_decode", "qwen8b_pow2"])
def test_full_size_sampled(fp8blk_lib, workload):
    """Every linear of the workload at full size; sampled rows and weight
    blocks bit-exact, sampled outputs within tolerance."""
    wl = synth.WORKLOADS[workload]
    gen = synth.generator(6)
    for li, (name, k, n) in enumerate(wl.linears):
        print("full-size %s %s M=%d K=%d N=%d" % (workload, name, wl.m, k, n), flush=True)
        x, w = synth.linear_inputs(workload, li)
        check_linear_sampled(x, w, wl.pow2, DEV, gen)
        del x, w
        torch.cuda.empty_cache()


@pytest.mark.parametrize("workload", ["llama8b_prefill", "qwen8b_pow2"])
def test_full_size_whole_tensors(fp8blk_lib, workload):
    """Every linear of the workload at full size, every activation and weight
    code and scale compared with the oracle bit for bit (not sampled)."""
    import block_scaled_fp8_quant_amd as fb
    wl = synth.WORKLOADS[workload]
    for li, (name, k, n) in enumerate(wl.linears):
        print("whole-tensor %s %s M=%d K=%d N=%d" % (workload, name, wl.m, k, n), flush=True)
        x, w = synth.linear_inputs(workload, li)
        qa, sa = fb.quant_act(x.to(DEV), wl.pow2)
        qw, sw = fb.quant_weight(w.to(DEV), wl.pow2)
        torch.cuda.synchronize()
        qa_r, sa_r = oracle_quant_whole(x, wl.pow2)
        assert_codes_equal(qa.cpu().numpy(), qa_r, "%s activation codes" % name)
        assert_scales_equal(sa.cpu().numpy(), sa_r, "%s activation scales" % name)
        del qa_r, sa_r
        qw_r, sw_r = oracle_quant_whole(w, wl.pow2, weight=True)
        assert_codes_equal(qw.cpu().numpy(), qw_r, "%s weight codes" % name)
        assert_scales_equal(sw.cpu().numpy(), sw_r, "%s weight scales" % name)
        del x, w, qa, sa, qw, sw, qw_r, sw_r
        torch.cuda.empty_cache()
