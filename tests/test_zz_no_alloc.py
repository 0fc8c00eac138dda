"""GPU check of the allocation-free split-K GEMM (fp8blk_gemm_noalloc),
called through the C ABI: its output must equal, bit for bit, that of
fp8blk_gemm_ws with a caller workspace (same kernels, same split count)
on two calls in a row, the second with a smaller problem, and a third
call whose shape takes the unsplit path. Guard bytes around every output
must stay intact, and sampled outputs must be within the GEMM tolerance of
the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_within_tolerance, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def operands(m, n, k, seed):
    gen = synth.generator(0x6E, seed)
    x = synth.activation(m, k, gen, 0.005, 30.0)
    w = synth.weight(n, k, gen)
    return x, w


def test_noalloc_matches_workspace_entry_point(fp8blk_lib):
    fb = fp8blk_lib
    stream = torch.cuda.current_stream().cuda_stream
    # decode down projection (32 MiB of partials, the largest split), then a
    # smaller split problem, then a shape the split rule leaves unsplit
    cases = [(256, 4096, 14336), (64, 2048, 8192), (96, 28672, 4096)]
    for i, (m, n, k) in enumerate(cases):
        print("noalloc case %d: M=%d N=%d K=%d" % (i, m, n, k), flush=True)
        need = fb.fp8blk_gemm_workspace_size(m, n, k)
        assert need <= fb.GEMM_SCRATCH_BYTES
        assert (need > 0) == (i < 2)
        x, w = operands(m, n, k, i)
        qa, sa = fb.quant_act(x.to(DEV))
        qw, sw = fb.quant_weight(w.to(DEV))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        y_ws, c_ws = guarded((m, n), torch.bfloat16, DEV)
        y_na, c_na = guarded((m, n), torch.bfloat16, DEV)
        fb.fp8blk_gemm_ws(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k, y_ws.data_ptr(),
                          ws.data_ptr(), ws.numel(), stream)
        fb.fp8blk_gemm_noalloc(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k,
                               y_na.data_ptr(), stream)
        torch.cuda.synchronize()
        c_ws()
        c_na()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), "case %d differs" % i
        # sampled rows and one weight block against the oracle
        rows = np.array(sorted({0, m - 1, m // 2, 17 % m}))
        qa_r, sa_r = oracle.quant_act_ref(x[torch.from_numpy(rows)])
        qw_r, sw_r = oracle.quant_weight_ref(w[:128])
        y_ref = oracle.gemm_ref(qa_r, sa_r, qw_r, sw_r)
        got = y_na[torch.from_numpy(rows).to(DEV)][:, :128].float().cpu().numpy()
        assert_within_tolerance(got, y_ref, what="noalloc gemm case %d" % i)
