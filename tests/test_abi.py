"""The C ABI of libfp8blk.so on the CPU: it loads, exports every function
include/fp8blk.h declares, and rejects bad arguments with the documented
status before making any HIP call (so no GPU is needed)."""

import ctypes
import os
import re

import pytest

import block_scaled_fp8_quant_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")

OK, INVALID, SHAPE, ALIGN = 0, 1, 2, 3
P = 0x10000          # a 16-byte aligned fake device address; never dereferenced
P4 = 0x10004         # 4-byte but not 16-byte aligned
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        pytest.skip("libfp8blk.so not built")
    return fb.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8blk_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fp8blk_quant_act", "fp8blk_quant_weight", "fp8blk_gemm", "fp8blk_gemm_ws", "fp8blk_gemm_workspace_size",
        "fp8blk_gemm_noalloc", "fp8blk_prefill_attention",
        "fp8blk_grouped_gemm",
        "fp8blk_rmsnorm_quant_act", "fp8blk_silu_mul_quant_act", "fp8blk_qkv_amax", "fp8blk_kv_scales",
        "fp8blk_kv_cache_write", "fp8blk_quant_act_t", "fp8blk_quant_weight_t", "fp8blk_gemm_rowscaled",
        "fp8blk_decode_attention", "fp8blk_decode_attention_workspace_size", "fp8blk_quant_weight_t_grouped",
        "fp8blk_quant_act_t_grouped", "fp8blk_grouped_gemm_rowscaled", "fp8blk_status_string"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen("nm -D --defined-only %s" % fb.LIB_PATH).read()
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_status_strings(lib):
    for st in range(6):
        assert lib.fp8blk_status_string(st)
    assert b"unknown" in lib.fp8blk_status_string(99)


def test_quant_act_validation(lib):
    f = lib.fp8blk_quant_act
    assert f(P, -1, 128, P, P, 0, NULL) == INVALID
    assert f(P, 4, 0, P, P, 0, NULL) == INVALID
    assert f(P, 4, 128, P, P, 2, NULL) == INVALID          # pow2 flag
    assert f(P, 4, 100, P, P, 0, NULL) == SHAPE
    assert f(NULL, 4, 128, P, P, 0, NULL) == INVALID
    assert f(P, 4, 128, NULL, P, 0, NULL) == INVALID
    assert f(P, 4, 128, P, NULL, 0, NULL) == INVALID
    assert f(P4, 4, 128, P, P, 0, NULL) == ALIGN
    assert f(P, 4, 128, P4, P, 0, NULL) == ALIGN
    assert f(P, 4, 128, P, P + 2, 0, NULL) == ALIGN
    assert f(NULL, 0, 128, NULL, NULL, 1, NULL) == OK       # M == 0 is a no-op


def test_quant_weight_validation(lib):
    f = lib.fp8blk_quant_weight
    assert f(P, -128, 128, P, P, 0, NULL) == INVALID
    assert f(P, 128, -128, P, P, 0, NULL) == INVALID
    assert f(P, 100, 128, P, P, 0, NULL) == SHAPE
    assert f(P, 128, 200, P, P, 0, NULL) == SHAPE
    assert f(P, 128, 128, P, P, -1, NULL) == INVALID
    assert f(NULL, 128, 128, P, P, 0, NULL) == INVALID
    assert f(P, 128, 128, P4, P, 0, NULL) == ALIGN
    assert f(NULL, 0, 128, NULL, NULL, 0, NULL) == OK


def test_gemm_validation(lib):
    f = lib.fp8blk_gemm
    assert f(P, P, P, P, -1, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 0, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 128, 0, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 130, 128, P, NULL) == SHAPE
    assert f(P, P, P, P, 4, 128, 130, P, NULL) == SHAPE
    assert f(P, P, P, P, 4, 128, (1 << 24) + 128, P, NULL) == SHAPE    # 32-bit tile offsets
    for i in range(5):
        args = [P, P, P, P]
        ptrs = args + [P]
        ptrs[i] = NULL
        assert f(ptrs[0], ptrs[1], ptrs[2], ptrs[3], 4, 128, 128, ptrs[4], NULL) == INVALID
    assert f(P4, P, P, P, 4, 128, 128, P, NULL) == ALIGN
    assert f(P, P, P4, P, 4, 128, 128, P, NULL) == ALIGN
    assert f(P, P, P, P, 4, 128, 128, P4, NULL) == ALIGN
    assert f(P, P + 1, P, P, 4, 128, 128, P, NULL) == ALIGN
    assert f(NULL, NULL, NULL, NULL, 0, 128, 128, NULL, NULL) == OK


def test_gemm_ws_validation(lib):
    f = lib.fp8blk_gemm_ws
    size = lib.fp8blk_gemm_workspace_size
    # the same argument checks as fp8blk_gemm, before the workspace is looked at
    assert f(P, P, P, P, -1, 128, 128, P, P, 1 << 30, NULL) == INVALID
    assert f(P, P, P, P, 4, 130, 128, P, P, 1 << 30, NULL) == SHAPE
    assert f(P4, P, P, P, 4, 128, 128, P, P, 1 << 30, NULL) == ALIGN
    assert f(NULL, NULL, NULL, NULL, 0, 128, 128, NULL, P, 0, NULL) == OK
    # a decode step's down projection (256 x 4096, K = 14336): 32 column tiles of 128, K split 8 ways
    need = size(256, 4096, 14336)
    assert need == 8 * 256 * 4096 * 4
    assert f(P, P, P, P, 256, 4096, 14336, P, P, need - 1, NULL) == INVALID
    assert f(P, P, P, P, 256, 4096, 14336, P, P + 4, need, NULL) == ALIGN
    # ranges of at least 8 K blocks, at least 64 blocks in all; a wide layer fills the CUs unsplit;
    # more than 256 rows never split
    assert size(1, 256, 8192) == 8 * 1 * 256 * 4
    assert size(256, 12288, 8192) == 2 * 256 * 12288 * 4
    assert size(256, 4096, 4096) == 0
    assert size(256, 28672, 16384) == 0
    assert size(257, 4096, 14336) == 0
    assert size(0, 4096, 14336) == 0 and size(256, 130, 14336) == 0 and size(256, 4096, 130) == 0


def test_grouped_gemm_validation(lib):
    f = lib.fp8blk_grouped_gemm
    assert f(P, P, P, P, P, 0, 4, 128, 128, P, NULL) == SHAPE          # E < 1
    assert f(P, P, P, P, P, 2, -1, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P, P, 2, 4, 100, 128, P, NULL) == SHAPE
    assert f(P, P, P, P, P, 2, 4, 128, (1 << 24) + 128, P, NULL) == SHAPE
    assert f(P, P, P, P, NULL, 2, 4, 128, 128, P, NULL) == INVALID      # offsets
    assert f(P, P, P, P, P + 2, 2, 4, 128, 128, P, NULL) == ALIGN
    assert f(P, P, P4, P, P, 2, 4, 128, 128, P, NULL) == ALIGN
    assert f(NULL, NULL, NULL, NULL, NULL, 3, 0, 128, 128, NULL, NULL) == OK


def test_rmsnorm_quant_act_validation(lib):
    f = lib.fp8blk_rmsnorm_quant_act
    assert f(P, P, 1e-5, -1, 128, P, P, P, 0, NULL) == INVALID
    assert f(P, P, 1e-5, 4, 0, P, P, P, 0, NULL) == INVALID
    assert f(P, P, 1e-5, 4, 128, P, P, P, 2, NULL) == INVALID          # pow2 flag
    assert f(P, P, -1e-5, 4, 128, P, P, P, 0, NULL) == INVALID         # eps < 0
    assert f(P, P, float("nan"), 4, 128, P, P, P, 0, NULL) == INVALID
    assert f(P, P, float("inf"), 4, 128, P, P, P, 0, NULL) == INVALID
    assert f(P, P, 1e-5, 4, 100, P, P, P, 0, NULL) == SHAPE
    for i in range(4):
        ptrs = [P, P, P, P]
        ptrs[i] = NULL
        assert f(ptrs[0], ptrs[1], 1e-5, 4, 128, ptrs[2], ptrs[3], P, 0, NULL) == INVALID
    assert f(P4, P, 1e-5, 4, 128, P, P, P, 0, NULL) == ALIGN
    assert f(P, P4, 1e-5, 4, 128, P, P, P, 0, NULL) == ALIGN           # gamma
    assert f(P, P, 1e-5, 4, 128, P4, P, P, 0, NULL) == ALIGN
    assert f(P, P, 1e-5, 4, 128, P, P + 2, P, 0, NULL) == ALIGN
    assert f(P, P, 1e-5, 4, 128, P, P, P4, 0, NULL) == ALIGN           # y, when given
    assert f(NULL, NULL, 0.0, 0, 128, NULL, NULL, NULL, 1, NULL) == OK  # M == 0 is a no-op


def test_silu_mul_quant_act_validation(lib):
    f = lib.fp8blk_silu_mul_quant_act
    assert f(P, -1, 128, P, P, P, 0, NULL) == INVALID
    assert f(P, 4, 0, P, P, P, 0, NULL) == INVALID
    assert f(P, 4, 128, P, P, P, 3, NULL) == INVALID
    assert f(P, 4, 192, P, P, P, 0, NULL) == SHAPE
    assert f(NULL, 4, 128, P, P, P, 0, NULL) == INVALID
    assert f(P, 4, 128, NULL, P, P, 0, NULL) == INVALID
    assert f(P, 4, 128, P, NULL, P, 0, NULL) == INVALID
    assert f(P4, 4, 128, P, P, P, 0, NULL) == ALIGN
    assert f(P, 4, 128, P4, P, P, 0, NULL) == ALIGN
    assert f(P, 4, 128, P, P + 1, P, 0, NULL) == ALIGN
    assert f(P, 4, 128, P, P, P4, 0, NULL) == ALIGN
    assert f(NULL, 0, 128, NULL, NULL, NULL, 0, NULL) == OK


def test_qkv_amax_validation(lib):
    f = lib.fp8blk_qkv_amax
    assert f(P, -1, 32, 8, 128, P, 1, NULL) == INVALID
    assert f(P, 4, 0, 8, 128, P, 1, NULL) == INVALID
    assert f(P, 4, 32, 0, 128, P, 1, NULL) == INVALID
    assert f(P, 4, 32, 8, 0, P, 1, NULL) == INVALID
    assert f(P, 4, 32, 8, 128, P, 2, NULL) == INVALID       # reset flag
    assert f(P, 4, 32, 8, 100, P, 1, NULL) == SHAPE          # D % 8
    assert f(NULL, 4, 32, 8, 128, P, 1, NULL) == INVALID
    assert f(P, 4, 32, 8, 128, NULL, 1, NULL) == INVALID
    assert f(P4, 4, 32, 8, 128, P, 1, NULL) == ALIGN
    assert f(P, 4, 32, 8, 128, P + 2, 1, NULL) == ALIGN
    assert f(NULL, 0, 32, 8, 128, P, 0, NULL) == OK          # T == 0 without reset: nothing to do


def test_kv_scales_validation(lib):
    f = lib.fp8blk_kv_scales
    assert f(P, -1, P, 0, NULL) == INVALID
    assert f(P, 3, P, 5, NULL) == INVALID
    assert f(NULL, 3, P, 0, NULL) == INVALID
    assert f(P, 3, NULL, 0, NULL) == INVALID
    assert f(P + 1, 3, P, 0, NULL) == ALIGN
    assert f(NULL, 0, NULL, 0, NULL) == OK


def test_kv_cache_write_validation(lib):
    f = lib.fp8blk_kv_cache_write
    ok = [P, P, 1024, 4, 8, 128, P, 16, 16, P, P, P, P, NULL]

    def call(**kw):
        a = list(ok)
        names = ["k", "v", "ld", "T", "Hkv", "D", "slot", "slots", "bs", "ks", "vs", "kc", "vc", "stream"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)
    assert call(T=-1) == INVALID
    assert call(Hkv=0) == INVALID
    assert call(D=0) == INVALID
    assert call(slots=-1) == INVALID
    assert call(ld=1000) == INVALID                           # ld < Hkv*D
    assert call(D=100, ld=800) == SHAPE                       # D % 8
    assert call(ld=1028) == SHAPE                             # ld % 8
    assert call(bs=0) == INVALID
    assert call(slots=24) == SHAPE                            # not whole pages of 16
    for name in ("k", "v", "slot", "ks", "vs", "kc", "vc"):
        assert call(**{name: NULL}) == INVALID, name
    for name, bad in (("k", P4), ("v", P4), ("slot", P4), ("ks", P + 2), ("kc", P4), ("vc", P4)):
        assert call(**{name: bad}) == ALIGN, name
    assert call(T=0, k=NULL, v=NULL, slot=NULL) == OK


def test_transposed_quant_validation(lib):
    f = lib.fp8blk_quant_act_t
    assert f(P, -128, 128, P, P, 0, NULL) == INVALID
    assert f(P, 128, 0, P, P, 0, NULL) == INVALID
    assert f(P, 128, 128, P, P, 2, NULL) == INVALID
    assert f(P, 100, 128, P, P, 0, NULL) == SHAPE          # M % 128
    assert f(P, 128, 96, P, P, 0, NULL) == SHAPE           # K % 64
    assert f(NULL, 128, 128, P, P, 0, NULL) == INVALID
    assert f(P, 128, 128, P4, P, 0, NULL) == ALIGN
    assert f(P, 128, 128, P, P + 2, 0, NULL) == ALIGN
    assert f(NULL, 0, 128, NULL, NULL, 0, NULL) == OK
    g = lib.fp8blk_quant_weight_t
    assert g(P, 100, 128, P, P, 0, NULL) == SHAPE
    assert g(P, 128, 200, P, P, 0, NULL) == SHAPE
    assert g(P, 128, 128, P, P, -1, NULL) == INVALID
    assert g(P, 128, 128, NULL, P, 0, NULL) == INVALID
    assert g(P4, 128, 128, P, P, 0, NULL) == ALIGN
    assert g(NULL, 0, 128, NULL, NULL, 0, NULL) == OK


def test_gemm_rowscaled_validation(lib):
    f = lib.fp8blk_gemm_rowscaled
    assert f(P, P, P, P, -1, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 130, 128, P, NULL) == SHAPE
    assert f(P, P, P, P, 4, 128, (1 << 24) + 128, P, NULL) == SHAPE
    assert f(P, P, NULL, P, 4, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P + 1, 4, 128, 128, P, NULL) == ALIGN
    assert f(NULL, NULL, NULL, NULL, 0, 128, 128, NULL, NULL) == OK


def test_decode_attention_validation(lib):
    f = lib.fp8blk_decode_attention
    names = ["q", "ldq", "B", "Hq", "Hkv", "D", "kc", "vc", "slots", "table", "max_blocks", "bs", "lens",
             "qs", "ks", "vs", "sm", "out", "ldo", "split", "ws", "ws_bytes", "stream"]
    ok = [P, 4096, 4, 32, 8, 128, P, P, 1024, P, 16, 16, P, P, P, P, 0.088, P, 4096, 0, NULL, 0, NULL]

    def call(**kw):
        a = list(ok)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)
    assert call(B=-1) == INVALID
    assert call(Hq=0) == INVALID
    assert call(max_blocks=0) == INVALID
    assert call(bs=0) == INVALID
    assert call(sm=float("nan")) == INVALID
    assert call(ldq=1024) == INVALID                      # ldq < Hq*D
    assert call(D=64, ldq=2048, ldo=2048) == SHAPE        # D != 128
    assert call(Hq=12) == SHAPE                           # Hq % Hkv
    assert call(Hq=128, ldq=16384, ldo=16384) == SHAPE    # Hq / Hkv = 16
    assert call(ldq=4100) == SHAPE
    assert call(slots=1000) == SHAPE                       # not whole pages of 16
    assert call(slots=1 << 28, Hkv=8) == SHAPE             # num_slots * Hkv >= 2^31
    for name in ("q", "kc", "vc", "table", "lens", "qs", "ks", "vs", "out"):
        assert call(**{name: NULL}) == INVALID, name
    for name, bad in (("q", P4), ("kc", P4), ("out", P4), ("table", P + 2), ("qs", P + 1)):
        assert call(**{name: bad}) == ALIGN, name
    assert call(B=0, q=NULL, out=NULL) == OK
    assert call(split=-256) == INVALID
    assert call(split=100) == SHAPE                        # not a multiple of 256
    assert call(ws=P + 8, ws_bytes=1 << 30) == ALIGN
    need = lib.fp8blk_decode_attention_workspace_size(4, 32, 8, 128, 256, 16, 0)
    assert need > 0
    assert call(max_blocks=256, ws=P, ws_bytes=need - 4) == INVALID   # workspace too small


def test_decode_attention_workspace_size(lib):
    size = lib.fp8blk_decode_attention_workspace_size
    # 4 sequences, 32/8 heads, 16 blocks of 16 tokens: one 256-token chunk -> not split
    assert size(4, 32, 8, 128, 16, 16, 0) == 0
    # 4096 addressable tokens, 32 (sequence, KV head) pairs: the automatic
    # chunk would bring the grid to 512 workgroups (16 chunks of 256) but is
    # at least 2048 tokens: 2 chunks; partials of (128 + 2) floats per query
    # head and chunk
    assert size(4, 32, 8, 128, 256, 16, 0) == 4 * 32 * 2 * 130 * 4
    # 32768 tokens, 32 pairs: 16 chunks of 2048 (512 workgroups)
    assert size(4, 32, 8, 128, 2048, 16, 0) == 4 * 32 * 16 * 130 * 4
    # 16384 tokens, 256 pairs: 2 chunks of 8192
    assert size(32, 32, 8, 128, 1024, 16, 0) == 32 * 32 * 2 * 130 * 4
    assert size(4, 32, 8, 128, 256, 16, 1024) == 4 * 32 * 4 * 130 * 4
    # 64 x 8 pairs fill the chip without splitting
    assert size(64, 32, 8, 128, 256, 16, 0) == 0
    assert size(256, 32, 8, 128, 256, 16, 0) == 0
    assert size(256, 32, 8, 128, 256, 16, 256) == 256 * 32 * 16 * 130 * 4
    assert size(4, 32, 8, 64, 256, 16, 0) == 0             # D != 128
    assert size(4, 32, 8, 128, 256, 16, 100) == 0          # split not a multiple of 256
    assert size(0, 32, 8, 128, 256, 16, 0) == 0


def test_grouped_backward_validation(lib):
    f = lib.fp8blk_quant_weight_t_grouped
    assert f(P, 0, 128, 128, P, P, 0, NULL) == INVALID          # E < 1
    assert f(P, 65536, 128, 128, P, P, 0, NULL) == SHAPE
    assert f(P, 2, 130, 128, P, P, 0, NULL) == SHAPE
    assert f(P4, 2, 128, 128, P, P, 0, NULL) == ALIGN
    assert f(NULL, 2, 0, 128, NULL, NULL, 0, NULL) == OK         # N == 0: no-op
    g = lib.fp8blk_quant_act_t_grouped
    assert g(P, 100, 128, P, 0, 256, P, P, 0, NULL) == INVALID    # E < 1
    assert g(P, 100, 100, P, 4, 256, P, P, 0, NULL) == SHAPE      # K % 64
    assert g(P, 100, 128, P, 4, 200, P, P, 0, NULL) == SHAPE      # ld % 128
    assert g(P, 100, 128, NULL, 4, 256, P, P, 0, NULL) == INVALID
    assert g(P, 100, 128, P + 2, 4, 256, P, P, 0, NULL) == ALIGN
    assert g(NULL, 0, 128, NULL, 4, 256, NULL, NULL, 0, NULL) == OK
    h = lib.fp8blk_grouped_gemm_rowscaled
    assert h(P, P, P, P, P, 0, 256, 128, 128, P, NULL) == INVALID    # E < 1
    assert h(P, P, P, P, P, 4, 256, 130, 128, P, NULL) == SHAPE
    assert h(P, P, P, P, P, 4, 200, 128, 128, P, NULL) == SHAPE       # ld % 128
    assert h(P, P, P, P, P, 4, (1 << 24) + 128, 128, 128, P, NULL) == SHAPE
    assert h(P, P, P, P, NULL, 4, 256, 128, 128, P, NULL) == INVALID
    assert h(P, P, P, P, P + 2, 4, 256, 128, 128, P, NULL) == ALIGN


def test_python_entry_points_raise(lib):
    with pytest.raises(fb.Fp8BlkError) as e:
        fb.fp8blk_gemm(P, P, P, P, 4, 130, 128, P, None)
    assert e.value.status == SHAPE


def test_tensor_api_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        fb.quant_act(torch.zeros(2, 128, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        fb.quant_act(torch.zeros(2, 128, dtype=torch.float32).cuda() if torch.cuda.is_available()
                     else torch.zeros(2, 128, dtype=torch.float32))


def test_gemm_noalloc_validation(lib):
    """The allocation-free GEMM checks its arguments like fp8blk_gemm, before
    any HIP call (the device lookup of its scratch comes after)."""
    f = lib.fp8blk_gemm_noalloc
    assert f(P, P, P, P, -1, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 0, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 100, 128, P, NULL) == SHAPE
    assert f(P, P, P, P, 4, 128, 200, P, NULL) == SHAPE
    assert f(NULL, P, P, P, 4, 128, 128, P, NULL) == INVALID
    assert f(P, P, P, P, 4, 128, 128, NULL, NULL) == INVALID
    assert f(P4, P, P, P, 4, 128, 128, P, NULL) == ALIGN
    assert f(P, P + 2, P, P, 4, 128, 128, P, NULL) == ALIGN
    assert f(NULL, NULL, NULL, NULL, 0, 128, 128, NULL, NULL) == OK     # M == 0 is a no-op


def test_split_workspace_fits_the_static_scratch(lib):
    """Every split the rule can choose fits FP8BLK_GEMM_SCRATCH_BYTES, so the
    allocation-free GEMM never has to reject a valid shape; the header's
    constant and the binding's agree."""
    src = open(HEADER).read()
    m = re.search(r"#define FP8BLK_GEMM_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fb.GEMM_SCRATCH_BYTES
    size = lib.fp8blk_gemm_workspace_size
    worst = 0
    for mm in (1, 2, 64, 100, 128, 200, 255, 256, 257):
        for n in range(128, 40000, 128 * 7):
            for k in (4096, 8192, 8320, 12288, 14336, 28672, 1 << 20):
                worst = max(worst, size(mm, n, k))
    assert 0 < worst <= fb.GEMM_SCRATCH_BYTES
    assert size(256, 4096, 14336) == fb.GEMM_SCRATCH_BYTES    # the decode down projection: the largest


def test_prefill_attention_validation(lib):
    f = lib.fp8blk_prefill_attention

    def call(q=P, ldq=4096, total_q=16, B=2, Hq=32, Hkv=8, D=128, cu=P, mx=8, kc=P, vc=P, slots=1024, table=P,
             mb=4, bs=16, lens=P, qs=P, ks=P, vs=P, sm=0.088, out=P, ldo=4096):
        return f(q, ldq, total_q, B, Hq, Hkv, D, cu, mx, kc, vc, slots, table, mb, bs, lens, qs, ks, vs, sm, out, ldo,
                 NULL)

    assert call(B=-1) == INVALID
    assert call(total_q=-1) == INVALID
    assert call(mx=-1) == INVALID
    assert call(ldq=4000) == INVALID          # < Hq * D
    assert call(sm=float("nan")) == INVALID
    assert call(D=64, ldq=2048, ldo=2048) == SHAPE
    assert call(Hq=24) == SHAPE               # Hq / Hkv = 3
    assert call(Hq=128, ldq=16384, ldo=16384) == SHAPE   # Hq / Hkv = 16
    assert call(slots=1000) == SHAPE          # not whole pages
    assert call(ldq=4100) == SHAPE            # not a multiple of 8
    assert call(cu=NULL) == INVALID
    assert call(out=NULL) == INVALID
    assert call(q=P4) == ALIGN
    assert call(cu=P + 2) == ALIGN
    assert call(B=0, q=NULL, cu=NULL, out=NULL) == OK      # nothing to do
    assert call(mx=0, q=NULL, cu=NULL, out=NULL) == OK
