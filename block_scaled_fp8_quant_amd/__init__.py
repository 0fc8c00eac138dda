"""Block-scaled FP8 (E4M3) W8A8 linear layers on AMD MI355X (gfx950).

A thin ctypes binding over libfp8blk.so (declared in include/fp8blk.h).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor shapes, dtypes and devices, allocates outputs with
PyTorch and passes raw pointers plus the current HIP stream. There is no
CPU fallback: if the library is missing, every call raises.

Two layers:
  * ``fp8blk_quant_act``, ``fp8blk_quant_weight``, ``fp8blk_gemm``,
    ``fp8blk_gemm_ws``, ``fp8blk_grouped_gemm``, ``fp8blk_rmsnorm_quant_act``,
    ``fp8blk_silu_mul_quant_act``, ``fp8blk_qkv_amax``, ``fp8blk_kv_scales``,
    ``fp8blk_kv_cache_write``, ``fp8blk_quant_act_t``,
    ``fp8blk_quant_weight_t``, ``fp8blk_gemm_rowscaled``,
    ``fp8blk_decode_attention``, ``fp8blk_prefill_attention``,
    ``fp8blk_gemm_noalloc``: the C entry points under their own names
    (integer device pointers, sizes, stream handle); they raise
    ``Fp8BlkError`` on a non-OK status;
  * ``quant_act``, ``quant_weight``, ``gemm``, ``grouped_gemm``,
    ``rmsnorm_quant_act``, ``silu_mul_quant_act``, ``qkv_amax``,
    ``kv_scales``, ``kv_cache_write``, ``quant_act_t``, ``quant_weight_t``,
    ``gemm_rowscaled`` (and ``dgrad``, ``wgrad`` built from them),
    ``decode_attention``, ``prefill_attention``: tensor versions that
    validate shapes and allocate outputs.

The library loaded is the in-tree libfp8blk.so, or the file the environment
variable FP8BLK_LIB names (a variant build of the same sources, e.g. the
host-sanitizer build the CPU tests use); a missing file raises.
"""

import ctypes
import os

LIB_PATH = os.environ.get("FP8BLK_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8blk.so")
BLOCK = 128

STATUS = {0: "FP8BLK_OK", 1: "FP8BLK_ERR_INVALID_ARG", 2: "FP8BLK_ERR_SHAPE",
          3: "FP8BLK_ERR_ALIGNMENT", 4: "FP8BLK_ERR_HIP", 5: "FP8BLK_ERR_SCRATCH"}

GEMM_SCRATCH_BYTES = 32 << 20   # FP8BLK_GEMM_SCRATCH_BYTES: static scratch of fp8blk_gemm_noalloc

_lib = None


class Fp8BlkError(RuntimeError):
    def __init__(self, func, status, text):
        super().__init__("%s failed: %s (%s)" % (func, STATUS.get(status, status), text))
        self.status = status


def declare(lib):
    """Give every C entry point the library exports its ctypes signature
    (a variant build may export a subset)."""
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sigs = {
        "fp8blk_quant_act": [vp, i64, i64, vp, vp, i32, vp],
        "fp8blk_quant_weight": [vp, i64, i64, vp, vp, i32, vp],
        "fp8blk_gemm": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8blk_gemm_ws": [vp, vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_size_t, vp],
        "fp8blk_gemm_noalloc": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8blk_grouped_gemm": [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp],
        "fp8blk_rmsnorm_quant_act": [vp, vp, f32, i64, i64, vp, vp, vp, i32, vp],
        "fp8blk_silu_mul_quant_act": [vp, i64, i64, vp, vp, vp, i32, vp],
        "fp8blk_qkv_amax": [vp, i64, i64, i64, i64, vp, i32, vp],
        "fp8blk_quant_act_t": [vp, i64, i64, vp, vp, i32, vp],
        "fp8blk_decode_attention": [vp, i64, i64, i64, i64, i64, vp, vp, i64, vp, i64, i64, vp, vp, vp, vp, f32,
                                    vp, i64, i64, vp, ctypes.c_size_t, vp],
        "fp8blk_prefill_attention": [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, vp, i64, vp, i64, i64, vp, vp,
                                     vp, vp, f32, vp, i64, vp],
        "fp8blk_quant_weight_t": [vp, i64, i64, vp, vp, i32, vp],
        "fp8blk_quant_weight_t_grouped": [vp, i64, i64, i64, vp, vp, i32, vp],
        "fp8blk_quant_act_t_grouped": [vp, i64, i64, vp, i64, i64, vp, vp, i32, vp],
        "fp8blk_grouped_gemm_rowscaled": [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp],
        "fp8blk_gemm_rowscaled": [vp, vp, vp, vp, i64, i64, i64, vp, vp],
        "fp8blk_kv_scales": [vp, i64, vp, i32, vp],
        "fp8blk_kv_cache_write": [vp, vp, i64, i64, i64, i64, vp, i64, i64, vp, vp, vp, vp, vp],
    }
    for name, args in sigs.items():
        if hasattr(lib, name):
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
    if hasattr(lib, "fp8blk_gemm_workspace_size"):
        lib.fp8blk_gemm_workspace_size.argtypes = [i64, i64, i64]
        lib.fp8blk_gemm_workspace_size.restype = ctypes.c_size_t
    if hasattr(lib, "fp8blk_decode_attention_workspace_size"):
        lib.fp8blk_decode_attention_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64]
        lib.fp8blk_decode_attention_workspace_size.restype = ctypes.c_size_t
    if hasattr(lib, "fp8blk_status_string"):
        lib.fp8blk_status_string.argtypes = [ctypes.c_int]
        lib.fp8blk_status_string.restype = ctypes.c_char_p
    return lib


def load():
    """Load libfp8blk.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfp8blk.so is not built (%s); run __graft_entry__.build() "
                           "or python -m block_scaled_fp8_quant_amd.build" % LIB_PATH)
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _call(name, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise Fp8BlkError(name, st, lib.fp8blk_status_string(st).decode())
    return st


# ------------------------------------------------------------ C entry points

def fp8blk_quant_act(x, M, K, q, s, pow2, stream):
    return _call("fp8blk_quant_act", x, M, K, q, s, int(pow2), stream)


def fp8blk_quant_weight(w, N, K, q, s, pow2, stream):
    return _call("fp8blk_quant_weight", w, N, K, q, s, int(pow2), stream)


def fp8blk_gemm(qa, sa, qw, sw, M, N, K, y, stream):
    return _call("fp8blk_gemm", qa, sa, qw, sw, M, N, K, y, stream)


def fp8blk_gemm_ws(qa, sa, qw, sw, M, N, K, y, workspace, workspace_bytes, stream):
    return _call("fp8blk_gemm_ws", qa, sa, qw, sw, M, N, K, y, workspace, workspace_bytes, stream)


def fp8blk_gemm_noalloc(qa, sa, qw, sw, M, N, K, y, stream):
    return _call("fp8blk_gemm_noalloc", qa, sa, qw, sw, M, N, K, y, stream)


def fp8blk_gemm_workspace_size(M, N, K):
    return load().fp8blk_gemm_workspace_size(M, N, K)


def fp8blk_grouped_gemm(qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream):
    return _call("fp8blk_grouped_gemm", qa, sa, qw, sw, offsets, E, total_M, N, K, y, stream)


def fp8blk_rmsnorm_quant_act(x, gamma, eps, M, K, q, s, y, pow2, stream):
    return _call("fp8blk_rmsnorm_quant_act", x, gamma, eps, M, K, q, s, y, int(pow2), stream)


def fp8blk_silu_mul_quant_act(gu, M, F, q, s, y, pow2, stream):
    return _call("fp8blk_silu_mul_quant_act", gu, M, F, q, s, y, int(pow2), stream)


def fp8blk_decode_attention(q, ldq, B, Hq, Hkv, D, k_cache, v_cache, num_slots, block_table, max_blocks,
                            block_size, context_lens, q_scale, k_scale, v_scale, sm_scale, out, ldo, split_tokens,
                            workspace, workspace_bytes, stream):
    return _call("fp8blk_decode_attention", q, ldq, B, Hq, Hkv, D, k_cache, v_cache, num_slots, block_table,
                 max_blocks, block_size, context_lens, q_scale, k_scale, v_scale, sm_scale, out, ldo, split_tokens,
                 workspace, workspace_bytes, stream)


def fp8blk_prefill_attention(q, ldq, total_q, B, Hq, Hkv, D, cu_seqlens_q, max_seqlen_q, k_cache, v_cache,
                             num_slots, block_table, max_blocks, block_size, context_lens, q_scale, k_scale, v_scale,
                             sm_scale, out, ldo, stream):
    return _call("fp8blk_prefill_attention", q, ldq, total_q, B, Hq, Hkv, D, cu_seqlens_q, max_seqlen_q, k_cache,
                 v_cache, num_slots, block_table, max_blocks, block_size, context_lens, q_scale, k_scale, v_scale,
                 sm_scale, out, ldo, stream)


def fp8blk_decode_attention_workspace_size(B, Hq, Hkv, D, max_blocks, block_size, split_tokens):
    return load().fp8blk_decode_attention_workspace_size(B, Hq, Hkv, D, max_blocks, block_size, split_tokens)


def fp8blk_quant_act_t(x, M, K, qt, st, pow2, stream):
    return _call("fp8blk_quant_act_t", x, M, K, qt, st, int(pow2), stream)


def fp8blk_quant_weight_t(w, N, K, qt, st, pow2, stream):
    return _call("fp8blk_quant_weight_t", w, N, K, qt, st, int(pow2), stream)


def fp8blk_quant_weight_t_grouped(w, E, N, K, qt, st, pow2, stream):
    return _call("fp8blk_quant_weight_t_grouped", w, E, N, K, qt, st, int(pow2), stream)


def fp8blk_quant_act_t_grouped(x, M, K, offsets, E, ld, qt, st, pow2, stream):
    return _call("fp8blk_quant_act_t_grouped", x, M, K, offsets, E, ld, qt, st, int(pow2), stream)


def fp8blk_grouped_gemm_rowscaled(qa, sa, qb, sb, offsets, E, ld, N, K, y, stream):
    return _call("fp8blk_grouped_gemm_rowscaled", qa, sa, qb, sb, offsets, E, ld, N, K, y, stream)


def fp8blk_gemm_rowscaled(qa, sa, qb, sb, M, N, K, y, stream):
    return _call("fp8blk_gemm_rowscaled", qa, sa, qb, sb, M, N, K, y, stream)


def fp8blk_qkv_amax(qkv, T, Hq, Hkv, D, amax, reset, stream):
    return _call("fp8blk_qkv_amax", qkv, T, Hq, Hkv, D, amax, int(reset), stream)


def fp8blk_kv_scales(amax, n, scale, pow2, stream):
    return _call("fp8blk_kv_scales", amax, n, scale, int(pow2), stream)


def fp8blk_kv_cache_write(k, v, ld, T, Hkv, D, slot, num_slots, block_size, k_scale, v_scale, k_cache, v_cache,
                          stream):
    return _call("fp8blk_kv_cache_write", k, v, ld, T, Hkv, D, slot, num_slots, block_size, k_scale, v_scale,
                 k_cache, v_cache, stream)


# ------------------------------------------------------------ tensor API

def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def quant_act(x, pow2=False, q=None, s=None):
    """1x128 group quantisation of bf16 X[M, K] -> (Q uint8 [M, K], S fp32 [M, K/128])."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    _check(x, "x", torch.bfloat16, (m, k))
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    q = torch.empty((m, k), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((m, k // BLOCK), dtype=torch.float32, device=x.device) if s is None else s
    _check(q, "q", torch.uint8, (m, k), x.device)
    _check(s, "s", torch.float32, (m, k // BLOCK), x.device)
    fp8blk_quant_act(x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), pow2, _stream(x.device))
    return q, s


def quant_weight(w, pow2=False, q=None, s=None):
    """128x128 block quantisation of bf16 W[N, K] (or an expert stack
    [E, N, K], quantised as [E*N, K]) -> (Q uint8 like W, S fp32
    [N/128, K/128] or [E, N/128, K/128])."""
    torch = _torch()
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N, K] or [E, N, K]")
    k = w.shape[-1]
    rows = w.numel() // k if k else 0
    if w.shape[-2] % BLOCK or k % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    sshape = tuple(w.shape[:-2]) + (w.shape[-2] // BLOCK, k // BLOCK)
    _check(w, "w", torch.bfloat16, tuple(w.shape))
    q = torch.empty(tuple(w.shape), dtype=torch.uint8, device=w.device) if q is None else q
    s = torch.empty(sshape, dtype=torch.float32, device=w.device) if s is None else s
    _check(q, "q", torch.uint8, tuple(w.shape), w.device)
    _check(s, "s", torch.float32, sshape, w.device)
    fp8blk_quant_weight(w.data_ptr(), rows, k, q.data_ptr(), s.data_ptr(), pow2, _stream(w.device))
    return q, s


def gemm(qa, sa, qw, sw, y=None, split=True, workspace=None):
    """Y[M, N] bf16 = block-scaled (QA, SA) x (QW, SW)^T.

    split: few-row problems may split K over a workspace (fp8blk_gemm_ws);
    ``workspace`` (a contiguous uint8 device tensor of at least
    fp8blk_gemm_workspace_size(M, N, K) bytes) is allocated here when not
    given. split=False runs fp8blk_gemm."""
    torch = _torch()
    if qa.dim() != 2 or qw.dim() != 2:
        raise ValueError("qa must be [M, K] and qw [N, K]")
    m, k = qa.shape
    n = qw.shape[0]
    if k % BLOCK or n % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    dev = qa.device
    _check(qa, "qa", torch.uint8, (m, k))
    _check(sa, "sa", torch.float32, (m, k // BLOCK), dev)
    _check(qw, "qw", torch.uint8, (n, k), dev)
    _check(sw, "sw", torch.float32, (n // BLOCK, k // BLOCK), dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if y is None else y
    _check(y, "y", torch.bfloat16, (m, n), dev)
    need = fp8blk_gemm_workspace_size(m, n, k) if split else 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the device of qa")
        fp8blk_gemm_ws(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k, y.data_ptr(),
                       workspace.data_ptr(), workspace.numel(), _stream(dev))
    else:
        fp8blk_gemm(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n, k, y.data_ptr(),
                    _stream(dev))
    return y


def grouped_gemm(qa, sa, qw, sw, offsets, y=None):
    """Expert-grouped GEMM: rows offsets[e]..offsets[e+1]-1 of (QA, SA) use
    expert e's (QW[e], SW[e]). offsets: int32 [E+1] on the device, from 0 to
    M, nondecreasing (not checked here: checking would need a device sync)."""
    torch = _torch()
    if qa.dim() != 2 or qw.dim() != 3:
        raise ValueError("qa must be [M, K] and qw [E, N, K]")
    m, k = qa.shape
    e, n, _ = qw.shape
    if k % BLOCK or n % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    dev = qa.device
    _check(qa, "qa", torch.uint8, (m, k))
    _check(sa, "sa", torch.float32, (m, k // BLOCK), dev)
    _check(qw, "qw", torch.uint8, (e, n, k), dev)
    _check(sw, "sw", torch.float32, (e, n // BLOCK, k // BLOCK), dev)
    _check(offsets, "offsets", torch.int32, (e + 1,), dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if y is None else y
    _check(y, "y", torch.bfloat16, (m, n), dev)
    fp8blk_grouped_gemm(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), offsets.data_ptr(),
                        e, m, n, k, y.data_ptr(), _stream(dev))
    return y


def _fused_outputs(m, k, dev, want_y, q, s, y):
    torch = _torch()
    q = torch.empty((m, k), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((m, k // BLOCK), dtype=torch.float32, device=dev) if s is None else s
    if y is None and want_y:
        y = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    _check(q, "q", torch.uint8, (m, k), dev)
    _check(s, "s", torch.float32, (m, k // BLOCK), dev)
    if y is not None:
        _check(y, "y", torch.bfloat16, (m, k), dev)
    return q, s, y


def rmsnorm_quant_act(x, gamma, eps, pow2=False, want_y=False, q=None, s=None, y=None):
    """RMSNorm of bf16 X[M, K] with weights gamma[K], rounded to bf16 and
    quantised per 1x128 group in one kernel -> (Q uint8 [M, K], S fp32
    [M, K/128], Y bf16 [M, K] or None). Y (the normalised bf16 values) is
    written if want_y or a y tensor is given."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    _check(x, "x", torch.bfloat16, (m, k))
    _check(gamma, "gamma", torch.bfloat16, (k,), x.device)
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    q, s, y = _fused_outputs(m, k, x.device, want_y, q, s, y)
    fp8blk_rmsnorm_quant_act(x.data_ptr(), gamma.data_ptr(), float(eps), m, k, q.data_ptr(), s.data_ptr(),
                             None if y is None else y.data_ptr(), pow2, _stream(x.device))
    return q, s, y


def silu_mul_quant_act(gu, pow2=False, want_y=False, q=None, s=None, y=None):
    """SiLU(gate) * up of bf16 GU[M, 2F] = [gate | up], rounded to bf16 and
    quantised per 1x128 group in one kernel -> (Q uint8 [M, F], S fp32
    [M, F/128], Y bf16 [M, F] or None)."""
    torch = _torch()
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be 2-D [M, 2F]")
    m, f = gu.shape[0], gu.shape[1] // 2
    _check(gu, "gu", torch.bfloat16, (m, 2 * f))
    if f % BLOCK:
        raise ValueError("F must be a multiple of 128")
    q, s, y = _fused_outputs(m, f, gu.device, want_y, q, s, y)
    fp8blk_silu_mul_quant_act(gu.data_ptr(), m, f, q.data_ptr(), s.data_ptr(),
                              None if y is None else y.data_ptr(), pow2, _stream(gu.device))
    return q, s, y


def quant_act_t(x, pow2=False, qt=None, st=None):
    """128x1 groups of bf16 X[M, K] (M % 128 == 0), written transposed ->
    (Q^T uint8 [K, M], S^T fp32 [K, M/128])."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    _check(x, "x", torch.bfloat16, (m, k))
    if m % BLOCK or k % 64:
        raise ValueError("M must be a multiple of 128 and K of 64")
    qt = torch.empty((k, m), dtype=torch.uint8, device=x.device) if qt is None else qt
    st = torch.empty((k, m // BLOCK), dtype=torch.float32, device=x.device) if st is None else st
    _check(qt, "qt", torch.uint8, (k, m), x.device)
    _check(st, "st", torch.float32, (k, m // BLOCK), x.device)
    fp8blk_quant_act_t(x.data_ptr(), m, k, qt.data_ptr(), st.data_ptr(), pow2, _stream(x.device))
    return qt, st


def quant_weight_t(w, pow2=False, qt=None, st=None):
    """128x128 block quantisation of bf16 W[N, K], written transposed ->
    (QW^T uint8 [K, N], SW^T fp32 [K/128, N/128]); an expert stack
    [E, N, K] gives [E, K, N] and [E, K/128, N/128] (each expert's W^T)."""
    torch = _torch()
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N, K] or an expert stack [E, N, K]")
    e = w.shape[0] if w.dim() == 3 else 1
    n, k = w.shape[-2:]
    _check(w, "w", torch.bfloat16, tuple(w.shape))
    if n % BLOCK or k % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    lead = (e,) if w.dim() == 3 else ()
    qt = torch.empty(lead + (k, n), dtype=torch.uint8, device=w.device) if qt is None else qt
    st = torch.empty(lead + (k // BLOCK, n // BLOCK), dtype=torch.float32, device=w.device) if st is None else st
    _check(qt, "qt", torch.uint8, lead + (k, n), w.device)
    _check(st, "st", torch.float32, lead + (k // BLOCK, n // BLOCK), w.device)
    fp8blk_quant_weight_t_grouped(w.data_ptr(), e, n, k, qt.data_ptr(), st.data_ptr(), pow2, _stream(w.device))
    return qt, st


def padded_tokens(m, e):
    """Length of the padded token axis the grouped wgrad operands are laid
    out on: room for every expert's tokens rounded up to 128 (at most
    m + 127 e), as a multiple of 128."""
    return (m // BLOCK + e) * BLOCK


def quant_act_t_grouped(x, offsets, pow2=False, ld=None, qt=None, st=None):
    """128x1 groups of bf16 X [M, K] whose rows are sorted by expert
    (offsets int32 [E+1] on the device): each expert's groups start at its
    first row, its last group completed with zeros. Written transposed on a
    padded token axis of ld columns (default padded_tokens(M, E)): expert e
    owns columns pad[e] .. pad[e+1], pad[e] = sum over e' < e of
    ceil(M_e' / 128) * 128. Returns (Q^T uint8 [K, ld], S^T fp32 [K, ld/128]);
    columns past pad[E] are not written."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    e = offsets.shape[0] - 1
    dev = x.device
    _check(x, "x", torch.bfloat16, (m, k))
    _check(offsets, "offsets", torch.int32, (e + 1,), dev)
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    ld = padded_tokens(m, e) if ld is None else ld
    qt = torch.empty((k, ld), dtype=torch.uint8, device=dev) if qt is None else qt
    st = torch.empty((k, ld // BLOCK), dtype=torch.float32, device=dev) if st is None else st
    _check(qt, "qt", torch.uint8, (k, ld), dev)
    _check(st, "st", torch.float32, (k, ld // BLOCK), dev)
    fp8blk_quant_act_t_grouped(x.data_ptr(), m, k, offsets.data_ptr(), e, ld, qt.data_ptr(), st.data_ptr(), pow2,
                               _stream(dev))
    return qt, st


def grouped_gemm_rowscaled(qa, sa, qb, sb, offsets, y=None):
    """Expert-grouped GEMM with per-row scales on both operands over each
    expert's tokens (the grouped wgrad): qa [N, ld] / sa [N, ld/128] and
    qb [K, ld] / sb [K, ld/128] from quant_act_t_grouped with the same
    offsets. Returns Y bf16 [E, N, K]."""
    torch = _torch()
    if qa.dim() != 2 or qb.dim() != 2 or qa.shape[1] != qb.shape[1]:
        raise ValueError("qa must be [N, ld] and qb [K, ld]")
    n, ld = qa.shape
    k = qb.shape[0]
    e = offsets.shape[0] - 1
    dev = qa.device
    if n % BLOCK or k % BLOCK or ld % BLOCK:
        raise ValueError("N, K and ld must be multiples of 128")
    _check(qa, "qa", torch.uint8, (n, ld))
    _check(sa, "sa", torch.float32, (n, ld // BLOCK), dev)
    _check(qb, "qb", torch.uint8, (k, ld), dev)
    _check(sb, "sb", torch.float32, (k, ld // BLOCK), dev)
    _check(offsets, "offsets", torch.int32, (e + 1,), dev)
    y = torch.empty((e, n, k), dtype=torch.bfloat16, device=dev) if y is None else y
    _check(y, "y", torch.bfloat16, (e, n, k), dev)
    fp8blk_grouped_gemm_rowscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), offsets.data_ptr(),
                                  e, ld, n, k, y.data_ptr(), _stream(dev))
    return y


def gemm_rowscaled(qa, sa, qb, sb, y=None):
    """Y[M, N] bf16 = sum_b SA[m, b] SB[n, b] (QA QB^T over K block b):
    per-row scales on both operands."""
    torch = _torch()
    if qa.dim() != 2 or qb.dim() != 2:
        raise ValueError("qa must be [M, K] and qb [N, K]")
    m, k = qa.shape
    n = qb.shape[0]
    if k % BLOCK or n % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    dev = qa.device
    _check(qa, "qa", torch.uint8, (m, k))
    _check(sa, "sa", torch.float32, (m, k // BLOCK), dev)
    _check(qb, "qb", torch.uint8, (n, k), dev)
    _check(sb, "sb", torch.float32, (n, k // BLOCK), dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if y is None else y
    _check(y, "y", torch.bfloat16, (m, n), dev)
    fp8blk_gemm_rowscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), m, n, k, y.data_ptr(),
                          _stream(dev))
    return y


def dgrad(dy, qwt, swt, pow2=False):
    """dX = dY W for Y = X W^T: dY [M, N] bf16 quantised in 1x128 groups,
    times the transposed weight codes (qwt [K, N], swt [K/128, N/128] from
    quant_weight_t). Returns dX bf16 [M, K]."""
    qa, sa = quant_act(dy, pow2)
    return gemm(qa, sa, qwt, swt)


def grouped_dgrad(dy, qwt, swt, offsets, pow2=False):
    """dX = dY_e W_e per expert: dY [M, N] (rows sorted by expert) in 1x128
    groups, times each expert's transposed weight codes (qwt [E, K, N], swt
    [E, K/128, N/128] from quant_weight_t of the stack). Returns dX bf16
    [M, K]."""
    qa, sa = quant_act(dy, pow2)
    return grouped_gemm(qa, sa, qwt, swt, offsets)


def grouped_wgrad(dy, x, offsets, pow2=False):
    """dW_e = dY_e^T X_e per expert (rows sorted by expert, offsets int32
    [E+1] on the device), both operands in 128x1 groups along each expert's
    tokens (the last group of an expert completed with zeros). Returns dW
    bf16 [E, N, K]."""
    qa, sa = quant_act_t_grouped(dy, offsets, pow2)
    qb, sb = quant_act_t_grouped(x, offsets, pow2)
    return grouped_gemm_rowscaled(qa, sa, qb, sb, offsets)


def wgrad(dy, x, pow2=False):
    """dW = dY^T X for Y = X W^T: dY [M, N] and X [M, K] (bf16, M % 128 ==
    0) quantised in 128x1 groups. Returns dW bf16 [N, K]."""
    qa, sa = quant_act_t(dy, pow2)
    qb, sb = quant_act_t(x, pow2)
    return gemm_rowscaled(qa, sa, qb, sb)


def decode_attention(q, k_cache, v_cache, block_table, block_size, context_lens, q_scale, k_scale, v_scale,
                     sm_scale=None, out=None, split=True, split_tokens=0, workspace=None):
    """FP8 decode attention: q [B, Hq, D] bf16 (or [B, Hq*D] rows with a row
    stride, e.g. a view into a qkv output), caches [slots, Hkv, D] uint8,
    block_table [B, max_blocks] int32, context_lens [B] int32, one-element
    fp32 scale tensors, all on the device. The caches are head-major pages
    [num_blocks, Hkv, block_size, D] (what kv_cache_write fills); block_size
    must match their third dimension. Returns out [B, Hq, D] bf16.
    split=False runs one workgroup per (sequence, KV head) over the whole
    context; otherwise contexts are cut into chunks of split_tokens tokens
    (0: the library's choice) whose partials go to ``workspace`` (a uint8
    device tensor, allocated here when None)."""
    torch = _torch()
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D] and alike")
    nblk, hkv, bs, d = k_cache.shape
    if bs != block_size:
        raise ValueError("block_size %d does not match the caches' pages of %d tokens" % (block_size, bs))
    slots = nblk * bs
    b = q.shape[0]
    hq = (q.shape[1] * q.shape[2] if q.dim() == 3 else q.shape[1]) // d
    dev = q.device
    if q.dtype != torch.bfloat16 or dev.type != "cuda":
        raise TypeError("q must be bf16 on a HIP device")
    if q.stride(-1) != 1 or (q.dim() == 3 and q.stride(1) != d):
        raise ValueError("each row of q must hold its Hq heads contiguously")
    ldq = q.stride(0) if b > 1 else hq * d
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype != torch.uint8 or c.device != dev or not c.is_contiguous():
            raise ValueError("%s must be a contiguous uint8 tensor on the device of q" % name)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks]")
    _check(block_table, "block_table", torch.int32, (b, block_table.shape[1]), dev)
    _check(context_lens, "context_lens", torch.int32, (b,), dev)
    for name, sc in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check(sc.reshape(-1), name, torch.float32, (1,), dev)
    out = torch.empty((b, hq, d), dtype=torch.bfloat16, device=dev) if out is None else out
    _check(out, "out", torch.bfloat16, (b, hq, d), dev)
    sm = 1.0 / d ** 0.5 if sm_scale is None else float(sm_scale)
    ws_ptr, ws_bytes = None, 0
    if split:
        need = fp8blk_decode_attention_workspace_size(b, hq, hkv, d, block_table.shape[1], block_size, split_tokens)
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous uint8 tensor on the device of q")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    fp8blk_decode_attention(q.data_ptr(), ldq, b, hq, hkv, d, k_cache.data_ptr(), v_cache.data_ptr(), slots,
                            block_table.data_ptr(), block_table.shape[1], block_size, context_lens.data_ptr(),
                            q_scale.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), sm, out.data_ptr(), hq * d,
                            split_tokens, ws_ptr, ws_bytes, _stream(dev))
    return out


def prefill_attention(q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, block_table, block_size, context_lens,
                      q_scale, k_scale, v_scale, sm_scale=None, out=None):
    """FP8 prefill attention: q [total_q, Hq, D] bf16 (or [total_q, Hq*D]
    rows with a row stride, e.g. a view into a qkv output) holding the new
    tokens of every sequence, sequence b's rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1 (int32 [B+1] on the device); new token i of
    sequence b attends causally to cached tokens 0 .. context_lens[b] - n_b
    + i of the head-major paged caches [num_blocks, Hkv, block_size, D].
    max_seqlen_q: a host bound on the new tokens per sequence. Returns out
    [total_q, Hq, D] bf16."""
    torch = _torch()
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D] and alike")
    nblk, hkv, bs, d = k_cache.shape
    if bs != block_size:
        raise ValueError("block_size %d does not match the caches' pages of %d tokens" % (block_size, bs))
    tq = q.shape[0]
    hq = (q.shape[1] * q.shape[2] if q.dim() == 3 else q.shape[1]) // d
    dev = q.device
    if q.dtype != torch.bfloat16 or dev.type != "cuda":
        raise TypeError("q must be bf16 on a HIP device")
    if q.stride(-1) != 1 or (q.dim() == 3 and q.stride(1) != d):
        raise ValueError("each row of q must hold its Hq heads contiguously")
    ldq = q.stride(0) if tq > 1 else hq * d
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype != torch.uint8 or c.device != dev or not c.is_contiguous():
            raise ValueError("%s must be a contiguous uint8 tensor on the device of q" % name)
    if block_table.dim() != 2 or cu_seqlens_q.dim() != 1:
        raise ValueError("block_table must be [B, max_blocks] and cu_seqlens_q [B + 1]")
    b = block_table.shape[0]
    _check(block_table, "block_table", torch.int32, (b, block_table.shape[1]), dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, (b + 1,), dev)
    _check(context_lens, "context_lens", torch.int32, (b,), dev)
    for name, sc in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check(sc.reshape(-1), name, torch.float32, (1,), dev)
    out = torch.empty((tq, hq, d), dtype=torch.bfloat16, device=dev) if out is None else out
    _check(out, "out", torch.bfloat16, (tq, hq, d), dev)
    sm = 1.0 / d ** 0.5 if sm_scale is None else float(sm_scale)
    fp8blk_prefill_attention(q.data_ptr(), ldq, tq, b, hq, hkv, d, cu_seqlens_q.data_ptr(), int(max_seqlen_q),
                             k_cache.data_ptr(), v_cache.data_ptr(), nblk * bs, block_table.data_ptr(),
                             block_table.shape[1], block_size, context_lens.data_ptr(), q_scale.data_ptr(),
                             k_scale.data_ptr(), v_scale.data_ptr(), sm, out.data_ptr(), hq * d, _stream(dev))
    return out


def qkv_amax(qkv, hq, hkv, d, amax=None, reset=True):
    """Running maxima of |Q|, |K|, |V| of a qkv projection output [T,
    (hq + 2*hkv)*d] (bf16, rows [Q | K | V]) into amax (fp32 [3] on the
    device; allocated when None). reset=False folds this chunk into the
    existing maxima. Returns amax."""
    torch = _torch()
    if qkv.dim() != 2:
        raise ValueError("qkv must be 2-D [T, (Hq + 2*Hkv) * D]")
    t, c = qkv.shape
    if c != (hq + 2 * hkv) * d:
        raise ValueError("qkv has %d columns, expected (Hq + 2*Hkv) * D = %d" % (c, (hq + 2 * hkv) * d))
    _check(qkv, "qkv", torch.bfloat16, (t, c))
    if amax is None:
        amax = torch.empty(3, dtype=torch.float32, device=qkv.device)
        reset = True
    _check(amax, "amax", torch.float32, (3,), qkv.device)
    fp8blk_qkv_amax(qkv.data_ptr(), t, hq, hkv, d, amax.data_ptr(), reset, _stream(qkv.device))
    return amax


def kv_scales(amax, pow2=False, scale=None):
    """Per-tensor scales from maxima (fp32 [n] on the device)."""
    torch = _torch()
    if amax.dim() != 1:
        raise ValueError("amax must be 1-D")
    n = amax.shape[0]
    _check(amax, "amax", torch.float32, (n,))
    scale = torch.empty(n, dtype=torch.float32, device=amax.device) if scale is None else scale
    _check(scale, "scale", torch.float32, (n,), amax.device)
    fp8blk_kv_scales(amax.data_ptr(), n, scale.data_ptr(), pow2, _stream(amax.device))
    return scale


def kv_cache_write(k, v, slot, k_scale, v_scale, k_cache, v_cache):
    """Quantize the K and V rows of T tokens ([T, Hkv*D] bf16, or column
    slices of a qkv output whose rows are contiguous) with the per-tensor
    scales (fp32 tensors of one element on the device) and write them to the
    paged caches k_cache / v_cache ([num_blocks, Hkv, block_size, D] uint8,
    head-major pages) at slots slot[t] (int64 [T] on the device; negative =
    skip; slot = block * block_size + offset)."""
    torch = _torch()
    if k.dim() != 2 or v.shape != k.shape:
        raise ValueError("k and v must be 2-D and of the same shape")
    t, width = k.shape
    dev = k.device
    for name, x in (("k", k), ("v", v)):
        if x.dtype != torch.bfloat16 or x.device != dev or x.device.type != "cuda":
            raise TypeError("%s must be bf16 on the same HIP device" % name)
        if x.stride(1) != 1 or (t > 1 and x.stride(0) != k.stride(0)):
            raise ValueError("%s rows must be contiguous with a common row stride" % name)
    ld = k.stride(0) if t > 1 else width
    if k_cache.dim() != 4:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, D]")
    nblk, hkv, bs, d = k_cache.shape
    if hkv * d != width:
        raise ValueError("cache pages hold %d x %d values per token, k rows %d" % (hkv, d, width))
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype != torch.uint8 or c.device != dev or not c.is_contiguous() or c.shape != k_cache.shape:
            raise ValueError("%s must be a contiguous uint8 cache like k_cache on the same device" % name)
    _check(slot, "slot", torch.int64, (t,), dev)
    _check(k_scale.reshape(-1), "k_scale", torch.float32, (1,), dev)
    _check(v_scale.reshape(-1), "v_scale", torch.float32, (1,), dev)
    fp8blk_kv_cache_write(k.data_ptr(), v.data_ptr(), ld, t, hkv, d, slot.data_ptr(), nblk * bs, bs,
                          k_scale.data_ptr(), v_scale.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                          _stream(dev))


def linear(x, qw, sw, pow2=False):
    """One W8A8 linear layer: quantise X per 1x128 group, then the
    block-scaled GEMM against pre-quantised weights. Returns Y bf16."""
    qa, sa = quant_act(x, pow2)
    return gemm(qa, sa, qw, sw)


__all__ = [
    "BLOCK", "Fp8BlkError", "LIB_PATH", "load",
    "fp8blk_quant_act", "fp8blk_quant_weight", "fp8blk_gemm", "fp8blk_gemm_ws", "fp8blk_gemm_workspace_size",
    "fp8blk_grouped_gemm",
    "fp8blk_rmsnorm_quant_act", "fp8blk_silu_mul_quant_act",
    "fp8blk_qkv_amax", "fp8blk_kv_scales", "fp8blk_kv_cache_write",
    "fp8blk_quant_act_t", "fp8blk_quant_weight_t", "fp8blk_gemm_rowscaled", "fp8blk_decode_attention",
    "fp8blk_decode_attention_workspace_size", "fp8blk_quant_weight_t_grouped", "fp8blk_quant_act_t_grouped",
    "fp8blk_grouped_gemm_rowscaled",
    "quant_act", "quant_weight", "gemm", "grouped_gemm", "rmsnorm_quant_act", "silu_mul_quant_act",
    "qkv_amax", "kv_scales", "kv_cache_write", "quant_act_t", "quant_weight_t", "gemm_rowscaled",
    "dgrad", "wgrad", "decode_attention", "linear", "padded_tokens", "quant_act_t_grouped",
    "grouped_gemm_rowscaled", "grouped_dgrad", "grouped_wgrad",
]
