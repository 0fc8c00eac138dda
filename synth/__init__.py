"""Seeded synthetic inputs for the block-FP8 linear layer.

This module draws random tensors and nothing else: it holds none of the
quantisation or GEMM arithmetic. Both the CPU oracle (``oracle/``) and the
HIP library (``block_scaled_fp8_quant_amd``) are fed from here, so they see
identical bytes.

The pages measure on Llama 3.1 8B, Qwen3-8B(-Base) and the Qwen3-30B
mixture-of-experts model with a math dataset (upppp.jp NeMo RL FP8 article,
«重要度サンプリングで精度を保つ», «KVキャッシュとAttentionにも拡張», «まとめ»).
Neither those weights nor that dataset are used: Gaussian tensors at those
models' linear-layer shapes stand in for them.

Every tensor is drawn in fp32 on the CPU from its own ``torch.Generator``
(seeded from the workload, the layer index and a user seed) and rounded to
bf16 with round-to-nearest-even.
"""

from dataclasses import dataclass

import torch

# (name, K, N): Y[M, N] = X[M, K] @ W[N, K]^T
LLAMA31_8B_LINEARS = (
    ("qkv", 4096, 6144),
    ("o_proj", 4096, 4096),
    ("gate_up", 4096, 28672),
    ("down", 14336, 4096),
)
QWEN3_8B_LINEARS = (
    ("qkv", 4096, 6144),
    ("o_proj", 4096, 4096),
    ("gate_up", 4096, 24576),
    ("down", 12288, 4096),
)

# Qwen3-30B-A3B mixture-of-experts block
MOE_TOKENS = 4096
MOE_HIDDEN = 2048
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_FFN = 768          # per-expert intermediate size; gate_up N = 2 * 768
MOE_ZIPF_S = 1.1


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: token count, layer shapes, input statistics."""
    name: str
    m: int
    linears: tuple
    outlier_frac: float
    outlier_scale: float
    pow2: bool


WORKLOADS = {
    # tiny: X [128, 256], W [384, 256], 1% outliers x50
    "tiny": Workload("tiny", 128, (("tiny", 256, 384),), 0.01, 50.0, False),
    # Llama-3.1-8B decode step, 256 tokens, 0.5% outliers x30
    "llama8b_decode": Workload("llama8b_decode", 256, LLAMA31_8B_LINEARS, 0.005, 30.0, False),
    # Llama-3.1-8B prefill/training, 8 sequences x 2048 tokens
    "llama8b_prefill": Workload("llama8b_prefill", 16384, LLAMA31_8B_LINEARS, 0.005, 30.0, False),
    # Qwen3-8B linears with power-of-two scales, 4096 tokens, no outliers
    "qwen8b_pow2": Workload("qwen8b_pow2", 4096, QWEN3_8B_LINEARS, 0.0, 1.0, True),
}

_WORKLOAD_IDS = {"tiny": 0, "llama8b_decode": 1, "llama8b_prefill": 2, "qwen8b_pow2": 3, "moe": 4}


def _gen(workload, part, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) << 16) + (_WORKLOAD_IDS[workload] << 8) + int(part))
    return g


def activation(m, k, gen, outlier_frac=0.0, outlier_scale=1.0):
    """X ~ N(0, 1) [m, k]; each entry independently becomes an outlier
    (multiplied by ``outlier_scale``) with probability ``outlier_frac``."""
    x = torch.randn(m, k, generator=gen, dtype=torch.float32)
    if outlier_frac > 0:
        mask = torch.rand(m, k, generator=gen) < outlier_frac
        x = torch.where(mask, x * outlier_scale, x)
    return x.to(torch.bfloat16)


def weight(n, k, gen, std=0.02):
    """W ~ N(0, std^2) [n, k] in nn.Linear layout."""
    return (torch.randn(n, k, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def linear_inputs(workload, layer, seed=0, m=None):
    """(X [M, K], W [N, K]) bf16 for one linear of a dense workload.

    ``layer`` is an index into the workload's linears or its name. ``m``
    overrides the token count (rows are drawn first, so a smaller ``m``
    is NOT a prefix of the full draw; use row sampling of the full tensor
    when a prefix is needed).
    """
    wl = WORKLOADS[workload]
    if isinstance(layer, str):
        layer = [nm for nm, _, _ in wl.linears].index(layer)
    name, k, n = wl.linears[layer]
    rows = wl.m if m is None else m
    gx = _gen(workload, 2 * layer, seed)
    gw = _gen(workload, 2 * layer + 1, seed)
    x = activation(rows, k, gx, wl.outlier_frac, wl.outlier_scale)
    w = weight(n, k, gw)
    return x, w


def moe_routing(seed=0, tokens=MOE_TOKENS, experts=MOE_EXPERTS, topk=MOE_TOPK, s=MOE_ZIPF_S):
    """Top-k expert choice per token with p_e proportional to (e+1)^-s.

    Each token draws ``topk`` distinct experts. Returns (token_of_row,
    expert_of_row, offsets): the (token, expert) pairs stably sorted by
    expert then token, and int32 offsets[E+1] of each expert's first row.
    """
    g = _gen("moe", 0, seed)
    p = torch.arange(1, experts + 1, dtype=torch.float64) ** (-s)
    p = (p / p.sum()).to(torch.float32)
    choice = torch.multinomial(p.expand(tokens, experts), topk, replacement=False, generator=g)
    tok = torch.arange(tokens).repeat_interleave(topk)
    exp = choice.reshape(-1)
    key = exp * tokens + tok                     # sort by expert, then token
    order = torch.argsort(key, stable=True)
    tok, exp = tok[order], exp[order]
    counts = torch.bincount(exp, minlength=experts)
    offsets = torch.zeros(experts + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return tok, exp, offsets


def moe_inputs(seed=0, which="gate_up", tokens=MOE_TOKENS, hidden=MOE_HIDDEN,
               experts=MOE_EXPERTS, topk=MOE_TOPK, ffn=MOE_FFN):
    """Grouped-GEMM inputs of the MoE block.

    gate_up: X = the token activations [tokens, hidden] gathered in expert
    order -> [tokens*topk, hidden]; W [experts, 2*ffn, hidden].
    down: X [tokens*topk, ffn] drawn directly (the SwiGLU between the two is
    not part of this path); W [experts, hidden, ffn].
    Returns (X, W, offsets int32 [experts+1]).
    """
    tok, _, offsets = moe_routing(seed, tokens, experts, topk)
    if which == "gate_up":
        x_tok = activation(tokens, hidden, _gen("moe", 1, seed))
        x = x_tok[tok]
        w = weight(experts * 2 * ffn, hidden, _gen("moe", 2, seed)).reshape(experts, 2 * ffn, hidden)
    elif which == "down":
        x = activation(tokens * topk, ffn, _gen("moe", 3, seed))
        w = weight(experts * hidden, ffn, _gen("moe", 4, seed)).reshape(experts, hidden, ffn)
    else:
        raise ValueError(which)
    return x, w, offsets


def small_moe_inputs(seed, tokens, hidden, experts, topk, n):
    """A reduced MoE case with the same recipe (for parity at oracle sizes):
    X [tokens*topk, hidden] in expert order, W [experts, n, hidden], offsets."""
    tok, _, offsets = moe_routing(seed, tokens, experts, topk)
    x_tok = activation(tokens, hidden, _gen("moe", 5, seed))
    w = weight(experts * n, hidden, _gen("moe", 6, seed)).reshape(experts, n, hidden)
    return x_tok[tok], w, offsets


def rmsnorm_inputs(m, k, gen, outlier_frac=0.005, outlier_scale=30.0):
    """(x [m, k], gamma [k]) bf16: residual-stream rows ~ N(0, 1) with
    outliers as in ``activation``, and norm weights gamma ~ N(1, 0.25^2)."""
    x = activation(m, k, gen, outlier_frac, outlier_scale)
    gamma = (1.0 + 0.25 * torch.randn(k, generator=gen, dtype=torch.float32)).to(torch.bfloat16)
    return x, gamma


def gate_up_output(m, f, gen, gate_std=2.0, up_std=1.0):
    """gu [m, 2f] bf16, the gate_up linear's output laid out [gate | up]:
    gate ~ N(0, gate_std^2), up ~ N(0, up_std^2)."""
    g = torch.randn(m, f, generator=gen, dtype=torch.float32) * gate_std
    u = torch.randn(m, f, generator=gen, dtype=torch.float32) * up_std
    return torch.cat([g, u], dim=1).to(torch.bfloat16)


def producer_inputs(workload, which, seed=0, m=None):
    """Full-size inputs of one fused producer of a workload:
    ``which`` = "rmsnorm": (x [M, hidden], gamma [hidden]), the RMSNorm in
    front of qkv / gate_up (hidden = the qkv linear's K; for "moe" the
    token rows [MOE_TOKENS, MOE_HIDDEN] before routing);
    ``which`` = "silu_mul": gu [M, 2F], the gate_up output in front of down
    (F = the down linear's K; for "moe" one row per routed (token, expert)
    pair, F = MOE_FFN)."""
    if workload == "moe":
        hidden, f = MOE_HIDDEN, MOE_FFN
        rows_x, rows_gu = MOE_TOKENS, MOE_TOKENS * MOE_TOPK
        frac, scale = 0.0, 1.0
    else:
        wl = WORKLOADS[workload]
        dims = {nm: k for nm, k, _ in wl.linears}
        hidden, f = dims["qkv"], dims["down"]
        rows_x = rows_gu = wl.m
        frac, scale = wl.outlier_frac, wl.outlier_scale
    if m is not None:
        rows_x = rows_gu = m
    if which == "rmsnorm":
        return rmsnorm_inputs(rows_x, hidden, _gen(workload, 0x40, seed), frac, scale)
    if which == "silu_mul":
        return gate_up_output(rows_gu, f, _gen(workload, 0x41, seed))
    raise ValueError(which)


def backward_inputs(workload, layer, seed=0, m=None):
    """(dY [M, N], X [M, K], W [N, K]) bf16 for the backward GEMMs of one
    linear of a dense workload: X and W as in ``linear_inputs``, the output
    gradient dY ~ N(0, 1) * 2^-10 with the workload's outlier recipe."""
    wl = WORKLOADS[workload]
    if isinstance(layer, str):
        layer = [nm for nm, _, _ in wl.linears].index(layer)
    x, w = linear_inputs(workload, layer, seed, m)
    g = _gen(workload, 0x60 + layer, seed)
    dy = activation(x.shape[0], w.shape[0], g, wl.outlier_frac, wl.outlier_scale).float() * 2.0 ** -10
    return dy.to(torch.bfloat16), x, w


# attention heads (query, key/value) and head size of each workload's model
ATTENTION = {
    "llama8b_decode": (32, 8, 128),
    "llama8b_prefill": (32, 8, 128),
    "qwen8b_pow2": (32, 8, 128),
    "moe": (32, 4, 128),              # Qwen3-30B-A3B
}


def kv_inputs(workload, seed=0, t=None):
    """A qkv projection output for the KV-cache path: [T, (Hq + 2*Hkv)*D]
    bf16, each row [Q | K | V], with Q ~ N(0, 1), K ~ N(0, 2^2) and
    V ~ N(0, 0.5^2), and 0.5% of the entries x30 (the workload's outlier
    recipe). T = the workload's token count. Returns (qkv, (Hq, Hkv, D))."""
    hq, hkv, d = ATTENTION[workload]
    rows = (MOE_TOKENS if workload == "moe" else WORKLOADS[workload].m) if t is None else t
    g = _gen(workload, 0x50, seed)
    parts = [torch.randn(rows, hq * d, generator=g, dtype=torch.float32),
             torch.randn(rows, hkv * d, generator=g, dtype=torch.float32) * 2.0,
             torch.randn(rows, hkv * d, generator=g, dtype=torch.float32) * 0.5]
    x = torch.cat(parts, dim=1)
    mask = torch.rand(x.shape, generator=g) < 0.005
    x = torch.where(mask, x * 30.0, x)
    return x.to(torch.bfloat16), (hq, hkv, d)


def attention_inputs(context_lens, hq, hkv, d=128, block_size=16, seed=0, spare_blocks=3):
    """A decode step over a paged KV cache: q [B, Hq, D] ~ N(0, 1) and, for
    every cached token, K ~ N(0, 2^2) and V ~ N(0, 0.5^2) rows [T, Hkv*D]
    (bf16), with the pages of all sequences shuffled over a pool that has
    ``spare_blocks`` unused pages. Returns a dict: q, k, v, slot [T] (the
    cache slot of each token row), block_table [B, max_blocks] int32 (-1
    past a sequence's pages), context_lens [B] int32, num_slots, block_size."""
    g = generator(0xA0, seed)
    lens = [int(n) for n in context_lens]
    b = len(lens)
    blocks = [(n + block_size - 1) // block_size for n in lens]
    max_blocks = max(1, max(blocks))
    pool = sum(blocks) + spare_blocks
    perm = torch.randperm(pool, generator=g)
    table = torch.full((b, max_blocks), -1, dtype=torch.int32)
    slots, used = [], 0
    for i, n in enumerate(lens):
        table[i, :blocks[i]] = perm[used:used + blocks[i]].to(torch.int32)
        used += blocks[i]
        for t in range(n):
            slots.append(int(table[i, t // block_size]) * block_size + t % block_size)
    tot = len(slots)
    q = torch.randn(b, hq, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(tot, hkv * d, generator=g) * 2.0).to(torch.bfloat16)
    v = (torch.randn(tot, hkv * d, generator=g) * 0.5).to(torch.bfloat16)
    return dict(q=q, k=k, v=v, slot=torch.tensor(slots, dtype=torch.int64), block_table=table,
                context_lens=torch.tensor(lens, dtype=torch.int32), num_slots=pool * block_size,
                block_size=block_size)


def prefill_inputs(seqs, hq, hkv, d=128, block_size=16, seed=0, spare_blocks=3):
    """A prefill step over a paged KV cache: ``seqs`` lists (n_new,
    context_len) per sequence (the new tokens are the last n_new of the
    context). q [total_q, Hq, D] ~ N(0, 1) for the new tokens, sequence b's
    rows cu_seqlens_q[b]..; K ~ N(0, 2^2) and V ~ N(0, 0.5^2) rows [T, Hkv*D]
    for every cached token (bf16), pages shuffled over a pool with
    ``spare_blocks`` unused pages. Returns a dict like attention_inputs plus
    cu_seqlens_q [B+1] int32 and max_seqlen_q."""
    g = generator(0xA1, seed)
    news = [int(n) for n, _ in seqs]
    lens = [int(L) for _, L in seqs]
    b = len(lens)
    blocks = [(n + block_size - 1) // block_size for n in lens]
    max_blocks = max(1, max(blocks))
    pool = sum(blocks) + spare_blocks
    perm = torch.randperm(pool, generator=g)
    table = torch.full((b, max_blocks), -1, dtype=torch.int32)
    slots, used = [], 0
    for i, n in enumerate(lens):
        table[i, :blocks[i]] = perm[used:used + blocks[i]].to(torch.int32)
        used += blocks[i]
        for t in range(n):
            slots.append(int(table[i, t // block_size]) * block_size + t % block_size)
    tot = len(slots)
    cu = [0]
    for n in news:
        cu.append(cu[-1] + n)
    q = torch.randn(cu[-1], hq, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(tot, hkv * d, generator=g) * 2.0).to(torch.bfloat16)
    v = (torch.randn(tot, hkv * d, generator=g) * 0.5).to(torch.bfloat16)
    return dict(q=q, k=k, v=v, slot=torch.tensor(slots, dtype=torch.int64), block_table=table,
                context_lens=torch.tensor(lens, dtype=torch.int32), num_slots=pool * block_size,
                block_size=block_size, cu_seqlens_q=torch.tensor(cu, dtype=torch.int32),
                max_seqlen_q=max(news) if news else 0)


def random_cache_codes(shape, seed, device):
    """E4M3 codes drawn on ``device``: magnitude codes 0..126 (finite values)
    with random signs, for caches too large to draw on the host."""
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 16) + 0xB0)
    mag = torch.randint(0, 127, shape, generator=g, device=device, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32) * 128
    return (mag + sign).to(torch.uint8)


def generator(tag, seed=0):
    """A seeded generator for ad-hoc test inputs (``tag`` < 256)."""
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) << 16) + (0xF0 << 8) + int(tag))
    return g
