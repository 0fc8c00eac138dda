"""Throughput of the block-FP8 W8A8 linear-layer path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
for every linear of the workload, 128x128 weight quantisation (weights
change every optimizer step), 1x128 activation quantisation and the
block-scaled GEMM; the MoE workload runs the expert-grouped GEMM instead.

Prints ONE JSON line (rank 0, N = 1). ``value`` is GEMM FLOPs per step over
the measured step time (quantisation included), in TFLOP/s. ``roofline``
covers the dominant kernel (the GEMM) with its average launch duration
measured by HIP events on the launch stream inside the timed region.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload and checks the timed GPU outputs on those rows against it
(``cpu_baseline.check``: codes and scales bit for bit, GEMM outputs within
the tolerance). ``breakdown`` adds the median/p10/p90 of the per-step and
per-GEMM event times, ``clocks`` the SCLK/MCLK seen during the timed region.
``workloads`` gives the other workloads' lines (Llama-3.1-8B decode M = 256,
Qwen3-8B with power-of-two scales M = 4096, Qwen3-30B-A3B MoE): GEMM times in
the step and with the weights cold in HBM (a 1 GiB write before each
launch), each linear against its roofline, and the quantisers' GB/s. ``producers`` (after the timed region) times the two fused
producer kernels at the workload's shapes -- RMSNorm -> 1x128 quantisation
of the qkv / gate_up input and SiLU(gate)*up -> quantisation of the down
input -- each against the HBM roofline; ``kv_cache`` does the same for the
FP8 KV-cache path (Q/K/V recalibration maxima, quantize-and-write of K and V
into the cache) at the workload's attention shapes; ``backward`` times the
dgrad and wgrad GEMMs of every linear (and their transposing quantizers)
against the same rooflines; ``attention`` times the FP8 decode attention over
the paged FP8 KV cache at the workload's heads for four context mixes,
against the HBM roofline (one call: the split path's two kernels together);
``prefill_attention`` the FP8 prefill attention (8 prompts of 2048 tokens,
causal) against the matrix-core roofline.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

HBM traffic of the GEMM comes from two rocprofv3 counter passes over this
same script (FETCH_SIZE, then WRITE_SIZE), each calibrated by a 1 GiB
device copy run in the same process (--copy-yardstick):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d F -o f -- python bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-yardstick
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d W -o w -- python bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-yardstick
  python bench.py --summarize-traffic F/f_counter_collection.csv W/w_counter_collection.csv
which writes profiles/traffic.json (each kernel's record keyed by a hash of
its sources, so a later change to them turns the reported traffic back into
null).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-FP8 W8A8 GEMM TFLOP/s + % FP8 MFMA peak (Llama-8B shapes)"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# kernels whose counter traffic is recorded (substrings of the kernel names)

def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama8b_prefill",
                   choices=["llama8b_prefill", "llama8b_decode", "qwen8b_pow2", "moe"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-producers", action="store_true", help="skip timing the fused producer kernels")
    p.add_argument("--no-kv", action="store_true", help="skip timing the FP8 KV-cache path")
    p.add_argument("--no-backward", action="store_true", help="skip timing the backward GEMMs")
    p.add_argument("--no-attention", action="store_true", help="skip timing the FP8 decode attention")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other workloads' GEMM and quantisation lines (``workloads``)")
    p.add_argument("--workload-steps", type=int, default=10, help="timed steps per other workload")
    p.add_argument("--cold-reps", type=int, default=7,
                   help="GEMM launches per linear timed after a 1 GiB write (weights cold in HBM)")
    p.add_argument("--backward-reps", type=int, default=3)
    p.add_argument("--producer-reps", type=int, default=20)
    p.add_argument("--cpu-sample-rows", type=int, default=8192)
    p.add_argument("--cpu-sample-wrows", type=int, default=1536)
    p.add_argument("--copy-yardstick", action="store_true",
                   help="after timing, run a 1 GiB device copy (counter calibration)")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc CSVs into profiles/traffic.json and exit")
    p.add_argument("--summarize-trace", metavar="STATS_CSV",
                   help="print a markdown table of a rocprofv3 --stats kernel_stats.csv")
    p.add_argument("--summarize-step-trace", metavar="TRACE_CSV",
                   help="per-layer durations of the step's GEMM launches in a rocprofv3 --kernel-trace "
                        "kernel_trace.csv of a bench run with the same --workload, --warmup and --steps")
    p.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                   help="print a per-kernel markdown summary of rocprofv3 counter_collection.csv files")
    return p.parse_args()


# the sources each recorded kernel is built from (by kernel-name substring,
# first match): a counter record stays valid while these files are unchanged
KERNEL_SOURCES = (("prefill_attention", ("prefill_attention.hip", "quant_common.h", "common.h")),
                  ("attention", ("attention.hip", "quant_common.h", "common.h")),
                  ("kv_", ("kv_cache.hip", "quant_common.h", "common.h")),
                  ("qkv_amax", ("kv_cache.hip", "quant_common.h", "common.h")),
                  ("gemm", ("gemm.hip", "ranges.h", "common.h")),
                  ("rowscaled", ("gemm.hip", "ranges.h", "common.h")),
                  ("splitk", ("gemm.hip", "ranges.h", "common.h")))
QUANT_SOURCES = ("quant.hip", "quant_common.h", "ranges.h", "common.h")


def source_hash(kernel="gemm_kernel"):
    h = hashlib.sha256()
    names = next((srcs for key, srcs in KERNEL_SOURCES if key in kernel), QUANT_SOURCES)
    for name in names:
        with open(os.path.join(ROOT, "block_scaled_fp8_quant_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_layers(workload, dev):
    """Synthetic bf16 inputs resident on the GPU plus preallocated outputs
    (and the split-K workspace of the few-row linears)."""
    import torch
    import synth
    import block_scaled_fp8_quant_amd as fb
    layers = []
    if workload == "moe":
        for which in ("gate_up", "down"):
            x, w, off = synth.moe_inputs(0, which)
            e, n, k = w.shape
            m = x.shape[0]
            layers.append(dict(name="moe_" + which, x=x.to(dev), w=w.to(dev), off=off.to(dev),
                               m=m, n=n, k=k, e=e, pow2=False,
                               qa=torch.empty(m, k, dtype=torch.uint8, device=dev),
                               sa=torch.empty(m, k // 128, dtype=torch.float32, device=dev),
                               qw=torch.empty(e, n, k, dtype=torch.uint8, device=dev),
                               sw=torch.empty(e, n // 128, k // 128, dtype=torch.float32, device=dev),
                               y=torch.empty(m, n, dtype=torch.bfloat16, device=dev),
                               flops=2.0 * m * n * k))
            del x, w
        return layers
    wl = synth.WORKLOADS[workload]
    for li, (name, k, n) in enumerate(wl.linears):
        x, w = synth.linear_inputs(workload, li)
        m = wl.m
        need = fb.fp8blk_gemm_workspace_size(m, n, k)
        layers.append(dict(name=name, x=x.to(dev), w=w.to(dev), m=m, n=n, k=k, e=0, pow2=wl.pow2,
                           ws=torch.empty(need, dtype=torch.uint8, device=dev) if need else None,
                           qa=torch.empty(m, k, dtype=torch.uint8, device=dev),
                           sa=torch.empty(m, k // 128, dtype=torch.float32, device=dev),
                           qw=torch.empty(n, k, dtype=torch.uint8, device=dev),
                           sw=torch.empty(n // 128, k // 128, dtype=torch.float32, device=dev),
                           y=torch.empty(m, n, dtype=torch.bfloat16, device=dev),
                           flops=2.0 * m * n * k))
        del x, w
    return layers


def step(fb, layers, events=None, whole_step=False):
    """One pass of the path. With ``events``, brackets every kernel launch
    with HIP events on the launch stream: events[kind] gets (start, end);
    with ``whole_step`` also the whole pass (events["step"])."""
    import torch
    stream = torch.cuda.current_stream()
    if events is not None and whole_step:
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)

    def timed(kind, fn):
        if events is None:
            fn()
            return
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        events.setdefault(kind, []).append((a, b))

    for L in layers:
        timed("quant_weight", lambda: fb.quant_weight(L["w"], L["pow2"], q=L["qw"], s=L["sw"]))
    for L in layers:
        timed("quant_act", lambda: fb.quant_act(L["x"], L["pow2"], q=L["qa"], s=L["sa"]))
        timed("gemm", lambda: run_gemm(fb, L))
    if events is not None and whole_step:
        s1 = torch.cuda.Event(enable_timing=True)
        s1.record(stream)
        events.setdefault("step", []).append((s0, s1))


def run_gemm(fb, L):
    """The layer's GEMM on its quantised operands (grouped for the MoE
    layers; split-K over the preallocated workspace where the rule splits)."""
    if L["e"]:
        fb.grouped_gemm(L["qa"], L["sa"], L["qw"], L["sw"], L["off"], y=L["y"])
    else:
        fb.gemm(L["qa"], L["sa"], L["qw"], L["sw"], y=L["y"], workspace=L["ws"])


def percentiles(vals):
    """Median, 10th and 90th percentile of a list of times."""
    import numpy as np
    a = np.asarray(vals, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


class ClockSampler:
    """The GPU's shader (SCLK) and memory (MCLK) clocks while the timed
    region runs: the current level of the amdgpu driver's DPM tables
    (sysfs pp_dpm_sclk / pp_dpm_mclk, the line marked '*'), read every 10 ms
    by a background thread (a file read, no GPU call), plus the table's
    levels. Where sysfs is not readable, one ``amd-smi metric --clock``
    reading after the region."""

    def __init__(self):
        import glob
        self.files = {}
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            sc, mc = os.path.join(dev, "pp_dpm_sclk"), os.path.join(dev, "pp_dpm_mclk")
            if os.access(sc, os.R_OK) and os.access(mc, os.R_OK):
                self.files = {"sclk_mhz": sc, "mclk_mhz": mc}
                break
        self.samples = {"sclk_mhz": [], "mclk_mhz": []}
        self._stop = None
        self._thread = None

    @staticmethod
    def _current(path):
        import re
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[mM][hH]z", line)
                        if m:
                            return int(m.group(1))
        except OSError:
            return None
        return None

    @staticmethod
    def _levels(path):
        import re
        try:
            with open(path) as f:
                return [int(m.group(1)) for m in re.finditer(r"(\d+)\s*[mM][hH]z", f.read())]
        except OSError:
            return []

    def _run(self):
        while not self._stop.is_set():
            for key, path in self.files.items():
                v = self._current(path)
                if v is not None:
                    self.samples[key].append(v)
            self._stop.wait(0.01)

    def start(self):
        import threading
        if not self.files:
            return
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        out = {}
        for key, vals in self.samples.items():
            if vals:
                out[key] = {"median": sorted(vals)[len(vals) // 2], "min": min(vals), "max": max(vals),
                            "samples": len(vals)}
        if out:
            for key, path in self.files.items():
                out[key]["levels"] = self._levels(path)
            out["source"] = "sysfs pp_dpm_sclk/pp_dpm_mclk, 10 ms samples over the timed region"
            return out
        return amd_smi_clocks()


def amd_smi_clocks():
    """One reading of amd-smi's clock metrics (text, trimmed), or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    if r.returncode != 0:
        return None
    lines = [ln.strip() for ln in r.stdout.splitlines() if ln.strip()]
    return {"source": "amd-smi metric --clock after the timed region", "text": " | ".join(lines)[:1500]}


RMS_EPS = 1e-5


def build_producers(workload, dev):
    """Full-size inputs of the two fused producers, resident on the GPU,
    with preallocated outputs."""
    import torch
    import synth
    x, gamma = synth.producer_inputs(workload, "rmsnorm")
    gu = synth.producer_inputs(workload, "silu_mul")
    pow2 = False if workload == "moe" else synth.WORKLOADS[workload].pow2
    m, k = x.shape
    mg, f = gu.shape[0], gu.shape[1] // 2
    P = dict(x=x.to(dev), gamma=gamma.to(dev), gu=gu.to(dev), pow2=pow2, m=m, k=k, mg=mg, f=f,
             q1=torch.empty(m, k, dtype=torch.uint8, device=dev),
             s1=torch.empty(m, k // 128, dtype=torch.float32, device=dev),
             q2=torch.empty(mg, f, dtype=torch.uint8, device=dev),
             s2=torch.empty(mg, f // 128, dtype=torch.float32, device=dev))
    del x, gamma, gu
    return P


def time_producers(fb, P, reps):
    """Average launch time of each fused producer (``reps`` launches replayed
    from a HIP graph between two HIP events on the launch stream) against
    the HBM roofline. Algorithmic
    bytes: bf16 input read once, E4M3 codes and fp32 scales written (plus
    gamma for RMSNorm). ``bf16_roundtrip_bytes_saved``: the bytes an unfused
    pipeline moves in addition (the producer's bf16 output written, then
    read back by the quantisation)."""
    m, k, mg, f = P["m"], P["k"], P["mg"], P["f"]
    kernels = (
        ("rmsnorm_quant_act", [m, k],
         lambda: fb.rmsnorm_quant_act(P["x"], P["gamma"], RMS_EPS, P["pow2"], q=P["q1"], s=P["s1"]),
         2 * m * k + 2 * k + m * k + 4 * m * k // 128, 4 * m * k),
        ("silu_mul_quant_act", [mg, 2 * f],
         lambda: fb.silu_mul_quant_act(P["gu"], P["pow2"], q=P["q2"], s=P["s2"]),
         4 * mg * f + mg * f + 4 * mg * f // 128, 4 * mg * f),
    )
    out = {}
    for name, shape, fn, nbytes, saved in kernels:
        # replayed from a HIP graph: at decode sizes a launch from Python
        # takes longer than the kernel, and the events would time that
        out[name] = hbm_entry(shape, graph_time_ms(fn, reps), nbytes)
        out[name]["bf16_roundtrip_bytes_saved"] = saved
    return out


def build_kv(workload, dev):
    """The workload's qkv projection output (one layer) and a paged KV cache
    of 2T slots (pages of 16 tokens, head-major), resident on the GPU, plus
    the scales and a slot permutation."""
    import torch
    import synth
    qkv, (hq, hkv, d) = synth.kv_inputs(workload)
    t = qkv.shape[0]
    dq = qkv.to(dev)
    del qkv
    slot = torch.randperm(2 * t, generator=synth.generator(0x70))[:t].to(dev)
    return dict(qkv=dq, hq=hq, hkv=hkv, d=d, t=t, slot=slot,
                amax=torch.empty(3, dtype=torch.float32, device=dev),
                scale=torch.empty(3, dtype=torch.float32, device=dev),
                kc=torch.zeros(2 * t // ATTN_BLOCK, hkv, ATTN_BLOCK, d, dtype=torch.uint8, device=dev),
                vc=torch.zeros(2 * t // ATTN_BLOCK, hkv, ATTN_BLOCK, d, dtype=torch.uint8, device=dev))


def graph_time_ms(fn, reps, rounds=3):
    """Average time of fn over ``reps`` calls captured in a HIP graph: the
    graph is replayed once to warm up, then ``rounds`` times between pairs of
    HIP events; the median replay, divided by reps (fn run once first,
    outside the graph)."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / reps)
    del graph
    return statistics.median(times)


def hbm_entry(shape, ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"input_shape": shape, "avg_launch_us": round(ms * 1e3, 2), "bound": "hbm",
            "algorithmic_bytes_per_launch": nbytes, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}


def time_kv(fb, K, reps):
    """The FP8 KV-cache path at the workload's attention shapes: the Q/K/V
    recalibration maxima (reset + reduction over the qkv output, read once)
    and the quantize-and-write of every token's K and V rows (bf16 read,
    codes written, slot read)."""
    qkv, hq, hkv, d, t = K["qkv"], K["hq"], K["hkv"], K["d"], K["t"]
    k = qkv[:, hq * d:(hq + hkv) * d]
    v = qkv[:, (hq + hkv) * d:]
    fb.qkv_amax(qkv, hq, hkv, d, amax=K["amax"], reset=True)
    fb.kv_scales(K["amax"], scale=K["scale"])
    ms_amax = graph_time_ms(lambda: fb.qkv_amax(qkv, hq, hkv, d, amax=K["amax"], reset=True), reps)
    ms_write = graph_time_ms(lambda: fb.kv_cache_write(k, v, K["slot"], K["scale"][1:2], K["scale"][2:3],
                                                        K["kc"], K["vc"]), reps)
    w = hkv * d
    out = {"heads": [hq, hkv, d],
           "qkv_amax": hbm_entry([t, (hq + 2 * hkv) * d], ms_amax, 2 * t * (hq + 2 * hkv) * d + 12),
           "kv_cache_write": hbm_entry([t, 2, w], ms_write, 2 * t * w * 2 + 2 * t * w + 8 * t + 8)}
    return out


ATTN_BATCH = 256           # sequences in one decode step
ATTN_BLOCK = 16            # tokens per cache page


def attention_case(workload, dev, lens, seed):
    """One decode step of the workload's attention heads over a paged FP8 KV
    cache holding ``lens`` tokens per sequence (pages shuffled over the pool;
    cache codes random finite E4M3, since the kernel's speed does not depend
    on the values)."""
    import torch
    import synth
    hq, hkv, d = synth.ATTENTION[workload]
    b = len(lens)
    blocks = [(n + ATTN_BLOCK - 1) // ATTN_BLOCK for n in lens]
    mb = max(1, max(blocks))
    g = synth.generator(0x78, seed)
    pool = sum(blocks) + 1
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    table = torch.full((b, mb), -1, dtype=torch.int32)
    used = 0
    for i, nb in enumerate(blocks):
        table[i, :nb] = perm[used:used + nb]
        used += nb
    return dict(q=torch.randn(b, hq, d, generator=g).to(torch.bfloat16).to(dev),
                kc=synth.random_cache_codes((pool, hkv, ATTN_BLOCK, d), 2 * seed + 1, dev),
                vc=synth.random_cache_codes((pool, hkv, ATTN_BLOCK, d), 2 * seed + 2, dev),
                table=table.to(dev), lens=torch.tensor(lens, dtype=torch.int32).to(dev),
                scales=torch.tensor([4.0 / 448, 0.004, 0.01], dtype=torch.float32, device=dev),
                out=torch.empty(b, hq, d, dtype=torch.bfloat16, device=dev),
                heads=(hq, hkv, d), blocks=sum(blocks), tokens=sum(lens))


def time_attention(fb, workload, dev, reps):
    """FP8 decode attention (one query token per sequence over its cached
    tokens) at the workload's heads, four context mixes: 256 sequences of
    2048 tokens, 256 ragged sequences of 1..4096 tokens, 32 sequences of
    16384 tokens, and 4 sequences of 32768 tokens (the library then splits
    the contexts into chunks merged by a second kernel). Algorithmic bytes:
    each cached token's K and V rows of every KV head once (2 Hkv D bytes),
    the block table entries in use, Q read and O written in bf16, lengths and
    scales (the split path's fp32 partials are not counted)."""
    import torch
    import synth
    g = synth.generator(0x79)
    mixes = {"b256_ctx2048": [2048] * ATTN_BATCH,
             "b256_ctx1to4096": torch.randint(1, 4097, (ATTN_BATCH,), generator=g).tolist(),
             "b32_ctx16384": [16384] * 32,
             "b4_ctx32768": [32768] * 4}
    out = {}
    for i, (name, lens) in enumerate(mixes.items()):
        A = attention_case(workload, dev, lens, i)
        hq, hkv, d = A["heads"]
        sc = A["scales"]
        b, mb = len(lens), A["table"].shape[1]
        need = fb.fp8blk_decode_attention_workspace_size(b, hq, hkv, d, mb, ATTN_BLOCK, 0)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        ms = graph_time_ms(lambda: fb.decode_attention(A["q"], A["kc"], A["vc"], A["table"], ATTN_BLOCK, A["lens"],
                                                       sc[0:1], sc[1:2], sc[2:3], out=A["out"], workspace=ws), reps)
        nbytes = 2 * A["tokens"] * hkv * d + 4 * A["blocks"] + 2 * 2 * b * hq * d + 4 * b + 12
        out[name] = hbm_entry([b, hq, hkv, d], ms, nbytes)
        out[name]["split"] = need > 0
        out[name]["tokens"] = A["tokens"]
        del A
        torch.cuda.empty_cache()
    return out


FP16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA


def time_prefill_attention(fb, workload, dev, reps):
    """FP8 prefill attention at the workload's heads: 8 fresh prompts of 2048
    tokens (each new token attends causally over its prompt in the paged FP8
    cache; random finite E4M3 codes, the kernel's speed does not depend on
    them). Timed from HIP-graph replays. Algorithmic work: the causal QK^T
    and PV products, 2 * D * Hq multiply-adds per (query, attended token)
    each; roofline: both on the fp16 matrix cores (2.5 PFLOP/s), where the
    kernel runs them: the E4M3 values are exact in fp16, the probabilities
    stay unquantized, and the FP8 instruction's narrower internal sum would
    make the scores inexact."""
    import torch
    import synth
    hq, hkv, d = synth.ATTENTION[workload]
    nseq, n = 8, 2048
    g = synth.generator(0x7A)
    pages = nseq * n // ATTN_BLOCK
    perm = torch.randperm(pages, generator=g).to(torch.int32)
    table = perm.reshape(nseq, n // ATTN_BLOCK).to(dev)
    kc = synth.random_cache_codes((pages, hkv, ATTN_BLOCK, d), 21, dev)
    vc = synth.random_cache_codes((pages, hkv, ATTN_BLOCK, d), 22, dev)
    q = torch.randn(nseq * n, hq, d, generator=g).to(torch.bfloat16).to(dev)
    cu = torch.arange(0, nseq * n + 1, n, dtype=torch.int32).to(dev)
    lens = torch.full((nseq,), n, dtype=torch.int32).to(dev)
    sc = torch.tensor([4.0 / 448, 0.004, 0.01], dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    ms = graph_time_ms(lambda: fb.prefill_attention(q, cu, n, kc, vc, table, ATTN_BLOCK, lens, sc[0:1], sc[1:2],
                                                     sc[2:3], out=out), reps)
    pairs = nseq * n * (n + 1) // 2                  # (query, attended token) pairs
    f_qk = f_pv = 2.0 * pairs * d * hq
    achieved = (f_qk + f_pv) / (ms * 1e-3) / 1e12
    peak = FP16_PEAK_TFLOPS
    del q, kc, vc, out
    torch.cuda.empty_cache()
    return {"input_shape": [nseq, n, hq, hkv, d], "avg_launch_us": round(ms * 1e3, 2), "bound": "mfma",
            "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None, "flops_per_launch": f_qk + f_pv,
            "peak_note": "QK^T and PV at the fp16 dense MFMA peak (E4M3 operands exact in fp16)"}


def time_backward(fb, workload, dev, reps):
    """The backward GEMMs of each linear of a dense workload at its shapes:
    dgrad dX = dY W (quant_act of dY, quant_weight_t of W, gemm) and wgrad
    dW = dY^T X (quant_act_t of dY and X, gemm_rowscaled). Each kernel is
    timed from HIP-graph replays; the two GEMMs get roofline entries like
    the forward GEMM's (FLOPs per launch averaged over the linears), the
    transposing quantizers HBM entries."""
    import torch
    import synth
    wl = synth.WORKLOADS[workload]
    pow2 = wl.pow2
    sums = {"dgrad": [0.0, 0.0, 0.0], "wgrad": [0.0, 0.0, 0.0], "quant_act_t": [0.0, 0.0], "quant_weight_t": [0.0, 0.0]}
    per_layer = {}
    for li, (name, k, n) in enumerate(wl.linears):
        dy, x, w = synth.backward_inputs(workload, li)
        m = x.shape[0]
        dy, x, w = dy.to(dev), x.to(dev), w.to(dev)
        qa, sa = fb.quant_act(dy, pow2)
        qwt, swt = fb.quant_weight_t(w, pow2)
        dx = torch.empty(m, k, dtype=torch.bfloat16, device=dev)
        qat, sat = fb.quant_act_t(dy, pow2)
        qbt, sbt = fb.quant_act_t(x, pow2)
        dw = torch.empty(n, k, dtype=torch.bfloat16, device=dev)
        need = fb.fp8blk_gemm_workspace_size(m, k, n)  # dX [m, k] contracts over n
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        t_dgrad = graph_time_ms(lambda: fb.gemm(qa, sa, qwt, swt, y=dx, workspace=ws), reps)
        t_wgrad = graph_time_ms(lambda: fb.gemm_rowscaled(qat, sat, qbt, sbt, y=dw), reps)
        t_qat = graph_time_ms(lambda: (fb.quant_act_t(dy, pow2, qt=qat, st=sat),
                                       fb.quant_act_t(x, pow2, qt=qbt, st=sbt)), reps)
        t_qwt = graph_time_ms(lambda: fb.quant_weight_t(w, pow2, qt=qwt, st=swt), reps)
        flops = 2.0 * m * n * k
        sums["dgrad"][0] += t_dgrad
        sums["dgrad"][1] += flops
        sums["dgrad"][2] += m * n + n * k + 4 * m * n // 128 + 4 * n * k // 16384 + 2 * m * k
        sums["wgrad"][0] += t_wgrad
        sums["wgrad"][1] += flops
        sums["wgrad"][2] += n * m + k * m + 4 * (n + k) * m // 128 + 2 * n * k
        sums["quant_act_t"][0] += t_qat
        sums["quant_act_t"][1] += (m * n + m * k) * (3 + 4 / 128)
        sums["quant_weight_t"][0] += t_qwt
        sums["quant_weight_t"][1] += 3 * n * k + 4 * n * k // 16384
        per_layer[name] = {"dgrad_us": round(t_dgrad * 1e3, 1), "wgrad_us": round(t_wgrad * 1e3, 1)}
        del dy, x, w, qa, sa, qwt, swt, dx, qat, sat, qbt, sbt, dw
        torch.cuda.empty_cache()
    L = len(wl.linears)
    out = {}
    for kind in ("dgrad", "wgrad"):
        ms, flops, nbytes = sums[kind]
        out[kind] = roofline(flops / L, nbytes / L, ms / L, None)
        out[kind]["tflops_all_linears"] = round(flops / (ms * 1e-3) / 1e12, 1)
    for kind in ("quant_act_t", "quant_weight_t"):
        ms, nbytes = sums[kind]
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[kind] = {"gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_all_linears": round(ms, 4)}
    out["per_layer"] = per_layer
    return out


def time_backward_moe(fb, dev, reps):
    """The expert-grouped backward GEMMs of the MoE block (gate_up and down,
    rows in expert order): grouped dgrad (quant_act of dY, the per-expert
    transposed weight blocks, the grouped GEMM) and grouped wgrad (the
    grouped transposed quantizer of dY and X on the padded token axis, the
    grouped GEMM with per-row scales). GEMM roofline entries as for the
    dense backward, algorithmic bytes counting the padded operands."""
    import torch
    import synth
    out = {}
    for which in ("gate_up", "down"):
        x, w, off = synth.moe_inputs(0, which)
        m, (e, n, k) = x.shape[0], w.shape
        g = synth.generator(0x61)
        dy = (synth.activation(m, n, g, 0.005, 30.0).float() * 2.0 ** -10).to(torch.bfloat16).to(dev)
        xd, od = x.to(dev), off.to(dev)
        qwt, swt = fb.quant_weight_t(w.to(dev))
        qa, sa = fb.quant_act(dy)
        dx = torch.empty(m, k, dtype=torch.bfloat16, device=dev)
        qat, sat = fb.quant_act_t_grouped(dy, od)
        qbt, sbt = fb.quant_act_t_grouped(xd, od)
        dw = torch.empty(e, n, k, dtype=torch.bfloat16, device=dev)
        t_dgrad = graph_time_ms(lambda: fb.grouped_gemm(qa, sa, qwt, swt, od, y=dx), reps)
        t_wgrad = graph_time_ms(lambda: fb.grouped_gemm_rowscaled(qat, sat, qbt, sbt, od, y=dw), reps)
        t_qat = graph_time_ms(lambda: (fb.quant_act_t_grouped(dy, od, qt=qat, st=sat),
                                       fb.quant_act_t_grouped(xd, od, qt=qbt, st=sbt)), reps)
        flops = 2.0 * m * n * k
        pad = int(sum(((int(off[i + 1]) - int(off[i]) + 127) // 128) * 128 for i in range(e)))
        out[which] = {
            "shape": [m, n, k, e],
            "dgrad": roofline(flops, m * n + e * n * k + 4 * m * n // 128 + 4 * e * n * k // 16384 + 2 * m * k,
                              t_dgrad, None),
            "wgrad": roofline(flops, (n + k) * pad + 4 * (n + k) * pad // 128 + 2 * e * n * k, t_wgrad, None),
            "quant_act_t_grouped_us": round(t_qat * 1e3, 1),
        }
        del x, w, dy, xd, qwt, swt, qa, sa, dx, qat, sat, qbt, sbt, dw
        torch.cuda.empty_cache()
    return out


def gemm_alg_bytes(L):
    """Algorithmic bytes of one GEMM launch: each operand once (codes, scales),
    the bf16 output written."""
    e = max(L["e"], 1)
    return (L["m"] * L["k"] + L["n"] * L["k"] * e + 4 * L["m"] * L["k"] // 128 + 4 * L["n"] * L["k"] * e // 16384
            + 2 * L["m"] * L["n"])


def time_workload(fb, workload, dev, steps, warmup, cold_reps, traffic_db):
    """One of the other workloads at its own shapes: ``steps`` eager passes of
    the path (quant_weight, quant_act, GEMM per linear; HIP events around each
    launch), then each GEMM timed alone ``cold_reps`` times right after a
    1 GiB write (the 256 MB last-level cache then holds none of its weights:
    a decode step's or an MoE layer's weights are read once per step from
    HBM). Below the ridge (decode, MoE) the roofline entry is the cold GEMM
    against the HBM peak; above it (Qwen3-8B, M = 4096) the in-step GEMM
    against the FP8 peak. Medians over the launches."""
    import torch
    stream = torch.cuda.current_stream()
    layers = build_layers(workload, dev)
    for _ in range(warmup):
        step(fb, layers)
    torch.cuda.synchronize()
    events = {}
    for _ in range(steps):
        step(fb, layers, events)
    flush = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros((), dtype=torch.int64, device=dev)
    flushes = {"write": flush.zero_,  # leaves the caches full of dirty lines
               "read": lambda: sink.copy_(flush.view(torch.int64).sum())}  # clean lines
    cold = {(L["name"], kind): [] for L in layers for kind in flushes}
    for _ in range(cold_reps):
        for L in layers:
            for kind, fl in flushes.items():
                fl()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                run_gemm(fb, L)
                b.record(stream)
                cold[(L["name"], kind)].append((a, b))
    torch.cuda.synchronize()
    nl = len(layers)
    ms = {k: [a.elapsed_time(b) for a, b in v] for k, v in events.items()}
    flops = sum(L["flops"] for L in layers)
    alg = sum(gemm_alg_bytes(L) for L in layers)
    per_layer = {}
    hot_total = cold_total = 0.0
    for i, L in enumerate(layers):
        hot = percentiles(ms["gemm"][i::nl])
        cold_pct = {key[1]: percentiles([a.elapsed_time(b) for a, b in v])
                    for key, v in cold.items() if key[0] == L["name"]}
        cl = cold_pct["write"]
        hot_total += hot["median"]
        cold_total += cl["median"]
        ab = gemm_alg_bytes(L)
        roof_us = max(L["flops"] / (FP8_PEAK_TFLOPS * 1e12), ab / (HBM_PEAK_GBS * 1e9)) * 1e6
        per_layer[L["name"]] = {"shape_mnk": [L["m"], L["n"], L["k"]] + ([L["e"]] if L["e"] else []),
                                "gemm_us": round(hot["median"] * 1e3, 1),
                                "gemm_us_p10_p90": [round(hot["p10"] * 1e3, 1), round(hot["p90"] * 1e3, 1)],
                                "gemm_cold_us": round(cl["median"] * 1e3, 1),
                                "gemm_cold_us_p10_p90": [round(cl["p10"] * 1e3, 1), round(cl["p90"] * 1e3, 1)],
                                "gemm_cold_read_flush_us": round(cold_pct["read"]["median"] * 1e3, 1),
                                "roofline_us": round(roof_us, 2),
                                "frac_of_roofline_cold": round(roof_us / (cl["median"] * 1e3), 4)}
    ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    hbm_bound = flops / alg < ridge
    avg_ms = (cold_total if hbm_bound else hot_total) / nl
    rec = (traffic_db or {}).get(workload) or {}
    traffic = rec.get("gemm_bytes_per_launch") if rec.get("source_hash") == source_hash() else None
    kb = kernel_bytes(layers)
    qa_ms = sum(ms["quant_act"]) / steps
    qw_ms = sum(ms["quant_weight"]) / steps
    out = {
        "config": {"workload": workload, "m": layers[0]["m"],
                   "linears": [[L["name"], L["k"], L["n"]] + ([L["e"]] if L["e"] else []) for L in layers],
                   "pow2": layers[0]["pow2"]},
        "gemm_tflops_in_step": round(flops / (hot_total * 1e-3) / 1e12, 1),
        "gemm_tflops_cold": round(flops / (cold_total * 1e-3) / 1e12, 1),
        "roofline": roofline(flops / nl, alg / nl, avg_ms, traffic),
        "timing": "cold (1 GiB written before each launch)" if hbm_bound else "in step (eager)",
        "cold_note": ("gemm_cold_us: a 1 GiB write before each launch (the last-level cache then holds "
                      "dirty lines, written back while the weights stream in); gemm_cold_read_flush_us: a "
                      "1 GiB read instead (clean lines); HIP events, launch overhead included"),
        "per_layer": per_layer,
        "quant_act": {"gbs": round(kb["quant_act"] / (qa_ms * 1e-3) / 1e9, 1),
                      "frac": round(kb["quant_act"] / (qa_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "ms_per_step": round(qa_ms, 4)},
        "quant_weight": {"gbs": round(kb["quant_weight"] / (qw_ms * 1e-3) / 1e9, 1),
                         "frac": round(kb["quant_weight"] / (qw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "ms_per_step": round(qw_ms, 4)},
        "layer_rate_tflops": round(flops / ((hot_total + qa_ms) * 1e-3) / 1e12, 1),
    }
    for L in layers:
        L.clear()
    del layers, flush
    torch.cuda.empty_cache()
    return out


def snapshot_sample(layers, workload, rows, wrows):
    """Host copies of the timed outputs on the rows the CPU baseline samples
    (the first ``rows`` activation rows and ``wrows`` weight rows of each
    linear; for the MoE layers, rows of the largest expert and its weights)."""
    out = []
    for L in layers:
        if L["e"]:
            offs = L["off"].cpu().numpy()
            import numpy as np
            e = int(np.argmax(np.diff(offs)))
            lo, hi = int(offs[e]), int(offs[e + 1])
            r0, r1 = lo, min(lo + rows, L["m"])
            qw, sw = L["qw"][e], L["sw"][e]
            yrows = min(r1, hi) - r0
        else:
            r0, r1 = 0, min(rows, L["m"])
            qw, sw = L["qw"], L["sw"]
            yrows = r1 - r0
        out.append({"qa": L["qa"][r0:r1].cpu().numpy(), "sa": L["sa"][r0:r1].cpu().numpy(),
                    "qw": qw[:wrows].cpu().numpy(), "sw": sw[:wrows // 128].cpu().numpy(),
                    "y": L["y"][r0:r0 + yrows, :wrows].float().cpu().numpy(), "yrows": yrows})
    return out


def kernel_bytes(layers):
    """Algorithmic HBM bytes per launch kind, summed over one step."""
    qa = sum(2 * L["m"] * L["k"] + L["m"] * L["k"] + 4 * L["m"] * L["k"] // 128 for L in layers)
    rows_w = [L["n"] * L["k"] * max(L["e"], 1) for L in layers]
    qw = sum(3 * r + 4 * r // 16384 for r in rows_w)
    return {"quant_act": qa, "quant_weight": qw}


def cpu_baseline(workload, rows, wrows, gpu_sample=None):
    """The oracle (untuned) on a bounded sample: for each linear, ``rows``
    activation rows and ``wrows`` weight rows are quantised and multiplied.
    Inputs are drawn first (untimed, like the GPU's resident inputs); the
    timed part is oracle work only. Scaled to TFLOP/s of GEMM work like the
    GPU value. With ``gpu_sample`` (the timed GPU outputs on the same rows,
    snapshot_sample), the oracle's results also check them: codes and scales
    bit for bit, the GEMM outputs within |y - y_ref| <= 2^-7 |y_ref| +
    1e-3 rms(y_ref)."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    cases = []
    if workload == "moe":
        for which in ("gate_up", "down"):
            x, w, off = synth.moe_inputs(0, which)
            offs = off.numpy()
            e = int(np.argmax(np.diff(offs)))
            lo = int(offs[e])
            cases.append((x[lo:lo + rows].clone(), w[e][:wrows].clone(), False))
            del x, w
        desc = "%d routed rows of the largest expert x %d weight rows, gate_up and down" % (rows, wrows)
    else:
        wl = synth.WORKLOADS[workload]
        for li in range(len(wl.linears)):
            x, w = synth.linear_inputs(workload, li)
            cases.append((x[:rows].clone(), w[:wrows].clone(), wl.pow2))
            del x, w
        desc = ("first %d activation rows x first %d weight rows of each of the %d linears: "
                "oracle quantisation (numpy) + block-wise fp64 GEMM" % (rows, wrows, len(wl.linears)))
    flops = 0.0
    results = []
    t0 = time.perf_counter()
    for xs, ws, pow2 in cases:
        qa, sa = oracle.quant_act_ref(xs, pow2)
        qw, sw = oracle.quant_weight_ref(ws, pow2)
        y = oracle.gemm_ref(qa, sa, qw, sw)
        flops += 2.0 * xs.shape[0] * ws.shape[0] * xs.shape[1]
        results.append((qa, sa, qw, sw, y))
    dt = time.perf_counter() - t0
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": desc, "seconds": round(dt, 2)}
    if gpu_sample is not None:
        out["check"] = check_sample(results, gpu_sample)
    return out


def check_sample(results, gpu_sample):
    """Compare the timed GPU outputs with the oracle's on the sampled rows."""
    import numpy as np
    import oracle
    codes_bad = scales_bad = 0
    worst = 0.0
    ok = True
    for (qa, sa, qw, sw, y), g in zip(results, gpu_sample):
        codes_bad += int(np.count_nonzero(g["qa"] != qa) + np.count_nonzero(g["qw"] != qw))
        scales_bad += int(np.count_nonzero(g["sa"].view(np.uint32) != sa.view(np.uint32))
                          + np.count_nonzero(g["sw"].view(np.uint32) != sw.view(np.uint32)))
        if g["yrows"] > 0:
            good, w = oracle.tolerance_ok(g["y"].astype(np.float64), y[:g["yrows"]])
            ok = ok and good
            worst = max(worst, float(w))
    return {"codes_mismatched": codes_bad, "scales_mismatched": scales_bad, "gemm_within_tolerance": bool(ok),
            "gemm_worst_ratio": round(worst, 4),
            "ok": bool(ok and codes_bad == 0 and scales_bad == 0)}


COPY_BYTES = 1 << 30


def roofline(flops, alg_bytes, avg_ms, traffic):
    """The GEMM's roofline entry: MFMA-bound when its arithmetic intensity
    (flops per algorithmic byte) is above the FP8 ridge (peak flops / peak
    HBM bandwidth, 625 flop/B), else HBM-bound (achieved = algorithmic bytes
    per launch / average launch time)."""
    ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    intensity = flops / alg_bytes
    sec = avg_ms * 1e-3
    if intensity >= ridge:
        bound, achieved, peak, unit = "mfma", flops / sec / 1e12, FP8_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", alg_bytes / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": round(alg_bytes), "flops_per_launch": flops,
            "intensity_flop_per_byte": round(intensity, 1), "avg_launch_ms": round(avg_ms, 4)}


def copy_yardstick():
    """A plain 1 GiB device-to-device copy: the counters' calibration."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


# GEMM-family kernels: a GEMM call is one dispatch of a primary kernel (the
# split-K path adds its reduction to the same call)
GEMM_PRIMARY = ("gemm_kernel<", "gemm_persistent_kernel<", "gemm_splitk_kernel", "grouped_gemm_kernel",
                "grouped_gemm_persistent_kernel")
GEMM_FAMILY = GEMM_PRIMARY + ("splitk_reduce_kernel",)


def summarize_traffic(fetch_csv, write_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel of a
    counter pass, scaled by what the same counters read for the 1 GiB copy
    into bytes; the GEMM's bytes per call are the GEMM family's bytes over
    the number of GEMM calls."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_f = [v for n, v in fetch.items() if "copyBuffer" in n]
    copy_w = [v for n, v in write.items() if "copyBuffer" in n]
    c_f, c_w = max(copy_f[0]), max(copy_w[0])
    f_scale = COPY_BYTES / (c_f * 1024.0)
    w_scale = COPY_BYTES / (c_w * 1024.0)
    kernels = {}
    gemm_bytes, gemm_calls = 0.0, 0
    for name in fetch:
        if name not in write or "copyBuffer" in name or name.startswith("void at::") or "at::native" in name:
            continue
        key = short_kernel_name(name)
        kf, kw = fetch[name], write[name]
        src = key.split("<")[0]
        b = statistics.mean(kf) * 1024 * f_scale + statistics.mean(kw) * 1024 * w_scale
        kernels[key] = {"source_hash": source_hash(src), "fetch_kib_per_dispatch": statistics.mean(kf),
                        "write_kib_per_dispatch": statistics.mean(kw), "dispatches": len(kf),
                        "bytes_per_launch": b}
        if any(k in key for k in GEMM_FAMILY):
            gemm_bytes += b * len(kf)
            if any(k in key for k in GEMM_PRIMARY):
                gemm_calls += len(kf)
    # records read by the bench: the GEMM call and the kernels it names
    # without template arguments
    for base in ("quant_act_kernel", "quant_weight_kernel", "rmsnorm_quant_act_rows_kernel",
                 "silu_mul_quant_act_kernel", "qkv_amax_kernel", "kv_cache_write_kernel",
                 "decode_attention_combine_kernel"):
        recs = [v for k, v in kernels.items() if k.split("<")[0] == base]
        if recs and base not in kernels:
            n = sum(r["dispatches"] for r in recs)
            kernels[base] = {"source_hash": recs[0]["source_hash"], "dispatches": n,
                             "bytes_per_launch": sum(r["bytes_per_launch"] * r["dispatches"] for r in recs) / n,
                             "note": "mean over its instantiations"}
    rec = {
        "source_hash": source_hash(),
        "gemm_calls": gemm_calls,
        "copy_fetch_kib": c_f, "copy_write_kib": c_w, "copy_bytes": COPY_BYTES,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "gemm_bytes_per_launch": gemm_bytes / gemm_calls if gemm_calls else None,
        "kernels": kernels,
    }
    return rec


def short_kernel_name(name):
    """A kernel name without its namespace, return type and argument list,
    template arguments kept (tile configurations tell the GEMMs apart)."""
    name = name.replace("void ", "").replace("fp8blk::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


# CUs and SIMDs of the MI355X; GRBM_GUI_ACTIVE counts GPU-busy cycles once per
# XCD, so cycles = GRBM_GUI_ACTIVE / 8.
N_XCD, N_CU, N_SIMD = 8, 256, 4


def summarize_counters(paths):
    """Markdown summary of rocprofv3 counter passes: per kernel and grid size,
    the mean per dispatch of every counter collected, the mean duration, and
    the ratios derived from them where their inputs were collected:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * CUs * SIMDs);
    MFMA FP8 FLOPs = SQ_INSTS_VALU_MFMA_MOPS_F8 * 512 and their rate;
    clock = cycles / duration; LDS-wait share = SQ_WAIT_INST_LDS /
    SQ_WAVE_CYCLES; bank-conflict cycles per LDS instruction; TA busy =
    TA_BUSY_avr / cycles; TA stalled by TCP = TA_ADDR_STALLED_BY_TC_CYCLES_sum
    / (cycles * CUs); L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)."""
    import csv
    import statistics
    groups = {}   # (kernel, grid) -> {dispatch key -> {counter: value, "_ns": duration}}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                d = groups.setdefault(key, {}).setdefault((path, r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
                if r.get("End_Timestamp") and r.get("Start_Timestamp"):
                    d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = []
    for (kernel, grid), disp in sorted(groups.items(), key=lambda kv: -sum(d.get("_ns", 0) for d in kv[1].values())):
        counters = sorted({c for d in disp.values() for c in d if c != "_ns"})
        mean = {c: statistics.mean(d[c] for d in disp.values() if c in d) for c in counters}
        ns = [d["_ns"] for d in disp.values() if "_ns" in d]
        dur = statistics.mean(ns) if ns else None
        row = ["`%s`" % kernel, str(grid // 64 if grid % 64 == 0 else grid), str(len(disp)),
               "%.1f" % (dur / 1e3) if dur else "-"]
        derived = []
        cycles = mean.get("GRBM_GUI_ACTIVE", 0) / N_XCD
        if cycles and dur:
            # the GUI-active window also covers the dispatch's set-up and
            # drain: for short kernels it is longer than the kernel itself
            ghz = cycles / dur
            derived.append("clock %.2f GHz" % ghz if ghz <= 2.5 else "GUI window %.1fx the kernel" % (ghz / 2.4))
        if cycles and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            derived.append("MFMA busy %.1f%%" % (100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_CU * N_SIMD)))
        if mean.get("SQ_INSTS_VALU_MFMA_MOPS_F8"):
            fl = mean["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
            derived.append("FP8 MFMA %.3g GFLOP" % (fl / 1e9) + (" = %.0f TFLOP/s" % (fl / dur / 1e3) if dur else ""))
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"):
            if mean.get("SQ_WAVE_CYCLES") and c in mean:
                derived.append("%s %.1f%%" % (c, 100 * mean[c] / mean["SQ_WAVE_CYCLES"]))
        if mean.get("SQ_WAVE_CYCLES") and mean.get("SQ_WAIT_INST_LDS"):
            derived.append("LDS wait %.1f%% of wave cycles" % (100 * mean["SQ_WAIT_INST_LDS"] / mean["SQ_WAVE_CYCLES"]))
        if mean.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 1):
            derived.append("%.2f conflict cycles per LDS instruction"
                           % (mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_INSTS_LDS"]))
        if cycles and "TA_BUSY_avr" in mean:
            derived.append("TA busy %.1f%%" % (100 * mean["TA_BUSY_avr"] / cycles))
        if cycles and "TA_ADDR_STALLED_BY_TC_CYCLES_sum" in mean:
            derived.append("TA stalled by TCP %.1f%%" % (100 * mean["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / (cycles * N_CU)))
        if mean.get("TCC_HIT_sum", 0) + mean.get("TCC_MISS_sum", 0) > 0:
            derived.append("L2 hit %.1f%%" % (100 * mean["TCC_HIT_sum"] / (mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"])))
        row.append("; ".join(derived) or "-")
        row.append(", ".join("%s %.4g" % (c, v) for c, v in mean.items()))
        lines.append("| " + " | ".join(row) + " |")
    head = ["| kernel | workgroups | dispatches | mean us | derived | counters (mean per dispatch) |",
            "|---|---|---|---|---|---|"]
    return "\n".join(head + lines)


def summarize_trace(stats_csv):
    """Markdown table of a rocprofv3 kernel_stats.csv: one row per kernel
    (template arguments kept; torch's own kernels folded into one row)."""
    import csv
    agg = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            key = "torch kernels (fills, copies, random numbers)" if "at::native" in name else \
                "`%s`" % short_kernel_name(name)
            a = agg.setdefault(key, {"calls": 0, "tot": 0.0, "min": float("inf"), "max": 0.0})
            a["calls"] += int(r["Calls"])
            a["tot"] += float(r["TotalDurationNs"])
            a["min"] = min(a["min"], float(r["MinNs"]))
            a["max"] = max(a["max"], float(r["MaxNs"]))
    total = sum(a["tot"] for a in agg.values())
    out = ["| kernel | calls | total ms | avg us | min us | max us | share % |", "|---|---|---|---|---|---|---|"]
    for k, a in sorted(agg.items(), key=lambda kv: -kv[1]["tot"]):
        out.append("| %s | %d | %.3f | %.1f | %.1f | %.1f | %.2f |" % (
            k, a["calls"], a["tot"] / 1e6, a["tot"] / a["calls"] / 1e3, a["min"] / 1e3, a["max"] / 1e3,
            100 * a["tot"] / total))
    return "\n".join(out)


def step_layer_names(workload):
    """The names of a workload's step layers, in launch order."""
    import synth
    if workload == "moe":
        return ["moe_gate_up", "moe_down"]
    return [nm for nm, _, _ in synth.WORKLOADS[workload].linears]


def summarize_step_trace(trace_csv, workload, warmup, steps):
    """The step's GEMM launches in a rocprofv3 kernel_trace.csv of a bench run
    (same workload, warm-up and step counts): the dispatches are taken in
    start order, a layer's GEMM launch being the GEMM-family dispatches
    (dense, persistent, grouped, split-K and its reduction) that follow its
    quant_act dispatch. Reports each layer's mean over the timed steps and
    the mean per launch, the figure the bench's roofline.avg_launch_ms gives
    from HIP events around the same launches."""
    import csv
    names = step_layer_names(workload)
    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    launches, cur = [], None
    want = (warmup + steps) * len(names)
    for r in rows:
        nm = r["Kernel_Name"]
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if "gemm" in nm or "splitk_reduce" in nm:
            if cur is not None:
                cur += dur
            continue
        if cur is not None:
            launches.append(cur)
            cur = None
            if len(launches) == want:
                break
        if "::quant_act_kernel(" in nm:
            cur = 0
    if cur is not None and len(launches) < want:
        launches.append(cur)
    if len(launches) < want:
        raise SystemExit("found %d GEMM launches, expected %d" % (len(launches), want))
    timed = launches[warmup * len(names):want]
    per_layer = {nm: sum(timed[i::len(names)]) / steps / 1e3 for i, nm in enumerate(names)}
    mean = sum(timed) / len(timed) / 1e3
    return ("Step GEMM launches in the per-dispatch trace (the %d timed steps; a launch is the GEMM-family "
            "dispatches after its layer's quant_act, a split-K launch with its reduction): %s us; mean per "
            "launch %.1f us." % (steps, ", ".join("%s %.1f" % kv for kv in per_layer.items()), mean))


def main():
    args = parse()
    if args.summarize_step_trace:
        print(summarize_step_trace(args.summarize_step_trace, args.workload, args.warmup, args.steps))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_traffic:
        rec = summarize_traffic(*args.summarize_traffic)
        db = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                db = json.load(f)
        db[args.workload] = rec
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path is single-GPU only (no collectives); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp8_quant_amd as fb
    fb.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    layers = build_layers(args.workload, dev)
    flops_step = sum(L["flops"] for L in layers)
    print("bench: workload %s, %d layers, %.1f GFLOP/step" % (args.workload, len(layers), flops_step / 1e9),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(fb, layers)
    torch.cuda.synchronize()

    events = {}
    clocks = ClockSampler()
    torch.cuda.synchronize()
    clocks.start()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(fb, layers, events, whole_step=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock_rec = clocks.stop()
    ms_step = (t1 - t0) * 1e3 / args.steps

    if args.copy_yardstick:
        copy_yardstick()
    per_kind = {k: [a.elapsed_time(b) for a, b in v] for k, v in events.items()}
    gemm_ms = sum(per_kind["gemm"]) / args.steps           # GEMM time per step
    gemm_avg_ms = sum(per_kind["gemm"]) / len(per_kind["gemm"])
    gemm_flops_launch = flops_step / len(layers)
    achieved = gemm_flops_launch / (gemm_avg_ms * 1e-3) / 1e12
    traffic, traffic_rec = None, {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(args.workload)
        if rec and rec.get("source_hash") == source_hash():
            traffic = rec.get("gemm_bytes_per_launch")
        if rec:
            traffic_rec = {k: v for k, v in rec.get("kernels", {}).items()
                           if v.get("source_hash") == source_hash(k)}
    kb = kernel_bytes(layers)
    alg_bytes_launch = sum(gemm_alg_bytes(L) for L in layers) / len(layers)
    breakdown = {
        "gemm_ms_per_step": round(gemm_ms, 4),
        "gemm_tflops": round(flops_step / (gemm_ms * 1e-3) / 1e12, 1),
        "quant_act_ms_per_step": round(sum(per_kind["quant_act"]) / args.steps, 4),
        "quant_act_gbs": round(kb["quant_act"] / (sum(per_kind["quant_act"]) / args.steps * 1e-3) / 1e9, 1),
        "quant_weight_ms_per_step": round(sum(per_kind["quant_weight"]) / args.steps, 4),
        "quant_weight_gbs": round(kb["quant_weight"] / (sum(per_kind["quant_weight"]) / args.steps * 1e-3) / 1e9, 1),
        "per_layer_gemm_us": {L["name"]: round(sum(per_kind["gemm"][i::len(layers)]) / args.steps * 1e3, 1)
                              for i, L in enumerate(layers)},
    }
    step_ms = percentiles(per_kind["step"])
    gemm_pct = {L["name"]: percentiles(per_kind["gemm"][i::len(layers)]) for i, L in enumerate(layers)}
    breakdown["step_ms_events"] = step_ms
    breakdown["per_layer_gemm_us_p10_p90"] = {k: [round(v["p10"] * 1e3, 1), round(v["p90"] * 1e3, 1)]
                                               for k, v in gemm_pct.items()}
    value = flops_step / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "m": layers[0]["m"],
                   "linears": [[L["name"], L["k"], L["n"]] for L in layers],
                   "pow2": layers[0]["pow2"],
                   "step": "quant_weight x%d + quant_act x%d + %s x%d" % (
                       len(layers), len(layers), "grouped_gemm" if layers[0]["e"] else "gemm", len(layers))},
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "roofline": roofline(gemm_flops_launch, alg_bytes_launch, gemm_avg_ms, traffic),
        "breakdown": breakdown,
        "clocks": clock_rec,
    }
    sample = None if args.no_cpu_baseline else snapshot_sample(layers, args.workload, args.cpu_sample_rows,
                                                               args.cpu_sample_wrows)
    for L in layers:                          # free the step's buffers
        L.clear()
    torch.cuda.empty_cache()
    if not args.no_workloads:
        traffic_db = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                traffic_db = json.load(f)
        out["workloads"] = {}
        for name in ("llama8b_decode", "qwen8b_pow2", "moe"):
            if name == args.workload:
                continue
            print("bench: workload %s" % name, file=sys.stderr, flush=True)
            out["workloads"][name] = time_workload(fb, name, dev, args.workload_steps, 3, args.cold_reps,
                                                   traffic_db)
    if not args.no_producers:
        print("bench: timing the fused producers", file=sys.stderr, flush=True)
        out["producers"] = time_producers(fb, build_producers(args.workload, dev), args.producer_reps)
        for name, key in (("rmsnorm_quant_act", "rmsnorm_quant_act_rows_kernel"),
                          ("silu_mul_quant_act", "silu_mul_quant_act_kernel")):
            t = traffic_rec.get(key, {}).get("bytes_per_launch")
            out["producers"][name]["traffic"] = None if t is None else round(t)
    if not args.no_backward:
        print("bench: timing the backward GEMMs", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        if args.workload == "moe":
            out["backward"] = time_backward_moe(fb, dev, args.backward_reps)
        else:
            out["backward"] = time_backward(fb, args.workload, dev, args.backward_reps)
    if not args.no_kv:
        print("bench: timing the FP8 KV-cache path", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        out["kv_cache"] = time_kv(fb, build_kv(args.workload, dev), args.producer_reps)
        for name, key in (("qkv_amax", "qkv_amax_kernel"), ("kv_cache_write", "kv_cache_write_kernel")):
            t = traffic_rec.get(key, {}).get("bytes_per_launch")
            out["kv_cache"][name]["traffic"] = None if t is None else round(t)
    if not args.no_attention:
        print("bench: timing the FP8 decode attention", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        out["attention"] = time_attention(fb, args.workload, dev, args.producer_reps)
        import synth
        g = synth.ATTENTION[args.workload][0] // synth.ATTENTION[args.workload][1]
        direct = traffic_rec.get("decode_attention_kernel<%d, false>" % g, {}).get("bytes_per_launch")
        part = traffic_rec.get("decode_attention_kernel<%d, true>" % g, {}).get("bytes_per_launch")
        merge = traffic_rec.get("decode_attention_combine_kernel", {}).get("bytes_per_launch")
        for entry in out["attention"].values():
            # counters are kept per kernel, averaged over the mixes that ran it:
            # the three direct-path mixes move the same algorithmic bytes within 0.4%
            t = (part + merge if part is not None and merge is not None else None) if entry["split"] else direct
            entry["traffic"] = None if t is None else round(t)
    if not args.no_attention:
        print("bench: timing the FP8 prefill attention", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        out["prefill_attention"] = time_prefill_attention(fb, args.workload, dev, 5)
        import synth
        g = synth.ATTENTION[args.workload][0] // synth.ATTENTION[args.workload][1]
        t = traffic_rec.get("prefill_attention_kernel<%d>" % g, {}).get("bytes_per_launch")
        out["prefill_attention"]["traffic"] = None if t is None else round(t)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_sample_rows, args.cpu_sample_wrows, sample)
        if not out["cpu_baseline"]["check"]["ok"]:
            print("bench: the timed outputs DIFFER from the oracle on the sample: %s"
                  % out["cpu_baseline"]["check"], file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
