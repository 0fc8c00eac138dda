"""Build libfp8blk.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m block_scaled_fp8_quant_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8blk.so")
# race-detection variant: the kernels that stage operands through LDS, with
# an extra barrier at every stage transition (same C ABI for those calls)
DEBUG_LIB = os.path.join(PKG, "libfp8blk_debug_barriers.so")
DEBUG_SOURCES = ("gemm.hip", "prefill_attention.hip", "attention.hip")
DEBUG_FLAGS = ["-DFP8BLK_DEBUG_BARRIERS=1"]

SOURCES = ("quant.hip", "gemm.hip", "kv_cache.hip", "attention.hip", "prefill_attention.hip")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the GEMM folds every partial with VALU FMAs,
    # which cannot read accumulation registers directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI
# layer (argument checks, launch set-up); each -fsanitize= applies to the
# host compilation only, the device code is built as usual.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _start(out, extra, sources, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I" + INCLUDE, "-I" + CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), tmp, out


def _finish(job, verbose):
    proc, tmp, out = job
    text, _ = proc.communicate()
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in text.splitlines() if noise not in ln]
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose=False, out=LIB, extra=(), sources=SOURCES, debug_variant=None):
    """Compile ``sources`` into ``out`` (atomically replaced; the in-tree
    library by default), with ``extra`` flags. Always rebuilds. The default
    call also builds the race-detection variant DEBUG_LIB, concurrently."""
    if debug_variant is None:
        debug_variant = out == LIB and not extra
    jobs = [_start(out, extra, sources, verbose)]
    if debug_variant:
        jobs.append(_start(DEBUG_LIB, DEBUG_FLAGS, DEBUG_SOURCES, verbose))
    done = [_finish(job, verbose) for job in jobs]
    return done[0]


def sanitizer_runtime():
    """The AddressSanitizer runtime to preload into a process that loads the
    host-sanitized library (the interpreter itself is not instrumented)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, shutil.which("clang"), "/opt/rocm/llvm/bin/clang"):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                               text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("AddressSanitizer runtime not found")


def build_host_sanitized(out, verbose=False):
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on
    its host code (for CPU tests of the C ABI; not for GPU runs)."""
    return build(verbose, out=out, extra=HOST_SANITIZE_FLAGS + ["-O1", "-g"], debug_variant=False)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
