"""The corrected-reciprocal quotient of the quantisation kernels equals IEEE
fp32 division wherever it decides a code, and their division-free scale
amax/448 equals the IEEE quotient (both exhaustive over bf16, CPU only).

The kernels use the quotient shortcut for scales s >= 2**-90; the same
check with the bound lowered to 2**-126 finds disagreeing codes, which is
why smaller scales take a true division."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "quotient_fastpath_check.c")
SCALE_SRC = os.path.join(HERE, "csrc", "scale_fastpath_check.c")
KV_SRC = os.path.join(HERE, "csrc", "kv_quotient_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("qcheck") / "qcheck")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-march=native", "-o", exe, SRC, "-lm"], check=True)
    return exe


def test_fast_quotient_is_exact_for_both_scale_modes(checker):
    procs = [subprocess.Popen([checker, mode, "-90"], stdout=subprocess.PIPE, text=True)
             for mode in ("0", "1")]
    outs = [p.communicate(timeout=600)[0] for p in procs]
    for p, out in zip(procs, outs):
        assert p.returncode == 0, out
        assert "code_mismatches=0" in out and "bit_mismatches=0" in out


def test_lower_bound_is_needed(checker):
    """With subnormal-range scales allowed, the shortcut does change codes."""
    out = subprocess.run([checker, "0", "-126"], capture_output=True, text=True, timeout=600).stdout
    assert "code_mismatches=0" not in out


def test_division_free_scale_is_exact(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "scheck")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SCALE_SRC, "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout
    assert "checked=32639 mismatches=0" in out.stdout


@pytest.fixture(scope="module")
def kv_checker(tmp_path_factory):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("kvcheck") / "kvcheck")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-march=native", "-o", exe, KV_SRC, "-lm"], check=True)
    return exe


def test_calibrated_scale_quotient_codes_are_exact(kv_checker):
    """The KV-cache write's quotient under arbitrary scales in
    [2^-90, 2^126]: every bf16 magnitude, the linear rule's scales and
    2000 random ones, codes equal to the clamped IEEE quotient's."""
    out = subprocess.run([kv_checker, "2000", "1", "-90"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "code_mismatches=0" in out.stdout


def test_calibrated_scale_lower_bound_is_needed(kv_checker):
    out = subprocess.run([kv_checker, "100", "2", "-126"], capture_output=True, text=True, timeout=300).stdout
    assert "code_mismatches=0" not in out
