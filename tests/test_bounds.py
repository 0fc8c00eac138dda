"""CPU checks of the GEMM kernels' bounds arithmetic (no GPU).

1. ``ranges.h`` (buffer-resource lengths, expert row ranges read from device
   offsets) compiled unchanged with g++ and exercised over edge cases and a
   host model of the grouped launch, valid and broken offsets
   (tests/csrc/ranges_check.cpp).
2. A model of the 256x256 tile's direct loads: each lane's VGPR offset, the
   scalar offset and the resource's base and length, as the tile sets them
   up, checked against the buffer range rule (a load is fetched only when
   its VGPR offset is below the resource length; the scalar offset is not
   range-checked). Every fetched byte must lie inside the operand and every
   row of the operand that the tile covers must be fetched. The same model
   with the tile's second half addressed through the scalar offset (the
   layout the resources replaced) fetches rows past the operand's end, so
   the check can tell the two apart.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_scaled_fp8_quant_amd", "csrc")


def test_ranges_header_on_cpu(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = str(tmp_path / "ranges_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-Werror", "-I" + CSRC, "-o", exe,
                    os.path.join(HERE, "csrc", "ranges_check.cpp")], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr


# --- model of the 256x256 tile's direct loads (8 waves, 4 x 1 KB windows of
# A and of B per wave; waves 0-3 also load waves 4-7's windows) ---
BK = 128
BM = BN = 256
WAVES = 8
WIN = BM // 8 // WAVES          # 1 KB windows per wave per operand (4)
HALF_ROWS = WAVES // 2 * WIN * 8  # rows between a wave's windows and its partner's (128)


def swz_key(row):
    return (row >> 1) & 7


def lane_offsets(wave, ld):
    """VGPR offsets of one wave's window loads: (row in the tile, offset)."""
    out = []
    for i in range(WIN):
        for lane in range(64):
            row = (wave * WIN + i) * 8 + (lane >> 3)
            out.append((row, row * ld + (((lane & 7) ^ swz_key(row)) << 4)))
    return out


def clamp_len(n):
    return 0 if n <= 0 else min(n, 0xFFFFFFFF)


def fetched(rows_total, ld, t0, kb0, kb, scalar_pair):
    """Operand rows the loading waves fetch for K block kb of a tile starting
    at row t0: a set of (operand row, byte offset within the row)."""
    got = set()
    base = t0 * ld + kb0 * BK
    length = clamp_len((rows_total - t0) * ld - kb0 * BK)
    base2 = (t0 + HALF_ROWS) * ld + kb0 * BK
    length2 = clamp_len((rows_total - t0 - HALF_ROWS) * ld - kb0 * BK)
    koff = kb * BK
    for wave in range(WAVES // 2):
        for row, v in lane_offsets(wave, ld):
            plans = [(base, length, v, koff, row)]
            if scalar_pair:   # partner rows through the scalar offset, first half's resource
                plans.append((base, length, v, koff + HALF_ROWS * ld, row + HALF_ROWS))
            else:             # partner rows through their own resource
                plans.append((base2, length2, v, koff, row + HALF_ROWS))
            for b, n, voff, soff, tile_row in plans:
                if voff + 16 <= n:            # range rule: the VGPR offset only
                    addr = b + soff + voff
                    got.add((addr // ld, addr % ld, t0 + tile_row))
    return got


@pytest.mark.parametrize("rows_total,t0", [(256, 0), (257, 256), (300, 256), (384, 256), (456, 256),
                                           (512, 256), (100, 0), (128, 0), (129, 0), (200, 0), (1, 0)])
@pytest.mark.parametrize("kb0,kbn", [(0, 2), (3, 2)])
def test_paired_loads_stay_inside_the_operand(rows_total, t0, kb0, kbn):
    ld = (kb0 + kbn) * BK
    for kb in range(kbn):
        got = fetched(rows_total, ld, t0, kb0, kb, scalar_pair=False)
        for row, col, tile_row in got:
            assert row < rows_total, "fetched row %d of %d" % (row, rows_total)
            assert row == tile_row, "fetched a row other than the lane's"
            assert kb0 * BK + kb * BK <= col < kb0 * BK + (kb + 1) * BK
        want = {(r, kb0 * BK + kb * BK + c * 16) for r in range(t0, min(rows_total, t0 + BM)) for c in range(8)}
        assert {(r, c) for r, c, _ in got} == want


@pytest.mark.parametrize("rows_total,t0", [(300, 256), (100, 0), (200, 0)])
def test_scalar_offset_pairing_is_caught(rows_total, t0):
    ld = 2 * BK
    got = fetched(rows_total, ld, t0, 0, 0, scalar_pair=True)
    assert any(row >= rows_total for row, _, _ in got)
