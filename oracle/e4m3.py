"""E4M3 codec for the oracle (test infrastructure only; see package header).

The greentreeone.com NeMo RL article, section «Технический прорыв», names the
element format only as "E4M3". Reading taken: the OCP 8-bit floating point
E4M3 variant ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, subnormals when the exponent field is 0, no infinities, and NaN only
for exponent and mantissa fields all ones (codes 0x7F and 0xFF). The largest
finite magnitude is 448 = 1.75 * 2**8. Rounding is to nearest with ties to an
even mantissa, and magnitudes beyond 448 saturate to 448 (never NaN).

Pins (tests/test_oracle_e4m3.py): the decode table against torch's own
float8_e4m3fn decoding and against the format's closed-form landmarks; the
encoder against ``encode_bruteforce`` (nearest finite code by exhaustive
search) on every bf16 bit pattern and on every midpoint between adjacent codes
+-1 fp32 ulp, and against torch's float8_e4m3fn cast on in-range values.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6      # exponent field 1, mantissa 0
_SUBNORMAL_STEP = 2.0 ** -9  # exponent field 0, mantissa 1


def decode_table():
    """Value of each of the 256 codes, float64; NaN at 0x7F and 0xFF.

    Built field by field from the format definition: sign, 4-bit exponent
    with bias 7, 3-bit mantissa; exponent field 0 holds subnormals
    m * 2**-9; otherwise the value is (1 + m/8) * 2**(e - 7).
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            vals[code] = np.nan
        elif exp_field == 0:
            vals[code] = sign * mant * _SUBNORMAL_STEP
        else:
            vals[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return vals


_TABLE = decode_table()


def decode(codes):
    """Decode an array of uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(values):
    """Round finite values to E4M3 codes (uint8), RNE with saturation at 448.

    ``values`` may be any float array; each value is widened exactly to
    float64. The sign bit of the input is kept for every result, so -0.0 and
    negative values that round to zero give 0x80.

    For a magnitude a:
      * a >= 448 saturates to the largest finite code (0x7E);
      * a < 2**-6 lies in the subnormal range, whose grid has step 2**-9:
        the mantissa is round_half_even(a / 2**-9), which may reach 8, the
        first normal code;
      * otherwise a lies in the binade [2**e, 2**(e+1)) whose grid has step
        2**(e-3): n = round_half_even(a / 2**(e-3)) is in [8, 16]; the code is
        (e + 7) * 8 + (n - 8), and n = 16 carries into the next binade.
    """
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encoder oracle: inputs must be finite")
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)

    sat = a >= E4M3_MAX
    sub = a < _MIN_NORMAL
    nrm = ~sat & ~sub

    code[sat] = 0x7E
    code[sub] = np.rint(a[sub] / _SUBNORMAL_STEP).astype(np.int64)

    an = a[nrm]
    _, ex = np.frexp(an)           # an = f * 2**ex with f in [0.5, 1)
    e = ex.astype(np.int64) - 1    # an in [2**e, 2**(e+1))
    n = np.rint(np.ldexp(an, (3 - e).astype(np.int32))).astype(np.int64)
    code[nrm] = (e + 7) * 8 + (n - 8)

    code |= np.signbit(v).astype(np.int64) << 7
    return code.astype(np.uint8)


def encode_bruteforce(values):
    """Independent twin of ``encode``: exhaustive nearest-code search.

    For each magnitude, every finite non-negative code (0x00..0x7E) is a
    candidate; the nearest one wins and a tie goes to the code with an even
    mantissa (even code number). Magnitudes above 448 therefore land on 448
    (saturation) because no larger finite code exists. The sign bit is copied
    from the input. Slow: intended for tests on at most a few 10**5 values.
    """
    v = np.asarray(values, dtype=np.float64).ravel()
    cand = np.arange(0x7F)                     # 0x00..0x7E
    cand_val = _TABLE[cand]
    out = np.empty(v.shape, dtype=np.uint8)
    chunk = 4096
    for i in range(0, v.size, chunk):
        # For |v| >= 448 every candidate lies at or below |v|, so the distances
        # |v| - c rank the candidates the same way for any such |v|; capping
        # at 896 keeps every distance exact in float64 (candidates are
        # multiples of 2**-9 below 2**9). Below 448 the two nearest distances
        # are exact by Sterbenz's lemma, so ties are seen as ties.
        a = np.minimum(np.abs(v[i:i + chunk]), 2 * E4M3_MAX)[:, None]
        d = np.abs(a - cand_val[None, :])
        best = d.min(axis=1, keepdims=True)
        is_best = d == best
        # among the (at most two) nearest codes prefer the even one
        even_best = is_best & (cand[None, :] % 2 == 0)
        pick = np.where(even_best.any(axis=1),
                        np.argmax(even_best, axis=1),
                        np.argmax(is_best, axis=1))
        out[i:i + chunk] = cand[pick] | (np.signbit(v[i:i + chunk]).astype(np.int64) << 7)
    return out.reshape(np.shape(values))
