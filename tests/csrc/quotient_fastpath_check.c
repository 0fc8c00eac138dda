/*
 * Exhaustive CPU check of the quotient used by the quantisation kernels.
 *
 * The kernels form RN32(|x| / s) as
 *     r = RN32(1 / s);  q0 = RN32(|x| * r);  e = fma(s, q0, -|x|);  q = fma(-e, r, q0)
 * whenever s >= 2**-90 (otherwise they divide). This program walks every
 * positive finite bf16 amax, derives s in the chosen scale mode, and checks
 * every bf16 magnitude |x| <= amax:
 *   - q is bit-identical to the IEEE fp32 quotient whenever that quotient is
 *     >= 2**-12 (smaller quotients encode to 0 either way);
 *   - the E4M3 code of q equals the code of the IEEE quotient, always.
 * The E4M3 encoder here follows the OCP definition (RNE, saturating at 448)
 * and is written independently of both the oracle and the kernels.
 *
 * usage: quotient_fastpath_check POW2 LOG2_MIN_SCALE   (exit 0 = all equal)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int e4m3_code(double a) {
  if (a >= 448.0) return 0x7E;
  if (a < 0x1p-6) return (int)nearbyint(a * 512.0);
  int e;
  frexp(a, &e);
  e -= 1;
  return (e + 7) * 8 + (int)nearbyint(ldexp(a, 3 - e)) - 8;
}

static float scale_of(float amax, int pow2) {
  if (!pow2) return amax / 448.0f;
  int k = (int)ceil(log2((double)amax / 448.0));
  while (ldexp(448.0, k - 1) >= amax) k--;
  while (ldexp(448.0, k) < amax) k++;
  return ldexpf(1.0f, k);
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  const int pow2 = atoi(argv[1]);
  const float min_scale = ldexpf(1.0f, atoi(argv[2]));
  long long pairs = 0, bad_bits = 0, bad_codes = 0;
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf16(ab);
    const float s = scale_of(amax, pow2);
    if (!(s >= min_scale)) continue;
    volatile float one = 1.0f;
    const float r = one / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      const float x = bf16(xb);
      const float q_ref = x / s;
      const float q0 = x * r;
      const float e = fmaf(s, q0, -x);
      const float q = fmaf(-e, r, q0);
      ++pairs;
      if (q_ref >= 0x1p-12f && bits(q) != bits(q_ref)) {
        if (bad_bits++ < 5) printf("bits: x=%a s=%a q=%a ieee=%a\n", x, s, q, q_ref);
      }
      if (e4m3_code(q) != e4m3_code(q_ref)) {
        if (bad_codes++ < 5) printf("code: x=%a s=%a q=%a ieee=%a\n", x, s, q, q_ref);
      }
    }
  }
  printf("pow2=%d pairs=%lld bit_mismatches=%lld code_mismatches=%lld\n", pow2, pairs, bad_bits, bad_codes);
  return (bad_bits || bad_codes) ? 1 : 0;
}
