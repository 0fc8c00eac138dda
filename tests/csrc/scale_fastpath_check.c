/*
 * Exhaustive CPU check of the scale the quantisation kernels compute
 * without a division:
 *     q0 = RN32(amax * R),  R = RN32(1/448);  s = fma(-fma(448, q0, -amax), R, q0)
 * against the IEEE fp32 quotient amax / 448, for every positive finite bf16
 * amax (the largest magnitude of a group is always a bf16 value), with
 * subnormal results included.
 *
 * usage: scale_fastpath_check   (prints the mismatch count; exit 0 = none)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  volatile float one = 1.0f, c448 = 448.0f;
  const float r = one / c448;
  long checked = 0, bad = 0;
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf16(ab);
    const float ref = amax / c448;
    const float q0 = amax * r;
    const float s = fmaf(-fmaf(c448, q0, -amax), r, q0);
    ++checked;
    if (bits(s) != bits(ref) && bad++ < 5) printf("amax=%a fast=%a ieee=%a\n", amax, s, ref);
  }
  printf("R=%a checked=%ld mismatches=%ld\n", r, checked, bad);
  return bad ? 1 : 0;
}
