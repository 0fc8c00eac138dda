/*
 * Exhaustive CPU check of the quotient the KV-cache write uses under a
 * calibrated scale 2^LOG2_MIN_SCALE <= s <= 2^126 (any value, not tied to
 * the data; the kernel divides for other scales -- above 2^126 the
 * reciprocal is subnormal):
 *     r = RN32(1/s);  q0 = RN32(|x| * r);
 *     q0 >= 448: the saturated code (the IEEE quotient is then above 432,
 *                and every quotient above 432 encodes to 448);
 *     else q = min(fma(fma(-s, q0, |x|), r, q0), 448)
 * against the IEEE quotient RN32(|x| / s) saturated at 448, compared by
 * E4M3 code, for every positive finite bf16 |x| and a set of scales: the
 * scales the linear layers' rule gives for every bf16 amax, log-uniform
 * random normal scales, and edge values (smallest normal, 1, largest).
 * The E4M3 encoder is the OCP definition (RNE, saturating at 448).
 *
 * usage: kv_quotient_check N_RANDOM SEED LOG2_MIN_SCALE   (exit 0 = all codes equal)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static int e4m3_code(double a) {
  if (a >= 448.0) return 0x7E;
  if (a < 0x1p-6) return (int)nearbyint(a * 512.0);
  int e;
  frexp(a, &e);
  e -= 1;
  return (e + 7) * 8 + (int)nearbyint(ldexp(a, 3 - e)) - 8;
}

static uint64_t state;
static uint32_t next_u32(void) {  /* xorshift64* */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1DULL) >> 32);
}

static long long pairs, bad;
static float min_scale;

static void check_scale(float s) {
  if (!(s >= min_scale && s <= 0x1p126f)) return;
  volatile float one = 1.0f;
  const float r = one / s;
  for (uint32_t xb = 0; xb < 0x7F80; ++xb) {
    const float a = bf16(xb);
    float q_ref = a / s;                   /* IEEE, may be inf */
    const int c_ref = (q_ref >= 448.0f) ? 0x7E : e4m3_code(q_ref);
    const float q0 = a * r;
    int c;
    if (q0 >= 448.0f) {
      c = 0x7E;
    } else {
      float q = fmaf(fmaf(-s, q0, a), r, q0);
      q = fminf(q, 448.0f);
      c = e4m3_code(q);
    }
    ++pairs;
    if (c != c_ref && bad++ < 5) printf("s=%a x=%a fast code %#x ieee code %#x\n", s, a, c, c_ref);
  }
}

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int n_random = atoi(argv[1]);
  min_scale = ldexpf(1.0f, atoi(argv[3]));
  state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)atoll(argv[2]);
  int scales = 0;
  /* the linear layers' scale rule on every bf16 amax: RN32(amax/448) */
  volatile float c448 = 448.0f;
  for (uint32_t ab = 1; ab < 0x7F80; ab += 7) {
    const float s = bf16(ab) / c448;
    if (s >= min_scale) { check_scale(s); ++scales; }
  }
  /* log-uniform random normal scales and edge values */
  for (int i = 0; i < n_random; ++i) {
    const uint32_t e = 1 + next_u32() % 254, m = next_u32() & 0x7FFFFF;
    const float s = from_bits((e << 23) | m);
    if (s >= min_scale) { check_scale(s); ++scales; }
  }
  const float edges[] = {0x1p-126f, 0x1.000002p-126f, 0x1p-90f, 0x1.000002p-90f, 1.0f, 0x1p126f,
                         0x1.fffffep125f, 0x1.fffffep-1f, 3.0f};
  for (unsigned i = 0; i < sizeof edges / sizeof edges[0]; ++i)
    if (edges[i] >= min_scale) { check_scale(edges[i]); ++scales; }
  printf("scales=%d pairs=%lld code_mismatches=%lld\n", scales, pairs, bad);
  return bad ? 1 : 0;
}
