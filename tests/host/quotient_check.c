/*
 * Host check of the division-free INT8 code computation used by the
 * quantization kernel: with y = RN(1/s), q0 = RN(x*y), r = fma(-q0, s, x),
 * the value RN(q0 + r*y) must equal the IEEE quotient RN(x/s) for every
 * operand pair the quantizer can produce (s = RN(a/127) of a block max a, and
 * |x| <= a). Cases: random blocks over a wide exponent range, block maxima
 * themselves, and quotients within a few ulps of every half-integer k + 1/2
 * (where rounding to the nearest code is decided).
 * Usage: quotient_check [n_random]   exit status 0 iff no mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t rng_state = 88172645463325252ull;
static uint64_t next_u64(void) {  /* xorshift64 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static long long n_cases = 0, n_bad = 0;
static void check(float x, float s) {
  const float y = 1.0f / s;
  const float q0 = x * y;
  const float r = fmaf(-q0, s, x);
  const float q1 = fmaf(r, y, q0);
  const float q = x / s;
  ++n_cases;
  if (to_bits(q1) != to_bits(q)) {
    if (n_bad < 5) printf("mismatch: x=%a s=%a x/s=%a corrected=%a\n", x, s, q, q1);
    ++n_bad;
  }
}

int main(int argc, char** argv) {
  const long long n = argc > 1 ? atoll(argv[1]) : 20000000LL;
  for (long long it = 0; it < n; ++it) {
    const uint64_t u = next_u64();
    /* block max a: random mantissa, exponent 2^-60 .. 2^20 */
    const float a = from_bits((uint32_t)(u & 0x007fffffu) | (uint32_t)((67 + (u >> 23) % 80) << 23));
    const float s = a / 127.0f;
    const float t = (float)((double)(next_u64() >> 11) * 0x1p-53) * 2.0f - 1.0f;
    float x = t * a;
    if ((it & 7) == 0) x = a;
    if ((it & 7) == 1) x = -a;
    check(x, s);
  }
  for (long long it = 0; it < n / 8; ++it) {
    const uint64_t u = next_u64();
    const float a = from_bits((uint32_t)(u & 0x007fffffu) | (uint32_t)((67 + (u >> 23) % 80) << 23));
    const float s = a / 127.0f;
    const float x = ((float)(next_u64() % 127) + 0.5f) * s;
    for (int d = -3; d <= 3; ++d) {
      check(from_bits(to_bits(x) + d), s);
      check(-from_bits(to_bits(x) + d), s);
    }
  }
  printf("%lld cases, %lld mismatches\n", n_cases, n_bad);
  return n_bad != 0;
}
