/* The e4m3 quantisers replace the division v / s of every value by a product
 * corrected once with the exact FMA remainder (Markstein's correction step):
 *
 *   y = fp32(1 / s);  q0 = fp32(v * y);  q = copysign(fma(fma(-q0, s, v), y, q0), v)
 *
 * for blocks whose scale s = fp32(amax / 448) is at least 2^-90.  This program
 * checks on the CPU (IEEE fp32 with subnormals, correctly rounded fmaf) that q
 * equals the IEEE quotient fp32(v / s) bit for bit whenever that quotient is at
 * least 2^-14 in magnitude, and that both lie below 2^-12 otherwise (e4m3 code
 * +-0 either way, the sign being that of v).
 *
 *   quotient_check bf16 EMIN EMAX   every bf16 amax with exponent in [EMIN, EMAX]
 *                                   and every bf16 v with |v| <= amax, both signs
 *   quotient_check fp32 N SEED      N random fp32 amax, 16 random v each, plus
 *                                   values on and next to the midpoints between
 *                                   e4m3 codes (the ties of the final rounding)
 *
 * A fourth argument "plain" drops the correction (q = copysign(q0, v)), which
 * must then show mismatches: the control that the check can fail.
 *
 * Prints "checked <n> mismatches <m>" and exits with status 1 if m > 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}
static uint32_t bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

static uint64_t checked, mismatches;
static int plain;

static void check(float v, float s, float y) {
  volatile float ref = v / s;
  const float q0 = v * y;
  const float q = copysignf(plain ? q0 : fmaf(fmaf(-q0, s, v), y, q0), v);
  ++checked;
  int ok;
  if (fabsf(ref) >= 0x1p-14f)
    ok = bits(q) == bits(ref);
  else
    ok = fabsf(q) < 0x1p-12f && signbit(q) == signbit(ref);
  if (!ok && mismatches++ < 5) printf("mismatch v=%a s=%a ieee=%a corrected=%a\n", v, s, ref, q);
}

static uint64_t state;
static uint64_t next(void) {  /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) return 2;
  plain = argc == 5 && !strcmp(argv[4], "plain");
  if (!strcmp(argv[1], "bf16")) {
    const int emin = atoi(argv[2]), emax = atoi(argv[3]);
    for (int ea = emin; ea <= emax; ++ea)
      for (uint32_t ma = 0; ma < 128; ++ma) {
        const float amax = from_bits(((uint32_t)(ea + 127) << 23) | (ma << 16));
        const float s = amax / 448.0f;
        if (s < 0x1p-90f) continue;
        const float y = 1.0f / s;
        for (uint32_t b = 0; b <= bits(amax) >> 16; ++b) {
          const float v = from_bits(b << 16);
          check(v, s, y);
          check(-v, s, y);
        }
      }
  } else if (!strcmp(argv[1], "fp32")) {
    const long n = atol(argv[2]);
    state = 0x9e3779b97f4a7c15ull ^ (uint64_t)atol(argv[3]);
    for (long i = 0; i < n; ++i) {
      uint32_t ea = 48 + (uint32_t)(next() % 200);
      if (ea > 254) ea = 254;
      const float amax = from_bits((ea << 23) | (uint32_t)(next() & 0x7fffff));
      const float s = amax / 448.0f;
      if (s < 0x1p-90f) continue;
      const float y = 1.0f / s;
      for (int k = 0; k < 16; ++k) {
        const uint32_t de = (uint32_t)(next() % 40);
        const uint32_t ev = ea > de ? ea - de : 1;
        float v = from_bits((ev << 23) | (uint32_t)(next() & 0x7fffff));
        if (v > amax) v = amax;
        check(next() & 1 ? -v : v, s, y);
        /* t = an e4m3 midpoint (1 + (2m + 1) / 16) * 2^e; w = fp32(t s) and its neighbours */
        const float t = from_bits(((uint32_t)(127 - 6 + (int)(next() % 15)) << 23) |
                                  ((uint32_t)(2 * (next() % 8) + 1) << 19));
        const float w = t * s;
        if (fabsf(w) <= amax) {
          check(w, s, y);
          check(from_bits(bits(w) + 1), s, y);
          check(from_bits(bits(w) - 1), s, y);
        }
      }
    }
  } else {
    return 2;
  }
  printf("checked %llu mismatches %llu\n", (unsigned long long)checked,
         (unsigned long long)mismatches);
  return mismatches ? 1 : 0;
}
