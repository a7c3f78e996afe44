/* Host check of the key store's division-free quotient (not the oracle).
 *
 * For a bf16 key value a with |a| <= amax (amax a positive finite bf16) and
 * b = RN(amax / 448) in [2^-60, 2^100], the store computes
 *     y = RN(1/b),  q0 = RN(a*y),  q = fma(fma(-b, q0, a), y, q0)
 * and takes the code's sign from a.  This program checks that |q| equals
 * |RN(a/b)| whenever either is at least 2^-11 (below that the e4m3fn code is
 * zero), also with the residual flushed to zero when it is subnormal.
 * Arguments: number of draws, seed.  Exit status 0 when no value differs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static float bf16(uint32_t bits) {
  uint32_t u = bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(int argc, char** argv) {
  const long n = argc > 1 ? atol(argv[1]) : 10000000L;
  state = argc > 2 ? strtoull(argv[2], 0, 10) : 88172645463325252ull;
  long tested = 0, bad = 0;
  for (long i = 0; i < n; ++i) {
    const uint64_t r = next();
    const uint32_t am = (uint32_t)(r & 0x7fff);
    if (am == 0 || (am >> 7) == 0xff) continue;
    const float amax = bf16(am);
    float a = bf16((uint32_t)((r >> 16) & 0xffff));
    if ((r >> 40) % 7 == 0)  /* values that are simple fractions of amax */
      a = bf16((uint32_t)((r >> 32) & 0x8000) | (uint32_t)(((uint64_t)am * ((r >> 48) & 0xff)) >> 8));
    if ((r >> 44) % 11 == 0) a = bf16((uint32_t)((r >> 32) & 0x8000) | am);  /* the amax element */
    if (!(fabsf(a) <= amax)) continue;
    const float b = amax / 448.0f;
    if (!(b >= 0x1p-60f && b <= 0x1p100f)) continue;
    const float y = 1.0f / b;
    const float q0 = a * y;
    const float q = a / b;
    for (int flush = 0; flush < 2; ++flush) {
      float res = fmaf(-b, q0, a);
      if (flush && fabsf(res) < 0x1p-126f) res = copysignf(0.0f, res);
      const float q1 = fmaf(res, y, q0);
      const int relevant = fabsf(q) >= 0x1p-11f || fabsf(q1) >= 0x1p-11f;
      if (relevant && (bits_of(q1) & 0x7fffffffu) != (bits_of(q) & 0x7fffffffu)) {
        if (bad < 5) printf("a=%a b=%a a/b=%a q=%a\n", a, b, q, q1);
        ++bad;
      }
    }
    ++tested;
  }
  printf("tested %ld pairs, %ld differ\n", tested, bad);
  return bad != 0;
}
