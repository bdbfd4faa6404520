// The FP8 quantize step divides by a row's scale s as q0 = x y, r = fma(-q0, s, x),
// q = fma(r, y, q0) with y the correctly rounded 1 / s (Markstein's division
// step), the quotient taking x's sign.  This program draws float32 pairs (scales
// 2^-40 .. 2^40, including all-ones and power-of-two mantissas; quotients within
// +-450, half of them near multiples of s and of s / 8) and checks against the
// correctly rounded x / s that every normal quotient is equal and that the E4M3
// code (the kernel's rounding, after the clamp to +-448) is equal for all.
// Usage: quant_division_check [pairs]; exit status 0 when nothing differs.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
static uint32_t e4m3_code(float y) {
  const uint32_t uu = u(y);
  const uint32_t sign = (uu >> 24) & 0x80u;
  const uint32_t a = uu & 0x7fffffffu;
  uint32_t mag;
  if (a < 0x3c800000u) mag = (uint32_t)rintf(f(a) * 512.0f);
  else mag = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | mag;
}
static uint32_t code_of(float q) { return e4m3_code(fminf(fmaxf(q, -448.f), 448.f)); }
static uint64_t st = 88172645463325252ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(int argc, char **argv) {
  long long n = argc > 1 ? atoll(argv[1]) : 100000000LL, bad = 0, tested = 0;
  for (long long i = 0; i < n; ++i) {
    uint64_t r = rnd();
    // s: a positive normal with a random mantissa and an exponent from 2^-40..2^40
    uint32_t se = 127 - 40 + (uint32_t)(r % 81);
    float s = f((se << 23) | (uint32_t)((r >> 8) & 0x7fffff));
    if (i % 4 == 0) s = f((se << 23) | 0x7fffff);            // all-ones mantissa
    if (i % 4 == 1) s = f((se << 23));                       // power of two
    float y = 1.0f / s;
    uint64_t r2 = rnd();
    // x: |x| <= 448 s, random bits, or near multiples of s (ties of the quotient)
    float x;
    if (i % 3 == 0) {
      float k = (float)(int)((r2 >> 20) % 900) - 450.f + (float)((r2 >> 40) & 7) / 8.f;
      x = k * s;
      x = f(u(x) + (uint32_t)((int)((r2 >> 50) % 5) - 2));
    } else {
      uint32_t xe = (uint32_t)((u(s) >> 23) - 30 + (r2 % 40));
      if (xe < 1 || xe > 254) continue;
      x = f((xe << 23) | (uint32_t)((r2 >> 8) & 0x7fffff) | ((uint32_t)(r2 >> 63) << 31));
    }
    if (!(fabsf(x) <= 448.f * s * 1.0001f)) continue;
    float want = x / s;
    float q0 = x * y;
    float rr = fmaf(-q0, s, x);
    float q1 = fmaf(rr, y, q0);
    q1 = copysignf(q1, x);   // the quotient's sign is x's (s > 0), zeros included
    ++tested;
    const int normal = fabsf(want) >= 0x1p-126f;
    if ((normal && u(q1) != u(want)) || code_of(q1) != code_of(want)) {
      if (bad < 10) printf("mismatch x=%a s=%a want=%a got=%a codes %x %x\n", x, s, want, q1, code_of(want), code_of(q1));
      ++bad;
    }
  }
  printf("tested %lld, mismatches %lld\n", tested, bad);
  return bad != 0;
}
