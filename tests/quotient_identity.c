/* Exhaustive host check of the division-free activation quotient.
 *
 * The activation quantizers on the GPU take q = x / s as q0 = x*r,
 * e = fma(-q0, s, x), q = copysign(fma(e, r, q0), x) with r = 1/s
 * (Markstein's correction step) whenever s >= 2^-100, and divide otherwise.
 * The codes must equal those of the correctly rounded quotient.  This
 * program walks the whole domain the quantizers meet: every positive finite
 * bf16 amax, its scale s = amax / Q (Q = 448 for E4M3FN, 127 for int8,
 * correctly rounded), and every bf16 x with |x| <= amax; where the two
 * quotients differ in any bit it compares their codes (E4M3FN: nearest
 * value, ties to the even code, saturating at 448, sign kept; int8: round
 * to nearest even, clamp to [-127, 127]).
 *
 * Prints one line per Q: "Q pairs quotient_diffs code_diffs".  Build with
 * -ffp-contract=off so the compiler fuses nothing on its own.  With the
 * argument "nosign" it drops the copysign (a planted mistake: negative zero
 * then encodes as positive zero) and samples every 61st amax.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Magnitude of E4M3FN code c (0 <= c <= 0x7E): bias 7, subnormals below 2^-6. */
static double e4m3_mag(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
}

static int e4m3_code(float q) {
  const int sign = signbit(q) ? 0x80 : 0;
  double a = fabs((double)q);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double d = fabs(e4m3_mag(c) - a);
    if (d < bd || (d == bd && !(c & 1))) { bd = d; best = c; }
  }
  return sign | best;
}

static int i8_code(float q) {
  float r = rintf(q);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return ((int)r) & 0xFF;
}

int main(int argc, char** argv) {
  const int nosign = argc > 1 && strcmp(argv[1], "nosign") == 0;
  const uint32_t stride = nosign ? 61 : 1;
  const float qmax[2] = {448.0f, 127.0f};
  for (int k = 0; k < 2; ++k) {
    long long pairs = 0, qdiff = 0, cdiff = 0;
#pragma omp parallel for reduction(+ : pairs, qdiff, cdiff) schedule(dynamic, 64)
    for (uint32_t a = 1; a < 0x7F80; a += stride) {
      const float amax = from_bits(a << 16);
      volatile float Q = qmax[k];
      const float s = amax / Q;
      if (!(s >= 0x1p-100f)) continue; /* these scales divide */
      const float r = 1.0f / s;
      for (uint32_t b = 0; b < 0x10000; ++b) {
        const float x = from_bits(b << 16);
        if (!(fabsf(x) <= amax)) continue;
        ++pairs;
        const float ref = x / s;
        const float q0 = x * r;
        const float e = fmaf(-q0, s, x);
        const float q = nosign ? fmaf(e, r, q0) : copysignf(fmaf(e, r, q0), x);
        if (to_bits(q) == to_bits(ref)) continue;
        ++qdiff;
        const int c1 = k ? i8_code(q) : e4m3_code(q);
        const int c2 = k ? i8_code(ref) : e4m3_code(ref);
        if (c1 != c2) ++cdiff;
      }
    }
    printf("%g %lld %lld %lld\n", qmax[k], pairs, qdiff, cdiff);
  }
  return 0;
}
