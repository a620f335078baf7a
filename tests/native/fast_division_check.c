/*
 * Exhaustive check behind the quantizers' reciprocal path.
 *
 * The GPU quantizers compute a code as round(x / s) with s = fl(amax / Q)
 * (Q = 127 for int8, 448 for E4M3) and IEEE binary32 division.  For rows
 * whose scale is at least 2^-96 they instead form r = fl(1 / s) once and,
 * per element, q0 = fl(x * r), e = fma(-q0, s, x), q = fma(e, r, q0).  q can
 * differ from fl(x / s) by one ulp, but the code it rounds to must not.
 *
 * Every input is a bf16 value, and |x| <= amax within a row, so the whole
 * domain is finite: every positive finite bf16 amax, every bf16 x in
 * [0, amax].  (The kernels apply the formulas to |x| and then copy x's sign,
 * which is what the division does too, -0 included; so x >= 0 covers all.)
 * This program walks the whole domain for both Q and prints the number of
 * pairs whose codes differ with s >= 2^-96 (must be 0) and, for
 * information, below it.
 *
 * Codes: int8 = clamp(rint(q), -127, 127); E4M3 = round-to-nearest-even of
 * clamp(q, -448, 448) on the E4M3 grid (subnormal quantum 2^-9).
 * Build: gcc -O2 -mfma -ffp-contract=off fast_division_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int code_i8(float q) {
  float r = rintf(q);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int)r;
}

/* E4M3 RNE of clamp(q) for q >= 0, returned as the value times 2^12 (unique). */
static long code_e4m3(float qf) {
  double q = qf > 448.0f ? 448.0 : (double)qf;
  if (q < 0.015625) return (long)rint(q * 512.0) * 8;
  int e;
  frexp(q, &e);                        /* q in [2^(e-1), 2^e) */
  double quantum = ldexp(1.0, e - 4);  /* 3 mantissa bits */
  return (long)(rint(q / quantum) * quantum * 4096.0);
}

int main(void) {
  const float Qs[2] = {127.0f, 448.0f};
  const float min_scale = ldexpf(1.0f, -96);
  int failed = 0;
  for (int qi = 0; qi < 2; ++qi) {
    long long pairs = 0, bad = 0, bad_tiny = 0;
    for (uint32_t ab = 1; ab < 0x7f80u; ++ab) {
      const float a = bf16(ab);
      const volatile float s = a / Qs[qi];
      const volatile float r = 1.0f / s;
      for (uint32_t xb = 0; xb <= ab; ++xb) {
        const float x = bf16(xb);
        const volatile float qd = x / s;
        const volatile float q0 = x * r;
        const float e = fmaf(-q0, s, x);
        const float q = fmaf(e, r, q0);
        ++pairs;
        const int differ = qi == 0 ? code_i8(q) != code_i8(qd) : code_e4m3(q) != code_e4m3(qd);
        if (differ) {
          if (s >= min_scale) {
            ++bad;
            if (bad <= 5) printf("  Q=%g amax=%a x=%a: %a vs %a\n", Qs[qi], a, x, q, qd);
          } else {
            ++bad_tiny;
          }
        }
      }
    }
    printf("Q=%g pairs=%lld code_mismatches_at_or_above_2^-96=%lld below=%lld\n", Qs[qi], pairs, bad, bad_tiny);
    if (bad) failed = 1;
  }
  return failed;
}
