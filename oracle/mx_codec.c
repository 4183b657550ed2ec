/*
 * OCP E4M3 encoding and MX block quantisation for the CPU oracle, as plain loops.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by oracle/formats.py (ctypes), which documents the readings;
 * nothing in the product path uses it. It shares no code with the HIP library.
 *
 * E4M3 (OCP 8-bit Floating Point v1.0): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds subnormals m * 2^-9; S.1111.111 is NaN, so the largest finite value is 448.
 * Encoding rounds to the nearest representable value, ties to the even mantissa, saturates at 448,
 * keeps the sign of zero and never produces NaN.
 *
 * MX block (OCP Microscaling Formats v1.0): 32 consecutive elements share the scale 2^s with
 * s = floor(log2 amax) - 8, clamped to [-127, 127]; s = -127 when amax = 0; stored as s + 127.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* |y| = f * 2^e with 1 <= f < 2 (normal range, |y| >= 2^-6): mantissa code rint(|y| 2^(3-e)) - 8,
 * a round-up to 16 carrying into the exponent. Below 2^-6 the grid is n * 2^-9 (n = 0 .. 8; n = 8
 * is the smallest normal, code 0x08). rint rounds half to even in the default rounding mode. */
static uint8_t e4m3_encode_one(double y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;
  const double a = fabs(y);
  int code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < 0.015625) {
    code = (int)rint(a * 512.0);
  } else {
    int ex;
    frexp(a, &ex); /* a = g * 2^ex, 0.5 <= g < 1, so e = ex - 1 */
    int e = ex - 1;
    int n = (int)rint(ldexp(a, 3 - e));
    if (n == 16) {
      n = 8;
      ++e;
    }
    code = ((e + 7) << 3) | (n - 8);
    if (code > 0x7E) code = 0x7E;
  }
  return (uint8_t)(code | sign);
}

void oracle_e4m3_encode(const double* y, uint8_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = e4m3_encode_one(y[i]);
}

/* v: nrows x ncols, row-major; blocks of 32 run along each row (ncols % 32 == 0).
 * codes: nrows x ncols; scales: nrows x (ncols / 32). */
void oracle_mx_quantize_rows(const double* v, size_t nrows, size_t ncols, uint8_t* codes,
                             uint8_t* scales) {
  const size_t nb = ncols / 32;
  for (size_t r = 0; r < nrows; ++r) {
    for (size_t b = 0; b < nb; ++b) {
      const double* blk = v + r * ncols + 32 * b;
      double amax = 0.0;
      for (int q = 0; q < 32; ++q) amax = fmax(amax, fabs(blk[q]));
      int s = -127;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* floor(log2 amax) = ex - 1 */
        s = ex - 1 - 8;
        if (s < -127) s = -127;
        if (s > 127) s = 127;
      }
      for (int q = 0; q < 32; ++q) codes[r * ncols + 32 * b + q] = e4m3_encode_one(ldexp(blk[q], -s));
      scales[r * nb + b] = (uint8_t)(s + 127);
    }
  }
}

/* The value each element takes after MX quantisation along one axis: v viewed as
 * [outer][L][inner] (L % 32 == 0), blocks of 32 consecutive positions along L for every (outer,
 * inner); out[i] = 2^s * value(code). The value of a code comes straight from its bit fields:
 * exponent field 0 gives man * 2^-9, else (1 + man / 8) * 2^(ex - 7). amax is a scratch array of
 * `inner` doubles. */
static double e4m3_value(uint8_t c) {
  const int ex = (c >> 3) & 0xF, man = c & 0x7;
  const double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);
  return (c & 0x80) ? -mag : mag;
}

void oracle_mx_roundtrip_axis(const double* v, double* out, size_t outer, size_t L, size_t inner,
                              double* amax) {
  for (size_t o = 0; o < outer; ++o) {
    for (size_t b = 0; b < L / 32; ++b) {
      const double* blk = v + (o * L + 32 * b) * inner;
      double* dst = out + (o * L + 32 * b) * inner;
      for (size_t i = 0; i < inner; ++i) amax[i] = 0.0;
      for (int q = 0; q < 32; ++q)
        for (size_t i = 0; i < inner; ++i) amax[i] = fmax(amax[i], fabs(blk[q * inner + i]));
      for (size_t i = 0; i < inner; ++i) { /* the block exponent s, kept in amax[i] */
        int s = -127;
        if (amax[i] > 0.0) {
          int ex;
          frexp(amax[i], &ex);
          s = ex - 1 - 8;
          if (s < -127) s = -127;
          if (s > 127) s = 127;
        }
        amax[i] = (double)s;
      }
      for (int q = 0; q < 32; ++q)
        for (size_t i = 0; i < inner; ++i) {
          const int s = (int)amax[i];
          dst[q * inner + i] = ldexp(e4m3_value(e4m3_encode_one(ldexp(blk[q * inner + i], -s))), s);
        }
    }
  }
}
