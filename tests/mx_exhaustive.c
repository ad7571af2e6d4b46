/* Exhaustive check of the oracle's E4M3 encoder over every float bit pattern.
 *
 * Independent reference: the 127 non-negative finite E4M3 magnitudes are
 * built from the format's definition (bias 7, 3 mantissa bits, subnormals
 * m*2^-9, exponent field 15 with mantissa 7 reserved for NaN), and each float
 * is mapped to the nearest magnitude by binary search, ties to the code with
 * an even mantissa, magnitudes at or above 448 (and infinities) saturating to
 * 448, the sign bit copied, NaN mapped to 0x7f.  Exits 0 when all 2^32
 * patterns agree, else prints the first few mismatches and exits 1.
 * Test-only helper: links the oracle's shared library, nothing else.        */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

extern uint8_t oracle_e4m3_encode(float v);

static double mag[127];

static uint8_t reference(uint32_t bits) {
  float f;
  memcpy(&f, &bits, 4);
  uint8_t sign = (uint8_t)((bits >> 31) << 7);
  if (isnan(f)) return 0x7f;
  double a = fabs((double)f);
  if (a >= 448.0) return sign | 0x7e;
  int lo = 0, hi = 126; /* mag[lo] <= a < mag[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (mag[mid] <= a) lo = mid; else hi = mid;
  }
  double dl = a - mag[lo], dh = mag[hi] - a;
  int code;
  if (dl < dh) code = lo;
  else if (dh < dl) code = hi;
  else code = (lo % 2 == 0) ? lo : hi; /* tie: even mantissa (code parity) */
  return sign | (uint8_t)code;
}

int main(void) {
  for (int c = 0; c < 127; ++c) {
    int e = c >> 3, m = c & 7;
    mag[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  }
  long long bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (long long i = 0; i < (1LL << 32); ++i) {
    uint32_t b = (uint32_t)i;
    float f;
    memcpy(&f, &b, 4);
    uint8_t want = reference(b), got = oracle_e4m3_encode(f);
    if (want != got) {
      if (bad < 5) {
#pragma omp critical
        printf("mismatch bits=%08x v=%.9g want=%02x got=%02x\n", b, (double)f, want, got);
      }
      bad++;
    }
  }
  printf("mismatches: %lld\n", bad);
  return bad != 0;
}
