/* Brute-force FP8 rounding check used only by the oracle's tests.
 *
 * For every fp32 bit pattern in [lo, hi) (NaNs skipped): clamp |v| to fmax,
 * find the nearest value of a sorted grid of non-negative finite FP8 values
 * (grid[i] is the value of code i) by search, break ties toward the even code,
 * restore the sign bit, and compare with the encoder under test.  The grid
 * comes from a library decoder (torch), not from the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

static uint8_t nearest_code(double a, const double *grid, int n) {
  int lo = 0, hi = n - 1;
  double dlo, dhi;
  if (a <= grid[0]) return 0;
  if (a >= grid[n - 1]) return (uint8_t)(n - 1);
  while (hi - lo > 1) {              /* grid[lo] <= a < grid[hi] */
    int mid = (lo + hi) / 2;
    if (grid[mid] <= a) lo = mid; else hi = mid;
  }
  dlo = a - grid[lo];
  dhi = grid[hi] - a;
  if (dlo < dhi) return (uint8_t)lo;
  if (dhi < dlo) return (uint8_t)hi;
  return (uint8_t)((lo % 2 == 0) ? lo : hi);
}

uint64_t count_mismatch(uint64_t lo, uint64_t hi, const double *grid, int n,
                        double fmax, enc_fn enc, uint32_t *first_bad) {
  uint64_t bad = 0;
  int64_t i;
  *first_bad = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (i = (int64_t)lo; i < (int64_t)hi; ++i) {
    uint32_t u = (uint32_t)i;
    float v;
    double a;
    uint8_t want, got;
    memcpy(&v, &u, 4);
    if (isnan(v)) continue;
    a = fabs((double)v);
    if (a > fmax) a = fmax;
    want = nearest_code(a, grid, n);
    if (signbit(v)) want |= 0x80;
    got = enc(v);
    if (got != want) {
      bad++;
#pragma omp critical
      if (u < *first_bad) *first_bad = u;
    }
  }
  return bad;
}
