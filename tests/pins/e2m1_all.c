/* Exhaustive pin of the oracle's E2M1 rounding (test infrastructure).
 *
 * Every non-negative finite fp32 value (bit patterns 0 .. 0x7F7FFFFF) is
 * rounded by the oracle's routine, passed in as a function pointer, and by
 * the rule written here independently as intervals on the value line:
 * round to the nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6} (codes 0..7), a tie
 * going to the even code, saturating at 6.  Returns the number of values on
 * which the two disagree.
 */
#include <stdint.h>
#include <string.h>

typedef void (*rne_fn)(int64_t n, const double* v, uint8_t* codes);

static unsigned interval_code(float x) {
  if (x <= 0.25f) return 0;  /* [0, 0.25]: tie at 0.25 goes to 0 */
  if (x < 0.75f) return 1;   /* (0.25, 0.75) -> 0.5 */
  if (x <= 1.25f) return 2;  /* [0.75, 1.25] -> 1 */
  if (x < 1.75f) return 3;   /* (1.25, 1.75) -> 1.5 */
  if (x <= 2.5f) return 4;   /* [1.75, 2.5] -> 2 */
  if (x < 3.5f) return 5;    /* (2.5, 3.5) -> 3 */
  if (x <= 5.0f) return 6;   /* [3.5, 5] -> 4 */
  return 7;                  /* (5, inf) -> 6 */
}

int64_t check_all(rne_fn f) {
  enum { CH = 1 << 20 };
  static double v[CH];
  static uint8_t c[CH];
  int64_t bad = 0;
  for (uint64_t b0 = 0; b0 < 0x7F800000ull; b0 += CH) {
    const uint64_t n = 0x7F800000ull - b0 < CH ? 0x7F800000ull - b0 : CH;
    for (uint64_t i = 0; i < n; ++i) {
      const uint32_t u = (uint32_t)(b0 + i);
      float x;
      memcpy(&x, &u, 4);
      v[i] = (double)x;
    }
    f((int64_t)n, v, c);
    for (uint64_t i = 0; i < n; ++i) {
      const float x = (float)v[i];
      if (c[i] != interval_code(x)) ++bad;
    }
  }
  return bad;
}
