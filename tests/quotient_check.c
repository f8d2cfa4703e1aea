/* Test support (CPU): the three-instruction quotient the GPU's routing and
 * selection kernels use for e / l, checked against IEEE binary32 division.
 *   q0 = RN(e r), rem = RN(e - q0 l) (one fma, exact), q = RN(q0 + rem r) (one fma),
 *   with r = RN(1 / l).
 * Domain of the callers: e in [0, 1] (an exponential of a non-positive number),
 * l >= 1 (a softmax row sum that contains its maximum's 1).  Exit status 0 iff
 *   - q equals e / l bit for bit whenever e / l is a normal number, and
 *   - rint(q 2^40) equals rint((e / l) 2^40) otherwise (the only use of q).
 * Cases: every e in [2^-30, 1] for a set of l (near 1, near 2 and random up to
 * 2^24), random (e, l) pairs, and e = RN(l M) for random rounding midpoints M
 * (quotients within about 2^-25 of a midpoint, some within 2^-40).
 * Usage: quotient_check <n_l_exhaustive> <n_random> <n_midpoint> */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float quot3(float e, float l, float r) {
  const float q0 = e * r;
  const float rem = fmaf(-q0, l, e);
  return fmaf(rem, r, q0);
}

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}

static long long bad = 0;
static void check(float e, float l) {
  const float r = 1.0f / l;
  const float q = e / l, m = quot3(e, l, r);
  int ok;
  if (fabsf(q) >= 0x1p-126f)
    ok = u_of(q) == u_of(m);
  else
    ok = rintf(ldexpf(q, 40)) == rintf(ldexpf(m, 40));
  if (!ok) {
    if (bad < 5) printf("mismatch e=%a l=%a q=%a three-step=%a\n", e, l, q, m);
    ++bad;
  }
}

int main(int argc, char** argv) {
  const int n_l = argc > 1 ? atoi(argv[1]) : 4;
  const long long n_rand = argc > 2 ? atoll(argv[2]) : 10000000LL;
  const long long n_mid = argc > 3 ? atoll(argv[3]) : 10000000LL;
  long long tot = 0;
  for (int i = 0; i < n_l; ++i) {
    float l;
    if (i == 0) l = 1.0f;
    else if (i == 1) l = f_of(0x3fffffffu);                     /* just below 2 */
    else if (i == 2) l = f_of(0x3f800001u);                     /* just above 1 */
    else l = f_of(0x3f800000u + (uint32_t)(next() % (24u << 23)));  /* [1, 2^24) */
    for (uint32_t ue = u_of(0x1p-30f); ue <= u_of(1.0f); ++ue, ++tot) check(f_of(ue), l);
    check(0.0f, l);
  }
  for (long long i = 0; i < n_rand; ++i, ++tot) {
    const uint32_t lo = u_of(0x1p-60f), hi = u_of(1.0f);
    const float e = f_of(lo + (uint32_t)(next() % (hi - lo + 1)));
    const float l = f_of(0x3f800000u + (uint32_t)(next() % (24u << 23)));
    check(e, l);
  }
  for (long long i = 0; i < n_mid; ++i) {
    const float l = f_of(0x3f800000u + (uint32_t)(next() % (24u << 23)));
    const int ex = -(int)(next() % 40) - 1;
    const uint64_t mant = (1ull << 24) | (next() & ((1ull << 24) - 1)) | 1ull; /* odd 25-bit: a midpoint */
    const double M = ldexp((double)mant, ex - 24);
    const float e = (float)((double)l * M); /* l M is exact in double; one rounding to binary32 */
    if (!(e >= 0.0f && e <= 1.0f)) continue;
    check(e, l);
    ++tot;
  }
  printf("quotient_check: %lld cases, %lld mismatched\n", tot, bad);
  return bad == 0 ? 0 : 1;
}
