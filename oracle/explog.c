/* The oracle's EXP and LOG (oracle/logsoftmax.py) replayed in C, for exhaustive sweeps of
 * billions of inputs that numpy would take minutes over.  TEST INFRASTRUCTURE: only tests/
 * load it.  It shares nothing with the HIP library: the constants come in from the Python
 * oracle (derived there from exact rationals) and the steps are those of the Python oracle,
 * one IEEE binary32 operation at a time (built with -ffp-contract=off, no fast-math; the
 * host's float multiply, add and divide round to nearest even).
 *
 * EXP(d), d <= 0 or NaN: Cody & Waite (1980) reduction d = k ln2 + r, ln2 as a head with 16
 * significant bits plus a rounded tail; exp(r) by the degree-7 Taylor polynomial in Horner
 * form; result p * 2^k from exponent bits; k < -125 gives +0; NaN returns itself.
 * LOG(s), s >= 1, +inf or NaN: s = 2^e f with f in [sqrt(1/2), sqrt(2)); log f by the atanh
 * series 2 (z + z^3/3 + ... + z^15/15), z = (f - 1)/(f + 1) (J.-M. Muller, Elementary
 * Functions); result e ln2_head + (e ln2_tail + log f); non-finite s returns itself.
 * The sweeps over bit-pattern ranges split the range over threads (each element's result
 * does not depend on the split).
 *
 * k = const[0..2]: 1/ln2, ln2 head, ln2 tail; const[3..10]: 1/n! for n = 0..7;
 * const[11]: sqrt 2; const[12..19]: 2/(2i+1) for i = 0..7.
 */
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}

static uint32_t to_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* t rounded to an integer, ties to even: adding and removing 1.5 * 2^23 leaves the integer
 * nearest t for |t| < 2^22 (the float sum has no fraction bits left); larger |t| are
 * integers already, and any t below -126 makes EXP +0 whatever its rounding. */
static float round_even(float t) {
  volatile float big = 12582912.0f;
  if (!(t > -4194304.0f && t < 4194304.0f)) return t;
  return (t + big) - big;
}

static float exp_one(float d, const float* k) {
  if (d != d) return d;
  const float t = d * k[0];
  const float kr = round_even(t);
  if (!(kr >= -125.0f)) return 0.0f;
  float r = d - kr * k[1];
  r = r - kr * k[2];
  float p = k[3 + 7];
  for (int n = 6; n >= 0; --n) p = p * r + k[3 + n];
  const int32_t ki = (int32_t)kr;
  return p * from_bits((uint32_t)(ki + 127) << 23);
}

static float log_one(float s, const float* k) {
  const uint32_t b = to_bits(s);
  if ((b & 0x7f800000u) == 0x7f800000u) return s;   /* inf or NaN */
  int32_t e = (int32_t)(b >> 23) - 127;
  float f = from_bits((b & 0x7fffffu) | 0x3f800000u);
  if (f > k[11]) {
    f = f * 0.5f;
    e += 1;
  }
  const float z = (f - 1.0f) / (f + 1.0f);
  const float w = z * z;
  float q = k[12 + 7];
  for (int i = 6; i >= 0; --i) q = q * w + k[12 + i];
  const float lf = z * q;
  const float ef = (float)e;
  return ef * k[1] + (ef * k[2] + lf);
}

/* out[i] = EXP / LOG of the float whose bit pattern is first + i, i < n. */
void oracle_exp_bits(uint32_t first, int64_t n, const float* k, float* out) {
#pragma omp parallel for schedule(static, 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = exp_one(from_bits(first + (uint32_t)i), k);
}

void oracle_log_bits(uint32_t first, int64_t n, const float* k, float* out) {
#pragma omp parallel for schedule(static, 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = log_one(from_bits(first + (uint32_t)i), k);
}

/* The same functions on given values. */
void oracle_exp(const float* x, int64_t n, const float* k, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = exp_one(x[i], k);
}

void oracle_log(const float* x, int64_t n, const float* k, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = log_one(x[i], k);
}
