/* Checks, on the host, the division-free arithmetic of the static-scale INT8
 * writer against the division-based rule, for every FP16 or BF16 input x
 * (finite, infinite and NaN) and a set of binary32 scales s inside the
 * writer's window [2^-64, 2^64]:
 *    rule:   code = clamp(rint(fl32(x / s)), -127, 127), the clamp ignoring
 *            a NaN operand as the GPU's fmaxf / fminf do (a NaN gives -127);
 *    writer: r = fl(1 / s); q0 = med3(fl(x r), -128, 128);
 *            q1 = fma(fma(-q0, s, x), r, q0);
 *            code = low byte of the bits of med3(q1, -127, 127) + 1.5 * 2^23,
 *            med3 being the hardware's median of three, which for a NaN
 *            operand gives the minimum of the other two (V_MED3_F32 on a quiet
 *            NaN; every NaN here is the quiet result of a product or an fma).
 * Scales: every power of two in the window, the all-ones significand at every
 * exponent, the window's ends, and `count` seeded random significands and
 * exponents. Usage: static_formula f16|bf16 count seed. Prints the counts;
 * exit status 1 on any mismatch. Built with -ffp-contract=off so that every
 * product and sum rounds where it is written. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_f16(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* xorshift64: a seeded stream of scale patterns */
static uint64_t rng_state;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

/* max / min with the NaN rule of the GPU code's fmaxf / fminf (LLVM
 * maxnum / minnum, any NaN operand, quiet or signaling, is ignored); the
 * host library's fmaxf instead returns NaN for a signaling NaN. */
static float maxnum(float a, float b) { return isnan(a) ? b : isnan(b) ? a : fmaxf(a, b); }
static float minnum(float a, float b) { return isnan(a) ? b : isnan(b) ? a : fminf(a, b); }

/* median of three with a NaN first operand giving the smaller bound */
static float med3(float x, float lo, float hi) { return isnan(x) ? lo : fminf(fmaxf(x, lo), hi); }

static long long checks, bad;

static void check_scale(int bf, float s) {
  const float magic = 12582912.0f;
  const float r = 1.0f / s;
  for (uint32_t xb = 0; xb < 0x10000; ++xb) {
    const float x = bf ? from_bf16((uint16_t)xb) : from_f16((uint16_t)xb);
    const float q = minnum(maxnum(rintf(x / s), -127.0f), 127.0f);
    const uint8_t want = (uint8_t)(int8_t)q;
    const float q0 = med3(x * r, -128.0f, 128.0f);
    const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
    const float t = med3(q1, -127.0f, 127.0f) + magic;
    ++checks;
    if ((uint8_t)(bits_of(t) & 0xff) != want) {
      if (bad < 10) printf("mismatch: s=%a x=%a want %d\n", s, x, (int)(int8_t)want);
      ++bad;
    }
  }
}

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int bf = strcmp(argv[1], "bf16") == 0;
  const long count = atol(argv[2]);
  rng_state = (uint64_t)atoll(argv[3]) * 0x9E3779B97F4A7C15ull + 1;
  long scales = 0;
  for (int e = -64; e <= 64; ++e) {
    check_scale(bf, ldexpf(1.0f, e));
    ++scales;
    if (e < 64) {
      check_scale(bf, ldexpf(1.0f, e) * from_bits(0x3FFFFFFFu));  /* 2^e * (2 - 2^-23) */
      ++scales;
    }
  }
  for (long i = 0; i < count; ++i) {
    const uint64_t u = next_u64();
    const int e = (int)(u % 128) - 64;               /* exponent in [-64, 63] */
    const uint32_t m = (uint32_t)(u >> 32) & 0x7FFFFFu;
    check_scale(bf, ldexpf(from_bits(0x3F800000u | m), e));
    ++scales;
  }
  printf("static codes: %ld scales, %lld checks, %lld mismatches\n", scales, checks, bad);
  return bad ? 1 : 0;
}
