/* Checks, on the host, the division-free arithmetic the per-token INT8
 * writer uses, against IEEE binary32 division:
 *  - the scale step: q0 = a * fl(1/127); fl32(a / 127) == fma(fma(-q0, 127,
 *    a), fl(1/127), q0) for every finite FP16 and BF16 magnitude a;
 *  - the code step: for FP16 scales s (every `stride`-th positive finite
 *    pattern, starting at `first`), every FP16 or BF16 x with |x| <= 127 s
 *    and a reciprocal r anywhere within one ulp of 1/s:
 *      q0 = fl(x r); q1 = fma(fma(-q0, s, x), r, q0)
 *    the low byte of the bits of q1 + 1.5 * 2^23 is
 *    clamp(rint(fl32(x / s)), -127, 127).
 * Usage: quant_formula f16|bf16 stride first. Prints the counts; exit
 * status 1 on any mismatch. Built with -ffp-contract=off so that every
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

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int bf = strcmp(argv[1], "bf16") == 0;
  const int stride = atoi(argv[2]), first = atoi(argv[3]);
  long long n = 0, bad = 0;

  const float r127 = 1.0f / 127.0f;
  for (int fmt = 0; fmt < 2; ++fmt)
    for (uint32_t b = 0; b < 0x8000; ++b) {
      const float a = fmt ? from_bf16((uint16_t)b) : from_f16((uint16_t)b);
      if (!isfinite(a)) continue;
      const float q0 = a * r127;
      const float q1 = fmaf(fmaf(-q0, 127.0f, a), r127, q0);
      ++n;
      if (q1 != a / 127.0f) ++bad;
    }
  printf("scale: %lld values, %lld mismatches\n", n, bad);

  const float magic = 12582912.0f;
  long long codes = 0, cbad = 0;
  for (uint32_t sb = (uint32_t)first; sb < 0x7c00; sb += (uint32_t)stride) {
    if (sb == 0) continue;
    const float s = from_f16((uint16_t)sb);
    const float r0 = 1.0f / s;
    const float rs[3] = {nextafterf(r0, 0.0f), r0, nextafterf(r0, INFINITY)};
    for (uint32_t xb = 0; xb < 0x10000; ++xb) {
      const float x = bf ? from_bf16((uint16_t)xb) : from_f16((uint16_t)xb);
      if (!(fabsf(x) <= 127.0f * s)) continue;
      const float q = fminf(fmaxf(rintf(x / s), -127.0f), 127.0f);
      const uint8_t want = (uint8_t)(int8_t)q;
      for (int k = 0; k < 3; ++k) {
        const float r = rs[k];
        const float q0 = x * r;
        const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
        ++codes;
        if ((uint8_t)(bits_of(q1 + magic) & 0xff) != want) ++cbad;
      }
    }
  }
  printf("codes: %lld checks, %lld mismatches\n", codes, cbad);
  return (bad || cbad) ? 1 : 0;
}
