/* Checks, on the host, the integer q of the page-pair decode kernels
 * (decode.hip, load_q_pieces) and the int32 sums built from it:
 *  - scaling: for every positive finite FP16 and BF16 head maximum m, the
 *    power of two 2^kq with kq = 22 - e (m = f 2^e, f in [0.5, 1)) puts
 *    rint(m 2^kq) in [2^21, 2^22], so every element's |qi| <= 2^22;
 *  - digits: for every qi in [-2^22, 2^22], the bytes of qi + 0x808080 taken
 *    with the kernel's byte-permute selectors (emulated below from the
 *    instruction's definition) and flipped in bit 7 give signed digits a, b,
 *    c in [-128, 127] with qi = 65536 a + 256 b + c, in the byte of the
 *    value's position;
 *  - sums: 256 B + C, with B and C sums over 128 dims of digit x code
 *    (|code| <= 127), stays inside int32 at the extremes (A is converted to
 *    float on its own).
 * Exit status 1 on any failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

/* V_PERM_B32: byte i of the result is selected by byte i of sel from the
 * eight bytes {src1 (bytes 0-3), src0 (bytes 4-7)}; selector 12 gives 0x00,
 * 13 and above 0xff (8-11 sign-replicate bytes, unused here). */
static uint32_t perm(uint32_t src0, uint32_t src1, uint32_t sel) {
  const uint64_t v = ((uint64_t)src0 << 32) | src1;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (sel >> (8 * i)) & 0xff;
    uint32_t b;
    if (s < 8)
      b = (uint32_t)(v >> (8 * s)) & 0xff;
    else if (s == 12)
      b = 0;
    else if (s >= 13)
      b = 0xff;
    else
      return 0xdeadbeef; /* not used by the kernel */
    r |= b << (8 * i);
  }
  return r;
}

static float from_f16(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int digit_word(const uint32_t u[4], uint32_t lo_sel, uint32_t hi_sel) {
  return (int)((perm(u[1], u[0], lo_sel) | perm(u[3], u[2], hi_sel)) ^ 0x80808080u);
}

int main(void) {
  long bad = 0, n = 0;
  /* scaling: every positive finite FP16 and BF16 maximum */
  for (int fmt = 0; fmt < 2; ++fmt)
    for (uint32_t h = 1; h < 0x7c00u || (fmt && h < 0x7f80u); ++h) {
      const float m = fmt ? from_bf16((uint16_t)h) : from_f16((uint16_t)h);
      int e;
      frexpf(m, &e);
      const float q = rintf(ldexpf(m, 22 - e));
      ++n;
      if (!(q >= 2097152.0f && q <= 4194304.0f)) {
        if (bad++ < 5) printf("scale: fmt %d bits %#x -> %g\n", fmt, h, q);
      }
    }
  /* digits: every value, in each of the four byte positions of a word */
  for (int qi = -4194304; qi <= 4194304; ++qi)
    for (int pos = 0; pos < 4; ++pos) {
      uint32_t u[4];
      for (int j = 0; j < 4; ++j) {
        const int other = (int)(((int64_t)qi * 7 + 3 * j + 11) % 4194305); /* neighbours */
        u[j] = (uint32_t)(j == pos ? qi : other) + 0x808080u;
      }
      const int wa = digit_word(u, 0x0c0c0602u, 0x06020c0cu);
      const int wb = digit_word(u, 0x0c0c0501u, 0x05010c0cu);
      const int wc = digit_word(u, 0x0c0c0400u, 0x04000c0cu);
      const int a = (int8_t)(wa >> (8 * pos)), b = (int8_t)(wb >> (8 * pos)),
                c = (int8_t)(wc >> (8 * pos));
      ++n;
      if (65536 * a + 256 * b + c != qi) {
        if (bad++ < 5) printf("digits: qi %d pos %d -> a %d b %d c %d\n", qi, pos, a, b, c);
      }
    }
  /* sums: the extremes of the two low digit sums over 128 dims */
  const int64_t bmax = 128LL * 128 * 127, cmax = 128LL * 128 * 127;
  if (256 * bmax + cmax > INT32_MAX) ++bad;
  printf("checked %ld, failed %ld\n", n, bad);
  return bad ? 1 : 0;
}
