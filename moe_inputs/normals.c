/* Standard normal draws for the seeded input generator (see gen.c).
 *
 * Box-Muller transform on a counter-based SplitMix64 stream: draw j of the
 * stream with key K is mix64(K + (j + 1) * golden) (Steele, Lea and Flood,
 * OOPSLA 2014); its upper and lower 32-bit halves give u1, u2 in (0, 1), and
 * normals 2j, 2j+1 are sqrt(-2 ln u1) * cos(2 pi u2) and * sin(2 pi u2), in fp32.
 * Built with -ffast-math and AVX2 so the transcendental calls vectorise through
 * glibc's libmvec; the result only feeds bf16, fp8 and fp4 encodings.  Every
 * pair goes through the same full-width vector loop (blocks are always computed
 * whole and the unused tail discarded), so a normal's value does not depend on
 * which call produced it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL
#define BLK 256

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static void block(uint64_t key, uint64_t p, float* out /* 2*BLK */) {
  float u1[BLK] __attribute__((aligned(64))), u2[BLK] __attribute__((aligned(64)));
  float rad[BLK] __attribute__((aligned(64))), ang[BLK] __attribute__((aligned(64)));
  float c[BLK] __attribute__((aligned(64))), s[BLK] __attribute__((aligned(64)));
  for (int j = 0; j < BLK; ++j) {
    uint64_t r = mix64(key + (p + (uint64_t)j + 1) * GOLDEN);
    u1[j] = ((float)(uint32_t)(r >> 32) + 0.5f) * 0x1p-32f;
    u2[j] = ((float)(uint32_t)(r & 0xffffffffu) + 0.5f) * 0x1p-32f;
  }
  for (int j = 0; j < BLK; ++j) {
    float v = u1[j] < 1.0f ? u1[j] : 0x1.fffffep-1f;
    rad[j] = sqrtf(-2.0f * logf(v));
    ang[j] = 6.28318530717958647692f * u2[j];
  }
  for (int j = 0; j < BLK; ++j) c[j] = cosf(ang[j]);
  for (int j = 0; j < BLK; ++j) s[j] = sinf(ang[j]);
  for (int j = 0; j < BLK; ++j) {
    out[2 * j] = rad[j] * c[j];
    out[2 * j + 1] = rad[j] * s[j];
  }
}

/* Normals with indices [2*p0, 2*p0 + 2*npairs) of the stream into out. */
void moe_in_normal_pairs(uint64_t key, uint64_t p0, uint64_t npairs, float* out) {
  float buf[2 * BLK] __attribute__((aligned(64)));
  for (uint64_t b = 0; b < npairs; b += BLK) {
    uint64_t n = (npairs - b) < BLK ? (npairs - b) : BLK;
    if (n == BLK) {
      block(key, p0 + b, out + 2 * b);
    } else {
      block(key, p0 + b, buf);
      memcpy(out + 2 * b, buf, sizeof(float) * 2 * n);
    }
  }
}
