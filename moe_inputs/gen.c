/* Seeded synthetic inputs for the expert-offload MoE layer step.
 *
 * This file holds no arithmetic of the method itself: it only draws numbers and
 * stores them in the byte formats the layer step reads (bf16 router weights and
 * activations; expert blobs in bf16, fp8-e4m3 with 1x128 fp32 scales, or
 * MXFP4).  Both the float64 oracle and the GPU path read exactly these bytes.
 *
 * Random numbers: fp32 standard normals from normals.c (Box-Muller on a
 * counter-based SplitMix64 stream).  A stream key is derived from (seed,
 * purpose, layer, unit, matrix), so every matrix element is addressable without
 * drawing its predecessors and pools fill in parallel.
 *
 * Purposes: 1 router, 2 routed expert, 3 shared expert, 4 decode activations,
 * 5 prefill activations.  Matrices within an expert: 0 gate, 1 up, 2 down.
 * Element index inside a matrix: Wg[i][h], Wu[i][h] -> i*H + h; Wd[h][i] -> h*I + i;
 * router Wr[e][h] -> e*H + h; decode noise e_t[h] -> t*H + h; prefill x[t][h] -> t*H + h.
 *
 * Expert blob layout (one (layer, expert) unit; the same bytes in the host pool
 * and in a GPU cache slot):
 *   bf16 : Wgu[I][2][H] bf16 (row i = gate row i, then up row i), WdT[I][H] bf16
 *          (row i = column i of Wd[H][I]).
 *   fp8  : Wgu codes [I][2][H], WdT codes [I][H] (OCP e4m3fn), then
 *          s_gu[I][2][H/128] fp32, then s_d[I/128][H] fp32.  One scale covers
 *          128 consecutive elements along the contraction dimension.
 *          s = max|w| / 448 (fp32), code = round-to-nearest-even(w / s), saturating.
 *   mxfp4: Wgu codes [I][2][H/2], WdT codes [I][H/2] (OCP e2m1, two per byte,
 *          even element in the low nibble), then s_gu[I][2][H/32] e8m0, then
 *          s_d[I/32][H] e8m0.  Per OCP MX v1.0: X = floor(log2 max|w|) - 2,
 *          code = round-to-nearest-even(w / 2^X) saturating at 6.
 * Weights are fp32 0.02 * N(0,1); bf16 values are round-to-nearest-even of them.
 * Activations: AR(1) x_0 = e_0, x_t = 0.8 x_{t-1} + 0.6 e_t with a float64 state,
 * stored as bf16 (RNE of the fp32 rounding of the state).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

void moe_in_normal_pairs(uint64_t key, uint64_t p0, uint64_t npairs, float* out);

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t moe_in_stream_key(uint64_t seed, uint32_t purpose, uint32_t layer, uint32_t unit,
                           uint32_t matrix) {
  uint64_t k = mix64(seed + GOLDEN);
  k = mix64(k ^ ((uint64_t)purpose + 2 * GOLDEN));
  k = mix64(k ^ ((uint64_t)layer + 3 * GOLDEN));
  k = mix64(k ^ ((uint64_t)unit + 4 * GOLDEN));
  k = mix64(k ^ ((uint64_t)matrix + 5 * GOLDEN));
  return k;
}

uint64_t moe_in_draw(uint64_t key, uint64_t j) { return mix64(key + (j + 1) * GOLDEN); }

/* fp32 normals [first, first + n) of a stream (any first, any n). */
static void normals_f32(uint64_t key, uint64_t first, uint64_t n, float* out) {
  if (n == 0) return;
  uint64_t p0 = first >> 1, p1 = (first + n + 1) >> 1;
  if ((first & 1) == 0 && ((first + n) & 1) == 0) {
    moe_in_normal_pairs(key, p0, p1 - p0, out);
    return;
  }
  float* tmp = (float*)malloc(sizeof(float) * 2 * (size_t)(p1 - p0));
  moe_in_normal_pairs(key, p0, p1 - p0, tmp);
  memcpy(out, tmp + (first & 1), sizeof(float) * (size_t)n);
  free(tmp);
}

void moe_in_normals(uint64_t key, uint64_t first, uint64_t n, double* out) {
  float* f = (float*)malloc(sizeof(float) * (size_t)(n ? n : 1));
  normals_f32(key, first, n, f);
  for (uint64_t j = 0; j < n; ++j) out[j] = f[j];
  free(f);
}

static inline uint32_t fbits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static inline uint16_t f32_to_bf16(float f) {
  uint32_t u = fbits(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP e4m3fn: round-to-nearest-even, saturating at +-448. */
static inline uint8_t enc_e4m3(float x) {
  uint32_t u = fbits(x);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  u &= 0x7fffffffu;
  if (u >= 0x43e00000u) return sign | 0x7e; /* |x| >= 448 */
  if (u < 0x3c800000u) {                    /* |x| < 2^-6: subnormal step 2^-9 */
    float a;
    memcpy(&a, &u, 4);
    long m = lrintf(a * 512.0f);
    return sign | (uint8_t)m; /* m == 8 encodes 2^-6 as exponent 1, mantissa 0 */
  }
  uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;
  int code = (int)r - (120 << 3);
  if (code > 0x7e) code = 0x7e;
  return sign | (uint8_t)code;
}

/* OCP e2m1: round-to-nearest-even, saturating at +-6.  Returns a 4-bit code. */
static inline uint8_t enc_e2m1(float v) {
  uint32_t u = fbits(v);
  uint8_t sign = (uint8_t)((u >> 28) & 0x8);
  u &= 0x7fffffffu;
  if (u < 0x3f800000u) { /* |v| < 1: subnormal step 0.5 */
    float a;
    memcpy(&a, &u, 4);
    return sign | (uint8_t)lrintf(a * 2.0f); /* 2 encodes 1.0 */
  }
  if (u >= 0x40e00000u) return sign | 7; /* |v| >= 7 */
  uint32_t r = (u + 0x1fffffu + ((u >> 22) & 1u)) >> 22;
  int code = (int)r - 252;
  if (code > 7) code = 7;
  return sign | (uint8_t)code;
}

uint8_t moe_in_enc_e4m3(float x) { return enc_e4m3(x); }
uint8_t moe_in_enc_e2m1(float v) { return enc_e2m1(v); }

int64_t moe_in_blob_bytes(int fmt, int64_t H, int64_t I) {
  if (fmt == 0) return 6 * I * H;
  if (fmt == 1) return 3 * I * H + 4 * (2 * I * (H / 128)) + 4 * ((I / 128) * H);
  if (fmt == 2) return 3 * I * H / 2 + 2 * I * (H / 32) + (I / 32) * H;
  return -1;
}

/* fp32 weights of one expert before encoding: Wg[I][H], Wu[I][H], Wd[H][I]. */
void moe_in_expert_f32(uint64_t seed, uint32_t purpose, uint32_t layer, uint32_t unit, int64_t H,
                       int64_t I, float* Wg, float* Wu, float* Wd) {
  float* dst[3] = {Wg, Wu, Wd};
  for (int m = 0; m < 3; ++m) {
    uint64_t key = moe_in_stream_key(seed, purpose, layer, unit, (uint32_t)m);
    normals_f32(key, 0, (uint64_t)(H * I), dst[m]);
    for (int64_t j = 0; j < H * I; ++j) dst[m][j] = 0.02f * dst[m][j];
  }
}

/* Branch-free array encoders (vectorisable).  Both round to nearest even. */
static void enc_e4m3_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) {
    uint32_t u = fbits(v[j]);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    uint32_t rn = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - 960u;
    float af;
    memcpy(&af, &a, 4);
    uint32_t sub = fbits(af * 512.0f + 12582912.0f) - 0x4b400000u; /* RNE(|v| * 2^9) */
    uint32_t code = a < 0x3c800000u ? sub : rn;
    code = code > 0x7eu ? 0x7eu : code;
    out[j] = (uint8_t)(sign | code);
  }
}

static void enc_e2m1_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) {
    uint32_t u = fbits(v[j]);
    uint32_t sign = (u >> 28) & 0x8u;
    uint32_t a = u & 0x7fffffffu;
    uint32_t rn = ((a + 0x1fffffu + ((a >> 22) & 1u)) >> 22) - 252u;
    float af;
    memcpy(&af, &a, 4);
    uint32_t sub = fbits(af * 2.0f + 12582912.0f) - 0x4b400000u; /* RNE(|v| * 2) */
    uint32_t code = a < 0x3f800000u ? sub : rn;
    code = code > 7u ? 7u : code;
    out[j] = (uint8_t)(sign | code);
  }
}

static inline uint8_t mx_scale_code(float amax) {
  if (amax == 0.f) return 0;
  int eb = (int)((fbits(amax) >> 23) & 0xff); /* biased exponent: floor(log2) + 127 for normals */
  int c = eb - 2;
  if (c < 0) c = 0;
  if (c > 254) c = 254;
  return (uint8_t)c;
}

static inline float pow2f(int e) { /* 2^e for -126 <= e <= 127 */
  uint32_t u = (uint32_t)(e + 127) << 23;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Encode n values (contraction along the array, n a multiple of the block) in
 * place of codes: fp8 codes + fp32 scales per 128, or e2m1 codes (one per byte,
 * unpacked) + e8m0 scales per 32.  tmp holds n floats. */
static void encode_run(int fmt, const float* w, int64_t n, float* tmp, uint8_t* codes,
                       void* scales) {
  if (fmt == 1) {
    float* sc = (float*)scales;
    for (int64_t b = 0; b < n / 128; ++b) {
      float amax = 0.f;
      for (int j = 0; j < 128; ++j) amax = fmaxf(amax, fabsf(w[b * 128 + j]));
      float s = amax > 0.f ? amax / 448.0f : 1.0f;
      sc[b] = s;
      for (int j = 0; j < 128; ++j) tmp[b * 128 + j] = w[b * 128 + j] / s;
    }
    enc_e4m3_array(tmp, n, codes);
  } else {
    uint8_t* sc = (uint8_t*)scales;
    for (int64_t b = 0; b < n / 32; ++b) {
      float amax = 0.f;
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(w[b * 32 + j]));
      uint8_t c = mx_scale_code(amax);
      sc[b] = c;
      float inv = pow2f(127 - (int)c);
      for (int j = 0; j < 32; ++j) tmp[b * 32 + j] = w[b * 32 + j] * inv;
    }
    enc_e2m1_array(tmp, n, codes);
  }
}

#define TILE 16

/* Generate one expert blob (routed expert when purpose == 2, shared when 3). */
void moe_in_expert_blob(uint64_t seed, int fmt, uint32_t purpose, uint32_t layer, uint32_t unit,
                        int64_t H, int64_t I, uint8_t* blob) {
  int64_t mx = H > I ? H : I;
  float* row = (float*)malloc(sizeof(float) * (size_t)mx * TILE);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)mx * TILE);
  uint8_t* codes = (uint8_t*)malloc((size_t)mx * TILE);
  float* fsc = (float*)malloc(sizeof(float) * (size_t)(mx / 32 + 1) * TILE);
  uint8_t* bsc = (uint8_t*)malloc((size_t)(mx / 32 + 1) * TILE);
  uint64_t kg = moe_in_stream_key(seed, purpose, layer, unit, 0);
  uint64_t ku = moe_in_stream_key(seed, purpose, layer, unit, 1);
  uint64_t kd = moe_in_stream_key(seed, purpose, layer, unit, 2);

  /* gate and up rows: contraction along H */
  for (int64_t i = 0; i < I; ++i) {
    for (int g = 0; g < 2; ++g) {
      normals_f32(g == 0 ? kg : ku, (uint64_t)(i * H), (uint64_t)H, row);
      for (int64_t h = 0; h < H; ++h) row[h] *= 0.02f;
      int64_t r = i * 2 + g;
      if (fmt == 0) {
        uint16_t* W = (uint16_t*)blob + r * H;
        for (int64_t h = 0; h < H; ++h) W[h] = f32_to_bf16(row[h]);
      } else if (fmt == 1) {
        float* S = (float*)(blob + 3 * I * H) + r * (H / 128);
        encode_run(1, row, H, tmp, blob + r * H, S);
      } else {
        uint8_t* W = blob + r * (H / 2);
        encode_run(2, row, H, tmp, codes, blob + 3 * I * H / 2 + r * (H / 32));
        for (int64_t h = 0; h < H; h += 2) W[h / 2] = (uint8_t)(codes[h] | (codes[h + 1] << 4));
      }
    }
  }
  /* down projection Wd[H][I]: contraction along I; stored transposed WdT[I][H].
   * Rows h are produced TILE at a time so the transposed writes are contiguous runs. */
  for (int64_t h0 = 0; h0 < H; h0 += TILE) {
    int64_t nh = H - h0 < TILE ? H - h0 : TILE;
    normals_f32(kd, (uint64_t)(h0 * I), (uint64_t)(nh * I), row); /* row[(h-h0)*I + i] */
    for (int64_t j = 0; j < nh * I; ++j) row[j] *= 0.02f;
    if (fmt == 0) {
      uint16_t* W = (uint16_t*)(blob + 4 * I * H);
      for (int64_t i = 0; i < I; ++i)
        for (int64_t hh = 0; hh < nh; ++hh) W[i * H + h0 + hh] = f32_to_bf16(row[hh * I + i]);
    } else if (fmt == 1) {
      uint8_t* W = blob + 2 * I * H;
      float* S = (float*)(blob + 3 * I * H + 4 * (2 * I * (H / 128)));
      for (int64_t hh = 0; hh < nh; ++hh) {
        encode_run(1, row + hh * I, I, tmp, codes + hh * I, fsc + hh * (I / 128));
        for (int64_t b = 0; b < I / 128; ++b) S[b * H + h0 + hh] = fsc[hh * (I / 128) + b];
      }
      for (int64_t i = 0; i < I; ++i)
        for (int64_t hh = 0; hh < nh; ++hh) W[i * H + h0 + hh] = codes[hh * I + i];
    } else {
      uint8_t* W = blob + I * H;
      uint8_t* S = blob + 3 * I * H / 2 + 2 * I * (H / 32);
      for (int64_t hh = 0; hh < nh; ++hh) {
        encode_run(2, row + hh * I, I, tmp, codes + hh * I, bsc + hh * (I / 32));
        for (int64_t b = 0; b < I / 32; ++b) S[b * H + h0 + hh] = bsc[hh * (I / 32) + b];
      }
      for (int64_t i = 0; i < I; ++i)
        for (int64_t hh = 0; hh < nh; hh += 2)
          W[i * (H / 2) + (h0 + hh) / 2] = (uint8_t)(codes[hh * I + i] | (codes[(hh + 1) * I + i] << 4));
    }
  }
  free(row);
  free(tmp);
  free(codes);
  free(fsc);
  free(bsc);
}

/* Routed-expert pool: blobs for layers [l0, l0+nl) x experts [0,E), each blob_bytes
 * long, in (layer, expert) order starting at pool.  Threads: nthreads (0 = all). */
void moe_in_pool(uint64_t seed, int fmt, int64_t l0, int64_t nl, int64_t E, int64_t H, int64_t I,
                 uint8_t* pool, int nthreads) {
  int64_t S = moe_in_blob_bytes(fmt, H, I);
  int64_t n = nl * E;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t b = 0; b < n; ++b) {
    int64_t l = l0 + b / E, e = b % E;
    moe_in_expert_blob(seed, fmt, 2, (uint32_t)l, (uint32_t)e, H, I, pool + b * S);
  }
}

/* Router weights Wr[E][H] bf16 for layers [l0, l0+nl), layer-major. */
void moe_in_router(uint64_t seed, int64_t l0, int64_t nl, int64_t E, int64_t H, uint16_t* out,
                   int nthreads) {
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t l = 0; l < nl; ++l) {
    float* row = (float*)malloc(sizeof(float) * (size_t)(E * H));
    uint64_t key = moe_in_stream_key(seed, 1, (uint32_t)(l0 + l), 0, 0);
    normals_f32(key, 0, (uint64_t)(E * H), row);
    for (int64_t j = 0; j < E * H; ++j) out[l * E * H + j] = f32_to_bf16(0.02f * row[j]);
    free(row);
  }
}

/* Decode activations: for each layer l in [l0, l0+nl) and stream s in [0, S), the AR(1)
 * sequence over token steps t in [0, ntok), stored as bf16 at
 * out[((t * nl + (l - l0)) * S + s) * H + h]. */
void moe_in_decode_acts(uint64_t seed, int64_t l0, int64_t nl, int64_t S, int64_t ntok, int64_t H,
                        uint16_t* out, int nthreads) {
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t ls = 0; ls < nl * S; ++ls) {
    int64_t l = ls / S, s = ls % S;
    uint64_t key = moe_in_stream_key(seed, 4, (uint32_t)(l0 + l), (uint32_t)s, 0);
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    float* e = (float*)malloc(sizeof(float) * (size_t)H);
    for (int64_t t = 0; t < ntok; ++t) {
      normals_f32(key, (uint64_t)(t * H), (uint64_t)H, e);
      for (int64_t h = 0; h < H; ++h) x[h] = (t == 0) ? (double)e[h] : 0.8 * x[h] + 0.6 * (double)e[h];
      uint16_t* o = out + ((t * nl + l) * S + s) * H;
      for (int64_t h = 0; h < H; ++h) o[h] = f32_to_bf16((float)x[h]);
    }
    free(x);
    free(e);
  }
}

/* Prefill activations: i.i.d. N(0,1) as bf16, out[(l - l0) * T * H + t * H + h]. */
void moe_in_prefill_acts(uint64_t seed, int64_t l0, int64_t nl, int64_t T, int64_t H,
                         uint16_t* out, int nthreads) {
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int64_t chunk = 256;
  int64_t nchunks = (T + chunk - 1) / chunk;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t c = 0; c < nl * nchunks; ++c) {
    int64_t l = c / nchunks, t0 = (c % nchunks) * chunk;
    int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
    uint64_t key = moe_in_stream_key(seed, 5, (uint32_t)(l0 + l), 0, 0);
    float* e = (float*)malloc(sizeof(float) * (size_t)((t1 - t0) * H));
    normals_f32(key, (uint64_t)(t0 * H), (uint64_t)((t1 - t0) * H), e);
    uint16_t* o = out + l * T * H + t0 * H;
    for (int64_t j = 0; j < (t1 - t0) * H; ++j) o[j] = f32_to_bf16(e[j]);
    free(e);
  }
}
