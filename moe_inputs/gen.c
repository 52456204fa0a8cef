/*
 * Seeded synthetic inputs for one sparse MoE FFN layer.
 *
 * This file produces the bytes that both the HIP path and the CPU oracle
 * consume: activations, router weights and expert weights.  It holds none of
 * the layer's arithmetic (no router, no dequantisation, no SwiGLU, no combine).
 *
 *   - Every element is a pure function of (seed, tensor id, flat index):
 *     a SplitMix64 finaliser over a Weyl counter gives 64 random bits, two
 *     such draws give two uniforms and the Box-Muller transform turns the pair
 *     into two normals (even index -> cosine branch, odd index -> sine branch).
 *     Any element can therefore be regenerated on any core in any order.
 *   - Weight groups are quantised with a min-max affine quantiser: scale =
 *     fp16((max-min)/(2^bits-1)), bias = fp16(min), q = clamp(rint((w-bias)/scale)).
 *     4-bit codes are packed two per byte, the even column in the low nibble.
 *   - NVFP4 blocks of 16 columns: block scale = E4M3(amax / (6 ts)) with the
 *     tensor scale ts given, codes = nearest E2M1 value of w / (ts * scale);
 *     E2M1 codes are packed as 4-bit codes.
 *   - Zipf-skewed routing is planted into activations by adding a multiple of
 *     the chosen experts' router rows (see gen_planted_x).
 *
 * fp16 and bf16 values are produced with round-to-nearest-even from fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- RNG --- */

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t tid) {
  return mix64(seed * 0x9E3779B97F4A7C15ULL + ((uint64_t)tid << 32) + 0x632BE59BD9B4E019ULL);
}

static inline uint64_t draw_bits(uint64_t key, uint64_t ctr) {
  return mix64(key + (ctr + 1) * 0x9E3779B97F4A7C15ULL);
}

/* uniform on the open interval (0, 1) */
static inline double u01(uint64_t b) { return ((double)(b >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* both normals of Box-Muller pair j: elements 2j (cosine) and 2j+1 (sine) */
static inline void normal_pair(uint64_t key, uint64_t j, double* c, double* s) {
  double u1 = u01(draw_bits(key, 2 * j));
  double u2 = u01(draw_bits(key, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925 * u2;
  *c = r * cos(th);
  *s = r * sin(th);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  double c, s;
  normal_pair(key, i >> 1, &c, &s);
  return (i & 1) ? s : c;
}

/* ------------------------------------------------------ fp16 / bf16 ---- */

static uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
  if (ax < 0x38800000u) {                                    /* below 2^-14: subnormal */
    float v;
    memcpy(&v, &ax, 4);
    float r = nearbyintf(v * 16777216.0f); /* exact scaling by 2^24, then RNE */
    return (uint16_t)(sign | (uint32_t)r);
  }
  uint32_t e = (ax >> 23) - 127 + 15;
  uint32_t m = ax & 0x7FFFFFu;
  uint32_t h = (e << 10) | (m >> 13);
  uint32_t rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

static uint16_t f32_to_bf16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7FFFu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

static double f16_bits_to_double(uint16_t h) {
  int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

static double bf16_bits_to_double(uint16_t h) {
  uint32_t x = (uint32_t)h << 16;
  float f;
  memcpy(&f, &x, 4);
  return (double)f;
}

/* dtype codes: 1 = fp16, 2 = bf16 */
static inline uint16_t round_to(double v, int dtype) {
  return dtype == 2 ? f32_to_bf16_bits((float)v) : f32_to_f16_bits((float)v);
}

static inline double decode(uint16_t b, int dtype) {
  return dtype == 2 ? bf16_bits_to_double(b) : f16_bits_to_double(b);
}

/* -------------------------------------------------------- exported ---- */

void gen_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* n normals with standard deviation sigma, elements [start, start+n) of the stream */
void gen_normal_f64(uint64_t seed, uint32_t tid, int64_t start, int64_t n, double sigma, double* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sigma * normal_at(key, (uint64_t)(start + i));
}

/* the same draws, rounded to fp16 (dtype 1) or bf16 (dtype 2) */
void gen_normal_half(uint64_t seed, uint32_t tid, int64_t start, int64_t n, double sigma, int dtype,
                     uint16_t* out) {
  uint64_t key = stream_key(seed, tid);
  if ((start & 1) == 0 && (n & 1) == 0) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i += 2) {
      double c, s;
      normal_pair(key, (uint64_t)(start + i) >> 1, &c, &s);
      out[i] = round_to(sigma * c, dtype);
      out[i + 1] = round_to(sigma * s, dtype);
    }
    return;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = round_to(sigma * normal_at(key, (uint64_t)(start + i)), dtype);
}

/* n uniforms on (0,1) */
void gen_uniform(uint64_t seed, uint32_t tid, int64_t start, int64_t n, double* out) {
  uint64_t key = stream_key(seed, tid);
  for (int64_t i = 0; i < n; ++i) out[i] = u01(draw_bits(key, (uint64_t)(start + i)));
}

/* round an fp64 array to fp16/bf16 bits (RNE through fp32) */
void gen_round_half(const double* v, int64_t n, int dtype, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = round_to(v[i], dtype);
}

/* decode fp16/bf16 bits to fp64 */
void gen_decode_half(const uint16_t* b, int64_t n, int dtype, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = decode(b[i], dtype);
}

/*
 * Quantise one group of `gs` values to `bits` with the min-max affine rule.
 * Writes codes (unpacked, one per byte) and the fp16 scale/bias bits.
 */
static void quant_group(const double* w, int gs, int bits, uint8_t* codes, uint16_t* s_bits, uint16_t* b_bits) {
  double lo = w[0], hi = w[0];
  for (int i = 1; i < gs; ++i) {
    if (w[i] < lo) lo = w[i];
    if (w[i] > hi) hi = w[i];
  }
  int qmax = (1 << bits) - 1;
  uint16_t sb = f32_to_f16_bits((float)((hi - lo) / qmax));
  uint16_t bb = f32_to_f16_bits((float)lo);
  double s = f16_bits_to_double(sb), b = f16_bits_to_double(bb);
  for (int i = 0; i < gs; ++i) {
    int q = 0;
    if (s > 0) {
      double r = nearbyint((w[i] - b) / s);
      q = r < 0 ? 0 : (r > qmax ? qmax : (int)r);
    }
    codes[i] = (uint8_t)q;
  }
  *s_bits = sb;
  *b_bits = bb;
}

/*
 * Store one group's codes at column offset `col` of a row.  bits 4: two per
 * byte, low nibble = even column; bits 5 and 6: a little-endian bit stream,
 * code i of the row at bits b*i .. b*i+b-1 (byte b*i/8, shifted by b*i%8,
 * spilling into the next byte; b = bits); bits 8: one per byte.  dst must
 * start zeroed for bits 5 and 6.
 */
static void store_codes(const uint8_t* codes, int gs, int bits, int64_t col, uint8_t* dst) {
  if (bits == 4) {
    for (int i = 0; i < gs; i += 2) dst[(col + i) / 2] = (uint8_t)(codes[i] | (codes[i + 1] << 4));
  } else if (bits == 5 || bits == 6) {
    for (int i = 0; i < gs; ++i) {
      int64_t bit = (int64_t)bits * (col + i);
      int sh = (int)(bit % 8);
      dst[bit / 8] |= (uint8_t)(codes[i] << sh);
      if (sh + bits > 8) dst[bit / 8 + 1] |= (uint8_t)(codes[i] >> (8 - sh));
    }
  } else {
    memcpy(dst + col, codes, (size_t)gs);
  }
}

/* quantise an explicit fp64 matrix [rows, K] (test helper, same rule as below) */
void gen_quantize_rows(const double* w, int64_t rows, int K, int bits, int gs, uint8_t* q, uint16_t* scales,
                       uint16_t* biases) {
  int64_t row_bytes = (int64_t)K * bits / 8;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t codes[256];
    memset(q + r * row_bytes, 0, (size_t)row_bytes);
    for (int g = 0; g < K / gs; ++g) {
      quant_group(w + r * K + (int64_t)g * gs, gs, bits, codes, &scales[r * (K / gs) + g], &biases[r * (K / gs) + g]);
      store_codes(codes, gs, bits, (int64_t)g * gs, q + r * row_bytes);
    }
  }
}

/*
 * Draw an expert weight tensor [E, N, K] of N(0, sigma) values (flat index
 * (e*N + n)*K + k of stream `tid`) and quantise it by groups of `gs` columns.
 *   q:      bits == 4: [E, N, K/2] bytes, low nibble = even column;
 *           bits == 5: [E, N, 5K/8] bytes, a little-endian 5-bit stream per row;
 *           bits == 6: [E, N, 3K/4] bytes, a little-endian 6-bit stream per row;
 *           bits == 8: [E, N, K] bytes
 *   scales, biases: [E, N, K/gs] fp16 bits
 */
void gen_quant_weights(uint64_t seed, uint32_t tid, int E, int N, int K, int bits, int gs, double sigma, uint8_t* q,
                       uint16_t* scales, uint16_t* biases) {
  uint64_t key = stream_key(seed, tid);
  int64_t rows = (int64_t)E * N;
  int64_t row_bytes = (int64_t)K * bits / 8;
  int ng = K / gs;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < rows; ++r) {
    double w[256];
    uint8_t codes[256];
    for (int g = 0; g < ng; ++g) {
      uint64_t base = (uint64_t)(r * K + (int64_t)g * gs); /* even, since gs and K are even */
      for (int i = 0; i < gs; i += 2) {
        double c, sn;
        normal_pair(key, (base + (uint64_t)i) >> 1, &c, &sn);
        w[i] = sigma * c;
        w[i + 1] = sigma * sn;
      }
      if (g == 0) memset(q + r * row_bytes, 0, (size_t)row_bytes);
      quant_group(w, gs, bits, codes, &scales[r * ng + g], &biases[r * ng + g]);
      store_codes(codes, gs, bits, (int64_t)g * gs, q + r * row_bytes);
    }
  }
}

/* ------------------------------------------------------ NVFP4 quantiser -- */

/* value of an FP8 E4M3 byte (OCP "fn": bias 7, subnormals m * 2^-9, 448 max) */
static double e4m3_value(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (b & 0x80) ? -v : v;
}

/* nearest E4M3 byte to v >= 0, ties to even mantissa, saturating at 448 */
static uint8_t e4m3_round(double v) {
  if (!(v > 0)) return 0;
  if (v >= 448.0) return 0x7E;
  int e2;
  frexp(v, &e2);
  int E = e2 - 1; /* v in [2^E, 2^(E+1)) */
  if (E < -6) E = -6; /* below 2^-6: the subnormal step 2^-9 */
  double m = nearbyint(ldexp(v, 3 - E)); /* default rounding: ties to even */
  if (m >= 16) {
    m = 8;
    E += 1;
  }
  int code = m < 8 ? (int)m : ((E + 7) << 3) | ((int)m - 8);
  return (uint8_t)(code > 0x7E ? 0x7E : code);
}

/* nearest E2M1 code (sign in bit 3) to r, ties to even mantissa, saturating at 6 */
static uint8_t e2m1_round(double r) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double a = fabs(r);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double d = fabs(a - mag[c]), db = fabs(a - mag[best]);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)(best == 0 ? 0 : (r < 0 ? 8 | best : best));
}

/* one block of 16 values: block scale = E4M3(amax / (6 ts)), codes = E2M1(w / (ts * scale)) */
static void quant_block_nvfp4(const double* w, double ts, uint8_t* codes, uint8_t* s_byte) {
  double amax = 0;
  for (int i = 0; i < 16; ++i)
    if (fabs(w[i]) > amax) amax = fabs(w[i]);
  uint8_t sb = e4m3_round(amax / (6.0 * ts));
  double step = ts * e4m3_value(sb);
  for (int i = 0; i < 16; ++i) codes[i] = step > 0 ? e2m1_round(w[i] / step) : 0;
  *s_byte = sb;
}

/* quantise an explicit fp64 matrix [rows, K] to NVFP4 with tensor scale ts */
void gen_quantize_rows_nvfp4(const double* w, int64_t rows, int K, double ts, uint8_t* q, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t codes[16];
    for (int g = 0; g < K / 16; ++g) {
      quant_block_nvfp4(w + r * K + (int64_t)g * 16, ts, codes, &scales[r * (K / 16) + g]);
      store_codes(codes, 16, 4, (int64_t)g * 16, q + r * (K / 2));
    }
  }
}

/*
 * Draw an expert weight tensor [E, N, K] of N(0, sigma) values (the same
 * streams and indices as gen_quant_weights) and quantise it to NVFP4 with
 * tensor scale ts: q [E, N, K/2] (two E2M1 codes per byte, low nibble = even
 * column), scales [E, N, K/16] E4M3 bytes.
 */
void gen_quant_nvfp4(uint64_t seed, uint32_t tid, int E, int N, int K, double sigma, double ts, uint8_t* q,
                     uint8_t* scales) {
  uint64_t key = stream_key(seed, tid);
  int64_t rows = (int64_t)E * N;
  int nb = K / 16;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < rows; ++r) {
    double w[16];
    uint8_t codes[16];
    for (int g = 0; g < nb; ++g) {
      uint64_t base = (uint64_t)(r * K + (int64_t)g * 16);
      for (int i = 0; i < 16; i += 2) {
        double c, sn;
        normal_pair(key, (base + (uint64_t)i) >> 1, &c, &sn);
        w[i] = sigma * c;
        w[i + 1] = sigma * sn;
      }
      quant_block_nvfp4(w, ts, codes, &scales[r * nb + g]);
      store_codes(codes, 16, 4, (int64_t)g * 16, q + r * (K / 2));
    }
  }
}

/*
 * Zipf-skewed expert sets for tokens [t0, t0+T): k distinct experts drawn without
 * replacement with P(rank r) proportional to r^-s over a seeded permutation of
 * the E experts (Fisher-Yates, stream 7); draws use stream 5.
 */
void gen_zipf_sets(uint64_t seed, int64_t t0, int T, int E, int k, double s, int32_t* sets) {
  uint64_t kperm = stream_key(seed, 7), kdraw = stream_key(seed, 5);
  int* perm = (int*)malloc(sizeof(int) * (size_t)E);
  double* pw = (double*)malloc(sizeof(double) * (size_t)E);
  for (int i = 0; i < E; ++i) perm[i] = i;
  for (int i = E - 1; i > 0; --i) {
    int j = (int)(u01(draw_bits(kperm, (uint64_t)i)) * (i + 1));
    if (j > i) j = i;
    int t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  for (int r = 0; r < E; ++r) pw[r] = pow((double)(r + 1), -s);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    uint8_t taken[256];
    memset(taken, 0, sizeof(taken));
    for (int j = 0; j < k; ++j) {
      double tot = 0;
      for (int r = 0; r < E; ++r)
        if (!taken[r]) tot += pw[r];
      double u = u01(draw_bits(kdraw, (uint64_t)(t0 + t) * 16 + (uint64_t)j)) * tot;
      int pick = -1;
      double c = 0;
      for (int r = 0; r < E; ++r) {
        if (taken[r]) continue;
        pick = r;
        c += pw[r];
        if (u < c) break;
      }
      taken[pick] = 1;
      sets[(int64_t)t * k + j] = perm[pick];
    }
  }
  free(perm);
  free(pw);
}

/*
 * Activations of tokens [t0, t0+T) with a planted routing preference:
 *   x_t = z_t + gamma * sum_{e in S_t} Wr[e] / |Wr[e]|^2,  z_t ~ N(0,1) (stream 0)
 * computed in fp64 from the already-rounded router rows, then rounded to dtype.
 * This raises token t's logits for its planted experts by about gamma.
 */
void gen_planted_x(uint64_t seed, int64_t t0, int T, int H, int E, int k, const uint16_t* wr, int dtype,
                   const int32_t* sets, double gamma, uint16_t* x) {
  uint64_t key = stream_key(seed, 0);
  double* inv = (double*)malloc(sizeof(double) * (size_t)E);
  for (int e = 0; e < E; ++e) {
    double n2 = 0;
    for (int h = 0; h < H; ++h) {
      double v = decode(wr[(int64_t)e * H + h], dtype);
      n2 += v * v;
    }
    inv[e] = n2 > 0 ? 1.0 / n2 : 0.0;
  }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      double v = normal_at(key, (uint64_t)(t0 + t) * (uint64_t)H + (uint64_t)h);
      for (int j = 0; j < k; ++j) {
        int e = sets[(int64_t)t * k + j];
        v += gamma * decode(wr[(int64_t)e * H + h], dtype) * inv[e];
      }
      x[(int64_t)t * H + h] = round_to(v, dtype);
    }
  }
  free(inv);
}
