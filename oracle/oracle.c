/*
 * CPU oracle for one sparse Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the HIP
 * path and is deliberately plain: every step is the textbook definition,
 * written out with sequential fp32 sums (compiled with -ffp-contract=off, so
 * each product and each sum is rounded separately), no blocking, no fusion.
 *
 * What it computes, and where the pages define it:
 *
 *   router      logits = x . Wr^T, then softmax and top-k (page "Qwen3.5 Block
 *               在llama.cpp中的映射与优化原理", section 4.1, the PyTorch router:
 *               F.linear -> softmax -> topk).  Selection is made on the logits
 *               in the order (larger logit first, then lower expert index);
 *               softmax is monotone, so this is the same set as topk over the
 *               probabilities, without ties created by rounding.  The selected
 *               probabilities are renormalised to sum to one.
 *   adaptive k  Shannon entropy of the routing distribution, averaged over the
 *               tokens of the call; k = 1 if H < 1.2, 2 if 1.2 <= H < 2.5,
 *               3 otherwise (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析",
 *               section 2.2, Entropy-Aware Routing).  Natural logarithm.
 *   pair sort   stable counting sort of (token, slot) pairs by expert, the
 *               grouping a gathered expert matmul needs (oMLX page, the sorted
 *               "_gather_sort" branch under "如何验证正确性").
 *   dequant     affine group quantisation, w = scale * q + bias with one
 *               scale/bias per row and 64-column group (oMLX page, "融合原理":
 *               scales are packed per output row).
 *   nvfp4       the oMLX page names an nvfp4 weight mode (its list of modes
 *               under "如何验证正确性") and gives no layout; read as NVIDIA's
 *               published NVFP4: E2M1 codes two per byte (even column in the
 *               low nibble), one FP8 E4M3 scale per row and 16 consecutive
 *               columns, one fp32 scale per tensor, w = (ts * s) * e2m1(q)
 *               in fp32 (two roundings), no bias.
 *   gate_up     the gate and up projections concatenated along the output
 *               axis, [gate, up] order, then split (oMLX page, steps 3 and 4).
 *   SwiGLU      h = silu(g) * u, silu(g) = g / (1 + e^-g).
 *   down        o = W_down . h
 *   load-aware  logits_final = logits - alpha * H_e, the per-expert load index
 *   correction  H_e weighted by a scale alpha, subtracted before selection
 *               (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 3.3,
 *               auxiliary routing head).  Every later step of the routing
 *               (entropy, selection, weights) uses the corrected logits.
 *   groups      the E experts in G groups of E/G consecutive experts and at
 *               most one expert chosen per group: each group's best expert,
 *               then the k best of those (llama.cpp page, section 1.1: 64
 *               experts in 4 groups of 16, the best of each group, 4 chosen).
 *   capacity    at most C (token, slot) pairs per expert: the first C in pair
 *               order are kept, the rest dropped and contribute nothing to the
 *               output (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section
 *               5.2: a per-expert token capacity, expert_capacity=8; which
 *               pairs overflow is not stated, so the earliest are kept).
 *   load stats  the least-used expert and the standard deviation of the
 *               per-expert activation counts (page "Qwen3.5-MoE与Qwen3-MoE
 *               架构差异深度解析", the closing advice on monitoring MoE health).
 *   combine     y = sum over the token's slots of weight * o, in slot order,
 *               with the weight applied after the down projection (llama.cpp
 *               page, section 4.2, the weighted-sum loop), rounded to the
 *               activation dtype with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* ------------------------------------------------ fp16 / bf16 (own) ---- */

float oracle_half_to_float(uint16_t b, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  int sign = b >> 15, e = (b >> 10) & 31, m = b & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* round-to-nearest-even from fp32, written with frexp/ldexp rather than bits */
uint16_t oracle_float_to_half(float f, int dtype) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = u >> 31;
  if (isnan(f)) return (uint16_t)(dtype == ORACLE_BF16 ? ((u >> 16) | 0x40) : ((sign << 15) | 0x7E00));
  if (dtype == ORACLE_BF16) {
    /* keep 8 significant bits: value = round_half_even(f / 2^(e-8)) * 2^(e-8) */
    if (isinf(f) || f == 0.0f) return (uint16_t)(u >> 16);
    if (fabs((double)f) < ldexp(1.0, -126)) { /* below the normal range: fixed grid 2^-133 */
      double r = nearbyint(ldexp(fabs((double)f), 133));
      return (uint16_t)((sign << 15) | (uint32_t)r);
    }
    int e;
    double m = frexp(fabs((double)f), &e); /* |f| = m * 2^e, m in [0.5, 1) */
    double r = nearbyint(ldexp(m, 8));     /* 8 significant bits, RNE */
    double v = ldexp(r, e - 8);
    float fv = (float)v;
    uint32_t uv;
    memcpy(&uv, &fv, 4);
    return (uint16_t)((sign << 15) | ((uv >> 16) & 0x7FFF));
  }
  double a = fabs((double)f);
  uint32_t mag;
  if (isinf(f) || a >= 65520.0) {
    mag = 0x7C00;
  } else if (a < ldexp(1.0, -14)) {
    mag = (uint32_t)nearbyint(ldexp(a, 24)); /* subnormal grid 2^-24 */
  } else {
    int e;
    double m = frexp(a, &e);               /* a = m * 2^e, m in [0.5,1) */
    double r = nearbyint(ldexp(m, 11));    /* 11 significant bits */
    if (r >= 2048.0) { r /= 2.0; e += 1; } /* rounding carried into the next binade */
    mag = (uint32_t)((e - 1 + 15) << 10) | ((uint32_t)r - 1024u);
    if (mag >= 0x7C00) mag = 0x7C00;
  }
  return (uint16_t)((sign << 15) | mag);
}

/* ------------------------------------------- NVFP4 element formats ---- */

enum { ORACLE_NVFP4 = 0x104 }; /* `bits` code of NVFP4 weights: 4-bit codes of the second format */

/* E2M1: sign bit 3, two exponent bits (bias 1), one mantissa bit; exponent
 * field 0 is subnormal (0 or 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
float oracle_e2m1_to_float(int code) {
  int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return sign ? -v : v;
}

/* FP8 E4M3 (the OCP "fn" variant): sign bit 7, four exponent bits (bias 7),
 * three mantissa bits; exponent field 0 is subnormal (m * 2^-9); 0x7F and
 * 0xFF are NaN and there are no infinities (largest finite 448). */
float oracle_e4m3_to_float(int byte) {
  int sign = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if ((byte & 0x7F) == 0x7F) return NAN;
  float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return sign ? -v : v;
}

static int code_bits(int bits) { return bits == ORACLE_NVFP4 ? 4 : bits; }
/* bytes of one scale: E4M3 bytes for NVFP4, fp16 otherwise */
static int scale_bytes(int bits) { return bits == ORACLE_NVFP4 ? 1 : 2; }

/* -------------------------------------------------------- dequant (A5) -- */

/*
 * One row of K weights.  bits 4: two codes per byte, even column in the low
 * nibble; bits 5 and 6: code k at bits b*k .. b*k+b-1 of the row read as a
 * little-endian bit stream (b = bits); bits 8: one code per byte; code q is
 * unsigned.  w = s*q + b in fp32
 * (two roundings), s and b fp16, one pair per 64-column group.
 * bits 16: the row is fp16 values, copied.
 * bits ORACLE_NVFP4: E2M1 codes packed as 4-bit codes, s_row the row's E4M3
 * block scales (one byte per gs = 16 columns), b_row unused, ts the tensor
 * scale: w = (ts * e4m3(s)) * e2m1(q) in fp32.
 */
void oracle_dequant_row(const void* q_row, const void* s_row, const uint16_t* b_row, int K, int bits, int gs,
                        float ts, float* out) {
  if (bits == 16) {
    const uint16_t* w = (const uint16_t*)q_row;
    for (int k = 0; k < K; ++k) out[k] = oracle_half_to_float(w[k], ORACLE_F16);
    return;
  }
  const uint8_t* q = (const uint8_t*)q_row;
  if (bits == ORACLE_NVFP4) {
    const uint8_t* sb = (const uint8_t*)s_row;
    for (int k = 0; k < K; ++k) {
      int code = (q[k / 2] >> (4 * (k & 1))) & 15;
      float s = ts * oracle_e4m3_to_float(sb[k / gs]);
      out[k] = s * oracle_e2m1_to_float(code);
    }
    return;
  }
  const uint16_t* s16 = (const uint16_t*)s_row;
  for (int k = 0; k < K; ++k) {
    int code;
    if (bits == 4) {
      code = (q[k / 2] >> (4 * (k & 1))) & 15;
    } else if (bits == 5 || bits == 6) {
      int64_t bit = (int64_t)bits * k;
      int sh = (int)(bit % 8);
      int v = q[bit / 8] >> sh;
      if (sh + bits > 8) v |= q[bit / 8 + 1] << (8 - sh);
      code = v & ((1 << bits) - 1);
    } else {
      code = q[k];
    }
    float s = oracle_half_to_float(s16[k / gs], ORACLE_F16);
    float b = oracle_half_to_float(b_row[k / gs], ORACLE_F16);
    float sq = s * (float)code;
    out[k] = sq + b;
  }
}

static int64_t row_bytes_of(int K, int bits) { return (int64_t)K * code_bits(bits) / 8; }

/* ---------------------------------------------------------- router (A1) -- */

void oracle_router_logits(const uint16_t* x, int dtype, int T, int H, const uint16_t* wr, int E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int h = 0; h < H; ++h) {
        float p = oracle_half_to_float(x[(int64_t)t * H + h], dtype) * oracle_half_to_float(wr[(int64_t)e * H + h], dtype);
        acc = acc + p;
      }
      logits[(int64_t)t * E + e] = acc;
    }
  }
}

/* -------------------------------------------- selection + weights (A2) -- */

/* experts ordered by larger logit first, lower index first among equals */
static void order_experts(const float* l, int E, int* order) {
  for (int i = 0; i < E; ++i) {
    int j = i;
    while (j > 0 && (l[order[j - 1]] < l[i] || (l[order[j - 1]] == l[i] && order[j - 1] > i))) {
      order[j] = order[j - 1];
      --j;
    }
    order[j] = i;
  }
}

/* softmax over all E experts (fp32, max-subtracted), then the chosen k renormalised */
static void select_one(const float* l, int E, int k, int kcap, int32_t* idx, float* w) {
  int order[256];
  float p[256];
  order_experts(l, E, order);
  float lmax = l[order[0]];
  float z = 0.0f;
  for (int e = 0; e < E; ++e) {
    p[e] = expf(l[e] - lmax);
    z = z + p[e];
  }
  for (int e = 0; e < E; ++e) p[e] = p[e] / z;
  float tot = 0.0f;
  for (int s = 0; s < k; ++s) tot = tot + p[order[s]];
  for (int s = 0; s < kcap; ++s) {
    if (s < k) {
      idx[s] = order[s];
      w[s] = p[order[s]] / tot;
    } else {
      idx[s] = -1;
      w[s] = 0.0f;
    }
  }
}

void oracle_select_topk(const float* logits, int T, int E, int k, int kcap, int32_t* idx, float* w) {
  for (int t = 0; t < T; ++t) select_one(logits + (int64_t)t * E, E, k, kcap, idx + (int64_t)t * kcap, w + (int64_t)t * kcap);
}

/*
 * Group-limited selection for one token: G groups of E/G consecutive experts.
 * First the best expert of every group (larger logit, then lower index), then
 * those G winners ordered by the same key; the first k are the slots.  The
 * weights are the softmax over all E experts renormalised over the chosen k,
 * as in select_one.
 */
static void select_grouped(const float* l, int E, int G, int k, int kcap, int32_t* idx, float* w) {
  int gs = E / G, win[256], order[256];
  float wl[256], p[256];
  for (int g = 0; g < G; ++g) {
    int b = g * gs;
    for (int e = g * gs + 1; e < (g + 1) * gs; ++e)
      if (l[e] > l[b]) b = e; /* strictly larger: the lower index stays on ties */
    win[g] = b;
    wl[g] = l[b];
  }
  order_experts(wl, G, order); /* order of the winners by (logit, then group = index order) */
  float lmax = l[win[order[0]]];
  float z = 0.0f;
  for (int e = 0; e < E; ++e) {
    p[e] = expf(l[e] - lmax);
    z = z + p[e];
  }
  for (int e = 0; e < E; ++e) p[e] = p[e] / z;
  float tot = 0.0f;
  for (int s = 0; s < k; ++s) tot = tot + p[win[order[s]]];
  for (int s = 0; s < kcap; ++s) {
    if (s < k) {
      idx[s] = win[order[s]];
      w[s] = p[win[order[s]]] / tot;
    } else {
      idx[s] = -1;
      w[s] = 0.0f;
    }
  }
}

/* groups <= 1: plain top-k; else group-limited (E % groups == 0, k <= groups) */
void oracle_select_topk_grouped(const float* logits, int T, int E, int groups, int k, int kcap, int32_t* idx,
                                float* w) {
  for (int t = 0; t < T; ++t) {
    if (groups <= 1)
      select_one(logits + (int64_t)t * E, E, k, kcap, idx + (int64_t)t * kcap, w + (int64_t)t * kcap);
    else
      select_grouped(logits + (int64_t)t * E, E, groups, k, kcap, idx + (int64_t)t * kcap, w + (int64_t)t * kcap);
  }
}

/* logits[t, e] -= alpha * health[e] (the product and the difference each rounded to fp32) */
void oracle_correct_logits(float* logits, int T, int E, const float* health, float alpha) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      float c = alpha * health[e];
      logits[(int64_t)t * E + e] = logits[(int64_t)t * E + e] - c;
    }
}

/*
 * Health figures of a vector of per-expert activation counts: the least-used
 * expert (the lowest index among the smallest counts) and the population
 * standard deviation of the counts, sqrt(sum_e (c_e - mean)^2 / E), computed
 * in fp64 and rounded to fp32.
 */
void oracle_load_stats(const int32_t* counts, int E, int32_t* least_used, float* stddev) {
  int m = 0;
  for (int e = 1; e < E; ++e)
    if (counts[e] < counts[m]) m = e;
  double mean = 0.0;
  for (int e = 0; e < E; ++e) mean += (double)counts[e];
  mean /= (double)E;
  double ss = 0.0;
  for (int e = 0; e < E; ++e) ss += ((double)counts[e] - mean) * ((double)counts[e] - mean);
  *least_used = m;
  *stddev = (float)sqrt(ss / (double)E);
}

/* -------------------------------------------------- adaptive k (A2') --- */

/* Shannon entropy (nats) of softmax(logits) for one token */
float oracle_token_entropy(const float* l, int E) {
  float lmax = l[0];
  for (int e = 1; e < E; ++e)
    if (l[e] > lmax) lmax = l[e];
  float p[256], z = 0.0f;
  for (int e = 0; e < E; ++e) {
    p[e] = expf(l[e] - lmax);
    z = z + p[e];
  }
  float h = 0.0f;
  for (int e = 0; e < E; ++e) {
    float pe = p[e] / z;
    if (pe > 0.0f) h = h - pe * logf(pe);
  }
  return h;
}

int oracle_entropy_k(float H) {
  if (H < 1.2f) return 1;
  if (H < 2.5f) return 2;
  return 3;
}

/* batch entropy: the mean over the call's tokens of the per-token entropy */
float oracle_batch_entropy(const float* logits, int T, int E) {
  float s = 0.0f;
  for (int t = 0; t < T; ++t) s = s + oracle_token_entropy(logits + (int64_t)t * E, E);
  return s / (float)T;
}

/*
 * Full routing.  k > 0: static top-k, kcap = k.  k == -1: entropy-adaptive,
 * kcap = 3, k_used chosen from the batch entropy; slots >= k_used get
 * index -1 and weight 0.  logits_out may be NULL.
 */
void oracle_route_ex(const uint16_t* x, int dtype, int T, int H, const uint16_t* wr, int E, int k,
                     const float* health, float alpha, int groups, int32_t* idx, float* w, int32_t* k_used,
                     float* h_mean, float* logits_out) {
  float* logits = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)T * E);
  oracle_router_logits(x, dtype, T, H, wr, E, logits);
  if (health) oracle_correct_logits(logits, T, E, health, alpha);
  int kcap = k > 0 ? k : 3, ku = k;
  float hm = 0.0f;
  if (k < 0) {
    hm = oracle_batch_entropy(logits, T, E);
    ku = oracle_entropy_k(hm);
  }
  oracle_select_topk_grouped(logits, T, E, groups, ku, kcap, idx, w);
  if (k_used) *k_used = ku;
  if (h_mean) *h_mean = hm;
  if (!logits_out) free(logits);
}

void oracle_route(const uint16_t* x, int dtype, int T, int H, const uint16_t* wr, int E, int k, int32_t* idx,
                  float* w, int32_t* k_used, float* h_mean, float* logits_out) {
  oracle_route_ex(x, dtype, T, H, wr, E, k, NULL, 0.0f, 0, idx, w, k_used, h_mean, logits_out);
}

/* ------------------------------------------------------ pair sort (A3) -- */

/*
 * Pairs p = t*kcap + s for s < k_used.  counts[e] = pairs routed to e,
 * offsets = exclusive prefix sum (E+1 entries), perm = pair ids grouped by
 * expert and ascending within an expert, pos = inverse of perm (-1 for the
 * unused slots).  perm entries past the last valid pair are -1.
 */
void oracle_sort_pairs(const int32_t* idx, int T, int kcap, int k_used, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* pos) {
  int64_t P = (int64_t)T * kcap;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p)
    if (p % kcap < k_used) counts[idx[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < P; ++p) perm[p] = -1;
  for (int64_t p = 0; p < P; ++p) {
    if (p % kcap >= k_used) {
      pos[p] = -1;
      continue;
    }
    int e = idx[p];
    int32_t at = offsets[e] + fill[e]++;
    perm[at] = (int32_t)p;
    pos[p] = at;
  }
  free(fill);
}

/*
 * Capacity: keep[p] = 1 for the first `capacity` valid pairs of every expert
 * in ascending pair id, 0 for the rest and for the unused slots; capacity
 * <= 0 keeps every valid pair.
 */
void oracle_capacity_keep(const int32_t* idx, int T, int kcap, int k_used, int E, int capacity, uint8_t* keep) {
  int64_t P = (int64_t)T * kcap;
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < P; ++p) {
    if (p % kcap >= k_used) {
      keep[p] = 0;
      continue;
    }
    int e = idx[p];
    keep[p] = (uint8_t)(capacity <= 0 || seen[e] < capacity);
    seen[e]++;
  }
  free(seen);
}

/* the pair sort over the kept pairs only (dropped pairs get pos -1) */
void oracle_sort_pairs_capped(const int32_t* idx, int T, int kcap, int k_used, int E, int capacity, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* pos) {
  int64_t P = (int64_t)T * kcap;
  uint8_t* keep = (uint8_t*)malloc((size_t)(P > 0 ? P : 1));
  oracle_capacity_keep(idx, T, kcap, k_used, E, capacity, keep);
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p)
    if (keep[p]) counts[idx[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < P; ++p) perm[p] = -1;
  for (int64_t p = 0; p < P; ++p) {
    if (!keep[p]) {
      pos[p] = -1;
      continue;
    }
    int e = idx[p];
    int32_t at = offsets[e] + fill[e]++;
    perm[at] = (int32_t)p;
    pos[p] = at;
  }
  free(fill);
  free(keep);
}

/* ------------------------------------------------ gate/up packing ------ */

/*
 * Concatenate gate [E, I, K] and up [E, I, K] along the output axis into
 * gate_up [E, 2I, K], gate rows first; weights, scales and biases alike
 * (NVFP4: codes and block scales; the two tensors must share their tensor
 * scale, which the caller keeps).
 */
void oracle_fuse_gate_up(const void* gq, const void* gs_, const uint16_t* gb, const void* uq, const void* us,
                         const uint16_t* ub, int E, int I, int K, int bits, int gsz, void* oq, void* os,
                         uint16_t* ob) {
  int64_t rb = row_bytes_of(K, bits);
  int64_t ng = K / gsz, sb = scale_bytes(bits);
  for (int e = 0; e < E; ++e) {
    uint8_t* dq = (uint8_t*)oq + (int64_t)e * 2 * I * rb;
    memcpy(dq, (const uint8_t*)gq + (int64_t)e * I * rb, (size_t)(I * rb));
    memcpy(dq + I * rb, (const uint8_t*)uq + (int64_t)e * I * rb, (size_t)(I * rb));
    if (bits != 16) {
      uint8_t* ds = (uint8_t*)os;
      memcpy(ds + (int64_t)e * 2 * I * ng * sb, (const uint8_t*)gs_ + (int64_t)e * I * ng * sb, (size_t)(I * ng * sb));
      memcpy(ds + ((int64_t)e * 2 * I + I) * ng * sb, (const uint8_t*)us + (int64_t)e * I * ng * sb,
             (size_t)(I * ng * sb));
    }
    if (bits != 16 && bits != ORACLE_NVFP4) {
      memcpy(ob + (int64_t)e * 2 * I * ng, gb + (int64_t)e * I * ng, sizeof(uint16_t) * (size_t)(I * ng));
      memcpy(ob + ((int64_t)e * 2 * I + I) * ng, ub + (int64_t)e * I * ng, sizeof(uint16_t) * (size_t)(I * ng));
    }
  }
}

/* ------------------------------------------- expert FFN (A5-A8) -------- */

typedef struct {
  const void* q;
  const void* s;
  const uint16_t* b;
  int K, bits, gs;
  float ts;  /* NVFP4 tensor scale */
} row_src;

static const void* rq(const row_src* r, int64_t row) { return (const uint8_t*)r->q + row * row_bytes_of(r->K, r->bits); }
static const void* rs(const row_src* r, int64_t row) {
  return r->s ? (const uint8_t*)r->s + row * (r->K / r->gs) * scale_bytes(r->bits) : NULL;
}
static const uint16_t* rbias(const row_src* r, int64_t row) { return r->b ? r->b + row * (r->K / r->gs) : NULL; }

/* out[n] = sum_k v[k] * W[row0 + n, k] for n in [0, N), sequential fp32 sums */
static void matvec(const row_src* W, int64_t row0, int N, const float* v, float* out) {
  int K = W->K;
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      oracle_dequant_row(rq(W, row0 + n), rs(W, row0 + n), rbias(W, row0 + n), K, W->bits, W->gs, W->ts, wrow);
      float acc = 0.0f;
      for (int k = 0; k < K; ++k) {
        float p = v[k] * wrow[k];
        acc = acc + p;
      }
      out[n] = acc;
    }
    free(wrow);
  }
}

static float silu(float g) { return g / (1.0f + expf(-g)); }

/*
 * One (token, expert): x [H] fp32 values; gate_up rows [2I, H] of this expert
 * (gate first), down rows [H, I].  h_out [I] (may be NULL), o [H].
 * gu_ts, d_ts: the tensor scales of NVFP4 weights (unused otherwise).
 */
void oracle_expert_ffn(const float* x, const void* guq, const void* gus, const uint16_t* gub, const void* dq,
                       const void* ds, const uint16_t* db, int H, int I, int bits, int gsz, float gu_ts, float d_ts,
                       float* h_out, float* o) {
  row_src gu = {guq, gus, gub, H, bits, gsz, gu_ts}, dn = {dq, ds, db, I, bits, gsz, d_ts};
  float* gu_v = (float*)malloc(sizeof(float) * 2 * (size_t)I);
  float* h = (float*)malloc(sizeof(float) * (size_t)I);
  matvec(&gu, 0, 2 * I, x, gu_v);
  for (int j = 0; j < I; ++j) {
    float g = gu_v[j], u = gu_v[I + j];
    h[j] = silu(g) * u;
  }
  matvec(&dn, 0, H, h, o);
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
  free(gu_v);
  free(h);
}

/* the same with separate gate [I, H] and up [I, H] rows (and tensor scales) */
void oracle_expert_ffn_unfused(const float* x, const void* gq, const void* gs_, const uint16_t* gb, const void* uq,
                               const void* us, const uint16_t* ub, const void* dq, const void* ds, const uint16_t* db,
                               int H, int I, int bits, int gsz, float g_ts, float u_ts, float d_ts, float* h_out,
                               float* o) {
  row_src ga = {gq, gs_, gb, H, bits, gsz, g_ts}, ua = {uq, us, ub, H, bits, gsz, u_ts},
          dn = {dq, ds, db, I, bits, gsz, d_ts};
  float* g = (float*)malloc(sizeof(float) * (size_t)I);
  float* u = (float*)malloc(sizeof(float) * (size_t)I);
  float* h = (float*)malloc(sizeof(float) * (size_t)I);
  matvec(&ga, 0, I, x, g);
  matvec(&ua, 0, I, x, u);
  for (int j = 0; j < I; ++j) h[j] = silu(g[j]) * u[j];
  matvec(&dn, 0, H, h, o);
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
  free(g);
  free(u);
  free(h);
}

/* ------------------------------------------------------ layer (A1-A9) -- */

/*
 * Expert part of the layer for selected tokens, given the routing:
 *   y_f32[i, :] = sum_{s < k_used} w[t, s] * o_{t,s}  (slot order, fp32)
 * for t = tokens[i].  gate_up: [E, 2I, H] tensor; down: [E, H, I].
 * h_out (may be NULL): [n, kcap, I] SwiGLU outputs, rows of unused slots untouched.
 */
void oracle_tokens_forward(const uint16_t* x, int dtype, int H, const int32_t* tokens, int n, const int32_t* idx,
                           const float* w, int kcap, int k_used, const void* guq, const void* gus,
                           const uint16_t* gub, const void* dq, const void* ds, const uint16_t* db, int I,
                           int bits, int gsz, float gu_ts, float d_ts, float* y_f32, float* h_out) {
  int64_t gu_rows = 2 * (int64_t)I, rbh = row_bytes_of(H, bits), rbi = row_bytes_of(I, bits);
  int64_t ngh = H / gsz, ngi = I / gsz, sb = scale_bytes(bits);
  float* xf = (float*)malloc(sizeof(float) * (size_t)H);
  float* o = (float*)malloc(sizeof(float) * (size_t)H);
  for (int i = 0; i < n; ++i) {
    int t = tokens[i];
    for (int h = 0; h < H; ++h) xf[h] = oracle_half_to_float(x[(int64_t)t * H + h], dtype);
    float* y = y_f32 + (int64_t)i * H;
    for (int h = 0; h < H; ++h) y[h] = 0.0f;
    for (int s = 0; s < k_used; ++s) {
      int e = idx[(int64_t)t * kcap + s];
      if (e < 0) continue; /* a dropped pair (capacity) contributes nothing */
      float ws = w[(int64_t)t * kcap + s];
      const uint8_t* eq = (const uint8_t*)guq + (int64_t)e * gu_rows * rbh;
      const uint8_t* es = gus ? (const uint8_t*)gus + (int64_t)e * gu_rows * ngh * sb : NULL;
      const uint16_t* eb = gub ? gub + (int64_t)e * gu_rows * ngh : NULL;
      const uint8_t* edq = (const uint8_t*)dq + (int64_t)e * H * rbi;
      const uint8_t* eds = ds ? (const uint8_t*)ds + (int64_t)e * H * ngi * sb : NULL;
      const uint16_t* edb = db ? db + (int64_t)e * H * ngi : NULL;
      float* hrow = h_out ? h_out + ((int64_t)i * kcap + s) * I : NULL;
      oracle_expert_ffn(xf, eq, es, eb, edq, eds, edb, H, I, bits, gsz, gu_ts, d_ts, hrow, o);
      for (int h = 0; h < H; ++h) {
        float c = ws * o[h];
        y[h] = y[h] + c;
      }
    }
  }
  free(xf);
  free(o);
}

/* round fp32 outputs to the activation dtype */
void oracle_round_output(const float* y_f32, int64_t n, int dtype, uint16_t* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_float_to_half(y_f32[i], dtype);
}

/*
 * The whole layer: route, then every token through its selected experts,
 * combine and round.  idx/w: [T, kcap]; y: [T, H] activation dtype;
 * y_f32 (may be NULL) the unrounded fp32 result.
 */
void oracle_layer_forward_ex(const uint16_t* x, int dtype, int T, int H, const uint16_t* wr, int E, int k,
                             const float* health, float alpha, int groups, int capacity, const void* guq,
                             const void* gus, const uint16_t* gub, const void* dq, const void* ds,
                             const uint16_t* db, int I, int bits, int gsz, float gu_ts, float d_ts, uint16_t* y,
                             float* y_f32, int32_t* idx, float* w, int32_t* k_used, float* h_mean) {
  int ku = 0;
  oracle_route_ex(x, dtype, T, H, wr, E, k, health, alpha, groups, idx, w, &ku, h_mean, NULL);
  if (k_used) *k_used = ku;
  int kcap = k > 0 ? k : 3;
  /* the experts of the dropped pairs become -1 in a copy; idx stays the routing */
  int64_t P = (int64_t)T * kcap;
  int32_t* idx_kept = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  uint8_t* keep = (uint8_t*)malloc((size_t)(P > 0 ? P : 1));
  oracle_capacity_keep(idx, T, kcap, ku, E, capacity, keep);
  for (int64_t p = 0; p < P; ++p) idx_kept[p] = keep[p] ? idx[p] : -1;
  int32_t* tokens = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int t = 0; t < T; ++t) tokens[t] = t;
  float* yf = y_f32 ? y_f32 : (float*)malloc(sizeof(float) * (size_t)T * H);
  oracle_tokens_forward(x, dtype, H, tokens, T, idx_kept, w, kcap, ku, guq, gus, gub, dq, ds, db, I, bits, gsz, gu_ts,
                        d_ts, yf, NULL);
  oracle_round_output(yf, (int64_t)T * H, dtype, y);
  if (!y_f32) free(yf);
  free(tokens);
  free(idx_kept);
  free(keep);
}

void oracle_layer_forward(const uint16_t* x, int dtype, int T, int H, const uint16_t* wr, int E, int k,
                          const void* guq, const void* gus, const uint16_t* gub, const void* dq, const void* ds,
                          const uint16_t* db, int I, int bits, int gsz, float gu_ts, float d_ts, uint16_t* y,
                          float* y_f32, int32_t* idx, float* w, int32_t* k_used, float* h_mean) {
  oracle_layer_forward_ex(x, dtype, T, H, wr, E, k, NULL, 0.0f, 0, 0, guq, gus, gub, dq, ds, db, I, bits, gsz, gu_ts,
                          d_ts, y, y_f32, idx, w, k_used, h_mean);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
