// Router: logits GEMV, top-k selection with renormalised softmax weights, and
// the entropy-adaptive top-1/2/3 variant.
//
// logits[t, e] = sum_h x[t, h] * Wr[e, h], fp32 accumulation (page "Qwen3.5
// Block在llama.cpp中的映射与优化原理", section 4.1: the router is one linear
// layer followed by softmax and top-k).  Selection is made on logits with the
// key (larger logit, lower index); weights are exp(l_s - l_1) / sum over the
// selected slots, the softmax renormalised over the selected experts.
// Entropy-adaptive k (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section
// 2.2): mean over the call's tokens of the Shannon entropy (nats) of the
// routing distribution; k = 1 if H < 1.2, 2 if H < 2.5, else 3.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// --------------------------------------------------------------- logits --
//
// A wave computes a TT-token x 4-expert tile; lane l owns the 8-element
// column slices h = 8*l + 512*i.  Products of two fp16 (or two bf16) values
// are exact in fp32; each lane sums its slice in order, then the wave sums the
// 64 lane partials with a butterfly.
template <int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr, float* __restrict__ logits,
                                                            int T, int H, int E, int act) {
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  const int t0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * 16 + wave * 4;
  if (e0 >= E) return;
  float acc[TT][4];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;

  for (int h = lane * 8; h < H; h += 512) {
    float xv[TT][8], wv[4][8];
#pragma unroll
    for (int a = 0; a < TT; ++a) {
      int t = t0 + a;
      u32x4 r = {0u, 0u, 0u, 0u};
      if (t < T) r = load16(x + (size_t)t * H + h);
      uint32_t w4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[a][2 * i] = act_to_f32(w4[i] & 0xFFFFu, act);
        xv[a][2 * i + 1] = act_to_f32(w4[i] >> 16, act);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int e = e0 + b;
      u32x4 r = {0u, 0u, 0u, 0u};
      if (e < E) r = load16(wr + (size_t)e * H + h);
      uint32_t w4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[b][2 * i] = act_to_f32(w4[i] & 0xFFFFu, act);
        wv[b][2 * i + 1] = act_to_f32(w4[i] >> 16, act);
      }
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[a][b] = fmaf(xv[a][i], wv[b][i], acc[a][b]);  // exact product
  }
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float s = wave_sum(acc[a][b]);
      int t = t0 + a, e = e0 + b;
      if (lane == 0 && t < T && e < E) logits[(size_t)t * E + e] = s;
    }
}

// ------------------------------------------------------------ selection --

struct Cand {
  float v;
  int i;
};

// larger value first, lower index first among equal values; index -1 = none
__device__ __forceinline__ Cand better(Cand a, Cand b) {
  if (a.i < 0) return b;
  if (b.i < 0) return a;
  if (a.v > b.v) return a;
  if (b.v > a.v) return b;
  return a.i < b.i ? a : b;
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    Cand d;
    d.v = __shfl_xor(c.v, o, WAVE);
    d.i = __shfl_xor(c.i, o, WAVE);
    c = better(c, d);
  }
  return c;
}

// One wave selects k of token t's E <= 256 logits (4 per lane, expert
// e = lane + 64*j).  Returns the selected logits/indices in slot order in
// every lane (arrays of MOE_MAX_K).
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, float* sv, int* si) {
  const int lane = lane_id();
  float v[4];
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = lane + 64 * j;
    live[j] = e < E;
    v[j] = live[j] ? row[e] : 0.0f;
  }
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s) {
    if (s < k) {
      Cand c = {0.0f, -1};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Cand d = {v[j], live[j] ? lane + 64 * j : -1};
        c = better(c, d);
      }
      c = wave_best(c);
      sv[s] = c.v;
      si[s] = c.i;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == c.i) live[j] = false;
    }
  }
}

// weights of the first k selected slots; slots [k, kcap) get index -1, weight 0
__device__ __forceinline__ void write_selection(int32_t* idx, float* w, const float* sv, const int* si, int k,
                                                int kcap) {
  float ex[MOE_MAX_K_DEV];
  float z = 0.0f;
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s) {
    if (s < k) {
      ex[s] = expf(sv[s] - sv[0]);
      z += ex[s];
    }
  }
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s) {
    if (s < kcap) {
      idx[s] = s < k ? si[s] : -1;
      w[s] = s < k ? ex[s] / z : 0.0f;
    }
  }
}

__global__ __launch_bounds__(256) void topk_static_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          int32_t* __restrict__ k_used, float* __restrict__ entropy) {
  const int t = blockIdx.x * 4 + threadIdx.x / WAVE;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (k_used) *k_used = k;
    if (entropy) *entropy = 0.0f;
  }
  if (t >= T) return;
  float sv[MOE_MAX_K_DEV];
  int si[MOE_MAX_K_DEV];
  wave_topk(logits + (size_t)t * E, E, k, sv, si);
  if (lane_id() == 0) write_selection(idx + (size_t)t * k, w + (size_t)t * k, sv, si, k, k);
}

// Shannon entropy (nats) of softmax(row): H = ln Z - sum_e p_e (l_e - l_max)
__device__ __forceinline__ float wave_entropy(const float* __restrict__ row, int E) {
  const int lane = lane_id();
  float v[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = lane + 64 * j;
    v[j] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = wave_max(m);
  float z = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (lane + 64 * j < E) {
      float d = v[j] - m;
      float p = expf(d);
      z += p;
      s1 += p * d;
    }
  }
  z = wave_sum(z);
  s1 = wave_sum(s1);
  return logf(z) - s1 / z;
}

// One workgroup of 16 waves.  Wave w handles tokens w, w+16, ...; its
// entropies are summed in token order, the 16 wave partials in wave order,
// so the batch entropy does not depend on timing.
__global__ __launch_bounds__(1024) void topk_entropy_kernel(const float* __restrict__ logits, int T, int E,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            int32_t* __restrict__ k_used,
                                                            float* __restrict__ entropy) {
  __shared__ float part[16];
  __shared__ int k_sh;
  const int wave = threadIdx.x / WAVE;
  float hs = 0.0f;
  for (int t = wave; t < T; t += 16) hs += wave_entropy(logits + (size_t)t * E, E);
  if (lane_id() == 0) part[wave] = hs;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
    for (int i = 0; i < 16; ++i) tot += part[i];
    float h = tot / (float)T;
    int k = h < 1.2f ? 1 : (h < 2.5f ? 2 : 3);
    k_sh = k;
    if (k_used) *k_used = k;
    if (entropy) *entropy = h;
  }
  __syncthreads();
  const int k = k_sh;
  for (int t = wave; t < T; t += 16) {
    float sv[MOE_MAX_K_DEV];
    int si[MOE_MAX_K_DEV];
    wave_topk(logits + (size_t)t * E, E, k, sv, si);
    if (lane_id() == 0)
      write_selection(idx + (size_t)t * MOE_K_ENTROPY_CAP_DEV, w + (size_t)t * MOE_K_ENTROPY_CAP_DEV, sv, si, k,
                      MOE_K_ENTROPY_CAP_DEV);
  }
}

// ------------------------------------------------------------- launchers --

hipError_t launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, int act,
                                hipStream_t st) {
  dim3 block(256);
  if (T < 4) {
    dim3 grid(T, (E + 15) / 16);
    router_logits_kernel<1><<<grid, block, 0, st>>>((const uint16_t*)x, (const uint16_t*)wr, logits, T, H, E, act);
  } else {
    dim3 grid((T + 3) / 4, (E + 15) / 16);
    router_logits_kernel<4><<<grid, block, 0, st>>>((const uint16_t*)x, (const uint16_t*)wr, logits, T, H, E, act);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, int32_t* k_used,
                       float* entropy, hipStream_t st) {
  if (k > 0) {
    topk_static_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, idx, w, k_used, entropy);
  } else {
    topk_entropy_kernel<<<1, 1024, 0, st>>>(logits, T, E, idx, w, k_used, entropy);
  }
  return hipGetLastError();
}

}  // namespace moe
