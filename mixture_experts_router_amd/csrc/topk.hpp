// Top-k selection of one token's logits by one wave (shared by the router
// kernels and the decode gate+up GEMV, which selects from the logits itself
// with the same operations, so every kernel sees the same experts and weights).
//
// Key: larger logit first, lower expert index first among equal logits.
// Groups (gs > 1 experts each, consecutive): choosing an expert retires its
// whole group, so at most one expert per group is chosen, and the slots are
// the best experts of the best groups in key order (page "Qwen3.5 Block在
// llama.cpp中的映射与优化原理", section 1.1: 64 experts in 4 groups of 16, the
// best of each group).  gs = 1 is plain top-k.
// Weights: exp(l_s - l_1) / sum over the selected slots of exp(l_s' - l_1),
// i.e. the softmax renormalised over the selected experts (page "Qwen3.5
// Block在llama.cpp中的映射与优化原理", section 4.1: linear -> softmax -> top-k).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct Cand {
  float v;
  int i;
};

// larger value first, lower index first among equal values; index -1 = none.
// Written with selects (no short-circuit branches): symmetric, so every lane
// of a reduction picks the same candidate.
__device__ __forceinline__ Cand better(Cand a, Cand b) {
  const bool a_none = a.i < 0, b_none = b.i < 0;
  const bool b_higher = (b.v > a.v) | ((b.v == a.v) & (b.i < a.i));
  const bool take_b = a_none | (!b_none & b_higher);
  Cand r;
  r.v = take_b ? b.v : a.v;
  r.i = take_b ? b.i : a.i;
  return r;
}

template <int CTRL>
__device__ __forceinline__ Cand dpp_cand(Cand c) {
  Cand d;
  d.v = dpp_f<CTRL>(c.v);
  d.i = dpp_i<CTRL>(c.i);
  return d;
}

// best candidate over the wave (the order is total, so every lane agrees)
__device__ __forceinline__ Cand wave_best(Cand c) {
  c = better(c, dpp_cand<DPP_QUAD_1032>(c));
  c = better(c, dpp_cand<DPP_QUAD_2301>(c));
  c = better(c, dpp_cand<DPP_ROW_HALF_MIRROR>(c));
  c = better(c, dpp_cand<DPP_ROW_MIRROR>(c));
  Cand r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j].v = readlane_f(c.v, 16 * j);
    r[j].i = __builtin_amdgcn_readlane(c.i, 16 * j);
  }
  return better(better(r[0], r[1]), better(r[2], r[3]));
}

// One wave selects k of token t's E <= 256 logits (4 per lane, expert
// e = lane + 64*j).  Returns the selected logits/indices in slot order in
// every lane (arrays of MOE_MAX_K).
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, float* sv, int* si, int gs) {
  const int lane = lane_id();
  float v[4];
  bool live[4];
  int grp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = lane + 64 * j;
    live[j] = e < E;
    v[j] = live[j] ? row[e] : 0.0f;
    grp[j] = e / gs;
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
      const int cg = c.i / gs;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (grp[j] == cg) live[j] = false;
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


// Select k experts of one token; every lane receives the same idx/w arrays.
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int* idx, float* w,
                                            int gs) {
  float sv[MOE_MAX_K_DEV];
  int si[MOE_MAX_K_DEV];
  wave_topk(row, E, k, sv, si, gs);
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
    idx[s] = s < k ? si[s] : -1;
    w[s] = s < k ? ex[s] / z : 0.0f;
  }
}

// The expert and routing weight of one slot of token t (the same values as
// route_token: z sums exp(l_s - l_1) in slot order), with one selection
// round per slot in a loop rather than unrolled over MOE_MAX_K slots: a
// decode kernel runs this before its first weight load, and a short code path
// is fetched into the instruction cache faster.
__device__ __forceinline__ void route_slot(const float* __restrict__ row, int E, int k, int slot, int& e_out,
                                           float& w_out, int gs) {
  const int lane = lane_id();
  float v[4];
  bool live[4];
  int grp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    live[j] = e < E;
    v[j] = live[j] ? row[e] : 0.0f;
    grp[j] = e / gs;
  }
  float v0 = 0.0f, z = 0.0f, mine = 0.0f;
  int mye = 0;
#pragma unroll 1
  for (int s = 0; s < k; ++s) {
    Cand c = {0.0f, -1};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const Cand d = {v[j], live[j] ? lane + 64 * j : -1};
      c = better(c, d);
    }
    c = wave_best(c);
    if (s == 0) v0 = c.v;
    const float ex = expf(c.v - v0);
    z += ex;
    if (s == slot) {
      mye = c.i;
      mine = ex;
    }
    const int cg = c.i / gs;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (grp[j] == cg) live[j] = false;
  }
  e_out = mye;
  w_out = mine / z;
}

}  // namespace moe
