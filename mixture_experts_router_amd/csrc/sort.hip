// Token -> expert pair sort.
//
// The (token, slot) pairs p = t*kcap + s with s < k_used are grouped by their
// expert, ascending pair id within an expert (a stable counting sort), which is
// the grouping a gathered expert matmul runs over (oMLX gate/up fusion page,
// the sorted "_gather_sort" branch under "如何验证正确性").
//
// Design: one workgroup per expert e, 16 waves.  The pair list is split into
// 16 contiguous segments, one per wave.  Pass 1 counts, with wave ballots,
// the pairs routed below e (its offset) and to e (per-segment counts); pass 2
// writes each pair of e at offset + (pairs of e in earlier segments) + (pairs
// of e earlier in the segment).  No global atomics, so the result is
// deterministic and identical to a sequential stable counting sort.
//
// Capacity C > 0 (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 5.2:
// a per-expert token capacity): only the first C pairs of every expert, in
// pair order, are listed; the others get pos = -1 and are left out of every
// later step.  The offsets then come from the capped counts of all experts,
// an LDS histogram that each workgroup builds for itself.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// expert e's part of the sort: one 1024-thread workgroup
template <int CH>
__device__ __forceinline__ void sort_expert(int e, const int32_t* __restrict__ idx, int T, int kcap,
                                            const int32_t* __restrict__ k_used_dev, int k_static, int E,
                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ perm, int32_t* __restrict__ pos, int cap) {
  __shared__ int s_lt[16], s_eq[16];
  __shared__ int hist[MOE_MAX_EXPERTS_DEV];
  const int lane = lane_id();
  const int wave = wave_id();
  const int ku = k_used_dev ? *k_used_dev : k_static;
  const int64_t P = (int64_t)T * kcap;
  const int64_t seg = ((P + 16 * 64 - 1) / (16 * 64)) * 64;
  const int64_t beg = wave * seg;
  const int64_t end = beg + seg < P ? beg + seg : P;

  // The segment is read in groups of CH rounds of 64 pairs whose loads all
  // go out together (addresses clamped, so every load is issued); pairs past
  // the segment or in unused slots read as "no expert".  CH follows the
  // segment length (the launcher picks it).
  // pair ids fit in 32 bits (perm and pos are int32)
  const uint32_t ukcap = (uint32_t)kcap, uend = (uint32_t)end, uP = (uint32_t)P;
  auto load_group = [&](int64_t c0, int* v) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const uint32_t p = (uint32_t)c0 + 64u * u + (uint32_t)lane;
      const bool valid = p < uend && (int)(p % ukcap) < ku;
      const int raw = idx[p < uP ? p : 0u];
      v[u] = valid ? raw : 0x7FFFFFFF;
    }
  };
  // the segment's first group stays in registers for the second pass (the
  // launcher sizes CH so that one group usually covers the segment)
  int lt = 0, eq = 0;
  int v0[CH];
  for (int64_t c0 = beg; c0 < end; c0 += 64 * CH) {
    int v[CH];
    load_group(c0, v);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      lt += __popcll(__ballot(v[u] < e));
      eq += __popcll(__ballot(v[u] == e));
      if (c0 == beg) v0[u] = v[u];
    }
  }
  if (lane == 0) {
    s_lt[wave] = lt;
    s_eq[wave] = eq;
  }
  __syncthreads();
  int off = 0, before = 0, cnt = 0;
  for (int w = 0; w < 16; ++w) {
    off += s_lt[w];
    cnt += s_eq[w];
    if (w < wave) before += s_eq[w];
  }
  if (cap > 0) {
    // capped offsets: histogram of all experts, then the capped counts below e
    for (int i = threadIdx.x; i < E; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int64_t p = threadIdx.x; p < P; p += blockDim.x)
      if ((int)(p % kcap) < ku) atomicAdd(&hist[idx[p]], 1);
    __syncthreads();
    off = 0;
    for (int i = 0; i < e; ++i) off += min(hist[i], cap);
    cnt = min(cnt, cap);
  }
  int r = before;  // rank within expert e of the segment's first pair of e
  for (int64_t c0 = beg; c0 < end; c0 += 64 * CH) {
    int v[CH];
    if (c0 == beg) {
#pragma unroll
      for (int u = 0; u < CH; ++u) v[u] = v0[u];
    } else {
      load_group(c0, v);
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int64_t p = c0 + 64 * u + lane;
      const uint64_t m = __ballot(v[u] == e);
      if (v[u] == e) {
        const int rank = r + (int)__popcll(m & lanemask_lt());
        if (cap <= 0 || rank < cap) {
          const int at = off + rank;
          perm[at] = (int32_t)p;
          pos[p] = at;
        } else {
          pos[p] = -1;
        }
      }
      r += (int)__popcll(m);
    }
  }
  if (threadIdx.x == 0) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + cnt;
  }
  if (e == E - 1) {
    // the unused tail of perm, and pos of the unused slots
    const int64_t total = off + cnt;
    for (int64_t p = total + threadIdx.x; p < P; p += blockDim.x) perm[p] = -1;
    if (ku < kcap)
      for (int64_t p = threadIdx.x; p < P; p += blockDim.x)
        if ((int)(p % kcap) >= ku) pos[p] = -1;
  }
}

template <int CH>
__global__ __launch_bounds__(1024) void sort_pairs_kernel(const int32_t* __restrict__ idx, int T, int kcap,
                                                          const int32_t* __restrict__ k_used_dev, int k_static, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ pos, int cap) {
  sort_expert<CH>(blockIdx.x, idx, T, kcap, k_used_dev, k_static, E, counts, offsets, perm, pos, cap);
}

// The sort and the batched GEMM's activation operand in one launch (they are
// independent): workgroups 0 .. E-1 sort, the others convert four tokens each
// (prep_a_row, one 256-thread group per token).
template <int CH>
__global__ __launch_bounds__(1024) void sort_prep_kernel(const int32_t* __restrict__ idx, int T, int kcap,
                                                         const int32_t* __restrict__ k_used_dev, int k_static, int E,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ pos, int cap,
                                                         const uint16_t* __restrict__ x, uint16_t* __restrict__ a,
                                                         int H, int act, int perm8, int32_t* __restrict__ tokexp,
                                                         int32_t* __restrict__ any_scaled) {
  if ((int)blockIdx.x < E) {
    sort_expert<CH>(blockIdx.x, idx, T, kcap, k_used_dev, k_static, E, counts, offsets, perm, pos, cap);
    return;
  }
  __shared__ uint32_t wmax[4][4];
  const int g = threadIdx.x / 256;
  const int64_t t = (int64_t)(blockIdx.x - E) * 4 + g;
  prep_a_row(x, a, t < T ? t : 0, t < T, H, act, perm8, tokexp, any_scaled, threadIdx.x % 256, wmax[g]);
}

hipError_t launch_sort_pairs(const int32_t* idx, int T, int kcap, const int32_t* k_used_dev, int k_static, int E,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t st,
                             int capacity) {
  const int64_t P = (int64_t)T * kcap;
  const int64_t rounds = (P + 16 * 64 - 1) / (16 * 64);  // rounds of 64 pairs per wave
  if (rounds >= 16)
    (void)launch_kernel(sort_pairs_kernel<16>, E, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets,
                        perm, pos, capacity);
  else if (rounds >= 4)
    (void)launch_kernel(sort_pairs_kernel<4>, E, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets,
                        perm, pos, capacity);
  else
    (void)launch_kernel(sort_pairs_kernel<2>, E, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets,
                        perm, pos, capacity);
  return hipGetLastError();
}

hipError_t launch_sort_prep(const int32_t* idx, int T, int kcap, const int32_t* k_used_dev, int k_static, int E,
                            int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t st,
                            int capacity, const void* x, int act, uint16_t* a, int H, bool perm8, int32_t* tokexp,
                            int32_t* any_scaled) {
  if (act == ACT_BF16 && (!tokexp || !any_scaled)) return hipErrorInvalidValue;
  const int64_t P = (int64_t)T * kcap;
  const int64_t rounds = (P + 16 * 64 - 1) / (16 * 64);
  const unsigned grid = (unsigned)(E + (T + 3) / 4);
  const uint16_t* xs = (const uint16_t*)x;
  const int p8 = perm8 ? 1 : 0;
  if (rounds >= 16)
    (void)launch_kernel(sort_prep_kernel<16>, grid, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts,
                        offsets, perm, pos, capacity, xs, a, H, act, p8, tokexp, any_scaled);
  else if (rounds >= 4)
    (void)launch_kernel(sort_prep_kernel<4>, grid, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets,
                        perm, pos, capacity, xs, a, H, act, p8, tokexp, any_scaled);
  else
    (void)launch_kernel(sort_prep_kernel<2>, grid, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets,
                        perm, pos, capacity, xs, a, H, act, p8, tokexp, any_scaled);
  return hipGetLastError();
}

}  // namespace moe
