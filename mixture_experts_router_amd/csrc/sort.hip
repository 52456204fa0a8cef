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

__global__ __launch_bounds__(1024) void sort_pairs_kernel(const int32_t* __restrict__ idx, int T, int kcap,
                                                          const int32_t* __restrict__ k_used_dev, int k_static, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ pos, int cap) {
  __shared__ int s_lt[16], s_eq[16];
  __shared__ int hist[MOE_MAX_EXPERTS_DEV];
  const int e = blockIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int ku = k_used_dev ? *k_used_dev : k_static;
  const int64_t P = (int64_t)T * kcap;
  const int64_t seg = ((P + 16 * 64 - 1) / (16 * 64)) * 64;
  const int64_t beg = wave * seg;
  const int64_t end = beg + seg < P ? beg + seg : P;

  int lt = 0, eq = 0;
  for (int64_t c = beg; c < end; c += 64) {
    int64_t p = c + lane;
    bool valid = p < end && (int)(p % kcap) < ku;
    int v = valid ? idx[p] : 0x7FFFFFFF;
    lt += __popcll(__ballot(v < e));
    eq += __popcll(__ballot(v == e));
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
  for (int64_t c = beg; c < end; c += 64) {
    int64_t p = c + lane;
    bool valid = p < end && (int)(p % kcap) < ku;
    int v = valid ? idx[p] : 0x7FFFFFFF;
    uint64_t m = __ballot(v == e);
    if (v == e) {
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

hipError_t launch_sort_pairs(const int32_t* idx, int T, int kcap, const int32_t* k_used_dev, int k_static, int E,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t st,
                             int capacity) {
  (void)launch_kernel(sort_pairs_kernel, E, 1024, 0, st, idx, T, kcap, k_used_dev, k_static, E, counts, offsets, perm, pos,
                capacity);
  return hipGetLastError();
}

}  // namespace moe
