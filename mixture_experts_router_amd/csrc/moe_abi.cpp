// C ABI of the MoE layer: argument validation, workspace layout, path
// dispatch and launches on the caller's stream.  No device allocation, no
// synchronisation.  Every validation happens before the first HIP call, so
// invalid arguments return an error with nothing enqueued (and can be tested
// without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

using moe::WView;

constexpr size_t kAlign = 256;
constexpr int kGemvMaxPairs = 16;  // decode path when T*kcap <= this

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int kcap_of(int k) { return k > 0 ? k : MOE_K_ENTROPY_CAP; }

// ------------------------------------------------------------ profiling --

struct Prof {
  hipEvent_t const* ev = nullptr;
  int n = 0;
  int next = 0;
  std::string plan;
};
thread_local Prof g_prof;

}  // namespace

namespace moe {
bool next_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof.ev || g_prof.next + 1 >= g_prof.n) return false;
  *start = g_prof.ev[g_prof.next];
  *stop = g_prof.ev[g_prof.next + 1];
  g_prof.next += 2;
  return true;
}
}  // namespace moe

namespace {

void plan_begin(hipStream_t st) {
  (void)st;
  g_prof.plan.clear();
  g_prof.next = 0;
}

void plan_step(const char* name, hipStream_t st) {
  (void)st;
  if (!g_prof.plan.empty()) g_prof.plan += ",";
  g_prof.plan += name;
}

// ------------------------------------------------------- device properties

struct DevProps {
  bool ok = false;
  bool gfx950 = false;
  int num_cu = 0;
};

std::mutex g_props_mu;
DevProps g_props[64];

moe_status device_props(DevProps* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_props_mu);
  DevProps& p = g_props[dev];
  if (!p.ok) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    p.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    p.num_cu = prop.multiProcessorCount;
    p.ok = true;
  }
  *out = p;
  return p.gfx950 ? MOE_OK : MOE_ERR_DEVICE;
}

// ---------------------------------------------------- scratch workspace --
//
// The workspace of moe_layer_forward_noalloc: a file-scope device array.  In
// host code `scratch` names a host-side stand-in, not device memory, so the
// device address is looked up once per device (with that device current)
// and only that address is handed to kernels.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_addr[64];

moe_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_ERR_HIP;
    }
    if ((reinterpret_cast<uintptr_t>(p) & (kAlign - 1)) != 0) return MOE_ERR_INTERNAL;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

// ----------------------------------------------------------- validation --

// the library's width code of a tensor: 4/5/6/8/16, or NVF4
int wcode(const moe_weights* w) { return w->format == MOE_FMT_NVFP4 ? moe::NVF4 : w->bits; }

moe_status check_weights(const moe_weights* w, int E, int N, int K) {
  if (!w || !w->q) return MOE_ERR_NULL;
  if (w->format == MOE_FMT_NVFP4) {
    // E2M1 codes, E4M3 scales per 16 columns, a finite positive tensor scale, no biases
    if (w->bits != 4 || w->group_size != 16 || w->biases) return MOE_ERR_QUANT;
    if (!w->scales) return MOE_ERR_NULL;
    if (!(w->tensor_scale > 0.0f) || !std::isfinite(w->tensor_scale)) return MOE_ERR_QUANT;
  } else if (w->format != MOE_FMT_AFFINE) {
    return MOE_ERR_QUANT;
  } else {
    if (w->bits != 4 && w->bits != 5 && w->bits != 6 && w->bits != 8 && w->bits != 16) return MOE_ERR_QUANT;
    if (w->bits == 16) {
      if (w->scales || w->biases) return MOE_ERR_QUANT;
    } else {
      if (!w->scales || !w->biases) return MOE_ERR_NULL;
      if (w->group_size != 64) return MOE_ERR_QUANT;
    }
  }
  if (w->E != E || w->N != N || w->K != K) return MOE_ERR_SHAPE;
  if (w->K % 64 != 0 || w->expert_stride_rows < w->N) return MOE_ERR_SHAPE;
  if (!aligned16(w->q)) return MOE_ERR_ALIGN;
  if (w->bits != 16 && !aligned16(w->scales)) return MOE_ERR_ALIGN;
  if (w->biases && !aligned16(w->biases)) return MOE_ERR_ALIGN;
  if (w->packed_sb && w->bits == 16) return MOE_ERR_QUANT;  // packed_sb: quantised weights only
  if (w->packed_sb && !aligned16(w->packed_sb)) return MOE_ERR_ALIGN;
  if (w->packed_q) {
    if (!aligned16(w->packed_q)) return MOE_ERR_ALIGN;
    if (w->N % 32 != 0 || w->expert_stride_rows % 32 != 0) return MOE_ERR_SHAPE;  // whole 32-row blocks
  }
  return MOE_OK;
}

// Buffers sized by T (x, y, routing outputs) may be NULL when T == 0.
moe_status check_router(const void* x, moe_dtype dt, int T, int H, const void* wr, int E, int k) {
  if ((!x && T != 0) || !wr) return MOE_ERR_NULL;
  if (dt != MOE_F16 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (T < 0 || H <= 0 || H % 64 != 0) return MOE_ERR_SHAPE;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (k == MOE_K_ENTROPY) {
    if (E < MOE_K_ENTROPY_CAP) return MOE_ERR_K;
  } else if (k < 1 || k > MOE_MAX_K || k > E) {
    return MOE_ERR_K;
  }
  if ((T != 0 && !aligned16(x)) || !aligned16(wr)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// same_scale: NVFP4 tensors must also share the tensor scale (one fused tensor)
bool compatible(const moe_weights* a, const moe_weights* b, bool same_scale) {
  if (a->format != b->format) return false;
  if (same_scale && a->format == MOE_FMT_NVFP4 && a->tensor_scale != b->tensor_scale) return false;
  return a->bits == b->bits && a->group_size == b->group_size && a->E == b->E && a->N == b->N && a->K == b->K &&
         (a->scales == nullptr) == (b->scales == nullptr) && (a->biases == nullptr) == (b->biases == nullptr);
}

// ------------------------------------------------------------ workspace --

struct Layout {
  size_t logits, idx, w, scal, counts, offsets, perm, pos, h, o, a16, hent, tokexp, sbgu, sbd, g32, u32, total;
};

// Which regions a call needs: the batched path's GEMM operands, and the
// per-call repacks of scales and biases when the weights carry no packed_sb.
// moe_layer_workspace_size reserves all of them (it cannot know the path or
// the weights); a call lays out only what it uses.
struct Needs {
  bool batched = true, sb_gu = true, sb_d = true;
};

Layout layout(int64_t T, int64_t H, int64_t E, int64_t kcap, int64_t I, uint32_t flags, Needs nd = Needs{}) {
  Layout L{};
  const int64_t P = T * kcap;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    size_t r = at;
    at += align_up(bytes);
    return r;
  };
  L.logits = take((size_t)(T * E * 4));
  L.idx = take((size_t)(P * 4));
  L.w = take((size_t)(P * 4));
  L.scal = take(16);  // k_used, entropy, the flag of scaled bf16 tokens
  L.counts = take((size_t)(E * 4));
  L.offsets = take((size_t)((E + 1) * 4));
  L.perm = take((size_t)(P * 4));
  L.pos = take((size_t)(P * 4));
  L.h = take((size_t)(P * I * 2));
  L.hent = take((size_t)(T * 4));  // adaptive k: per-token entropies
  L.tokexp = take((size_t)(T * 4));  // bf16 activations: per-token exponents
  if (nd.batched) {
    L.o = take((size_t)(P * H * 2));
    L.a16 = take((size_t)(T * H * 2));  // the activations as the GEMM's fp16 operand
    // scales and biases repacked when the weights carry no packed_sb
    if (nd.sb_gu) L.sbgu = take((size_t)moe::packed_sb_bytes((int)E, 2 * I, (int)H));
    if (nd.sb_d) L.sbd = take((size_t)moe::packed_sb_bytes((int)E, H, (int)I));
  }
  if (flags & MOE_FLAG_UNFUSED) {
    L.g32 = take((size_t)(P * I * 4));
    L.u32 = take((size_t)(P * I * 4));
  }
  L.total = at;
  return L;
}

WView view_of(const moe_weights* w, int64_t row_offset) {
  WView v;
  const bool f4 = w->format == MOE_FMT_NVFP4;
  const int64_t rb = (int64_t)w->K * w->bits / 8;
  const int64_t srb = f4 ? w->K / 16 : (w->K / 64) * 2;  // scale bytes per row
  v.q = (const uint8_t*)w->q + row_offset * rb;
  v.s = w->scales ? (const uint16_t*)((const uint8_t*)w->scales + row_offset * srb) : nullptr;
  v.b = w->biases ? (const uint16_t*)((const uint8_t*)w->biases + row_offset * srb) : nullptr;
  v.stride = w->expert_stride_rows;
  v.sb = (const uint8_t*)w->packed_sb;
  v.sb_stride = w->expert_stride_rows;
  v.ts = f4 ? w->tensor_scale : 1.0f;
  if (w->packed_q) {
    const int code = f4 ? moe::NVF4 : w->bits;
    v.pq = (const uint8_t*)w->packed_q +
           row_offset / 32 * moe::packed_q_units(w->K, code) * 32 * moe::packed_q_unit_bytes(code);
    v.pq_expert = moe::packed_q_expert_bytes(w->expert_stride_rows, w->K, code);
  }
  return v;
}

#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// Routing options, checked: the correction vector and its scale, and the
// experts per selection group (1: plain top-k).
struct RouteOpt {
  const float* health = nullptr;
  float alpha = 0.0f;
  int gs = 1;
  int cap = 0;  // expert capacity (0: none)
};

moe_status check_opts(const moe_route_opts* o, int E, int k, RouteOpt* out) {
  *out = RouteOpt{};
  if (!o) return MOE_OK;
  if (o->health && (reinterpret_cast<uintptr_t>(o->health) & 3u) != 0) return MOE_ERR_ALIGN;
  if (o->groups < 0 || o->capacity < 0) return MOE_ERR_OPTION;
  out->cap = o->capacity;
  if (o->groups > 1) {
    if (E % o->groups != 0) return MOE_ERR_OPTION;
    const int need = k == MOE_K_ENTROPY ? MOE_K_ENTROPY_CAP : k;
    if (need > o->groups) return MOE_ERR_OPTION;
    out->gs = E / o->groups;
  }
  out->health = o->health;
  out->alpha = o->alpha;
  return MOE_OK;
}

// the selection launches: static top-k, or the adaptive pass (two launches
// with scratch for the per-token entropies, one without)
// (clear_word: see launch_topk)
moe_status select_impl(const float* logits, int T, int E, int k, int gs, int32_t* idx, float* w, int32_t* k_used,
                       float* entropy, float* scratch, hipStream_t st, int32_t* clear_word = nullptr) {
  HIP_TRY(moe::launch_topk(logits, T, E, k, gs, idx, w, k_used, entropy, scratch, st, clear_word));
  if (k <= 0 && scratch) plan_step("entropy_tokens", st);
  plan_step(k > 0 ? "topk" : "topk_entropy", st);
  return MOE_OK;
}

moe_status route_impl(const void* x, moe_dtype dt, int T, int H, const void* wr, int E, int k, const RouteOpt& ro,
                      int32_t* idx, float* w, int32_t* k_used, float* entropy, float* logits, float* scratch,
                      hipStream_t st, int32_t* clear_word = nullptr) {
  HIP_TRY(moe::launch_router_logits(x, wr, logits, T, H, E, (int)dt, ro.health, ro.alpha, st));
  plan_step("router_logits", st);
  return select_impl(logits, T, E, k, ro.gs, idx, w, k_used, entropy, scratch, st, clear_word);
}

moe_status scratch_ptr(void** out);

// use_scratch: the workspace is this device's file-scope scratch array (ws
// and ws_bytes ignored); a call that needs more returns MOE_ERR_SCRATCH.
moe_status forward_impl(const void* x, moe_dtype dt, int T, int H, const void* router_w, int E, int k,
                        const moe_route_opts* opts, const moe_weights* gate_up, const moe_weights* gate,
                        const moe_weights* up, const moe_weights* down, void* y, uint32_t flags,
                        const moe_taps* taps, void* ws, size_t ws_bytes, hipStream_t st, bool use_scratch = false) {
  // ---- validation (host only)
  moe_status s = check_router(x, dt, T, H, router_w, E, k);
  if (s != MOE_OK) return s;
  RouteOpt ro;
  if ((s = check_opts(opts, E, k, &ro)) != MOE_OK) return s;
  if ((!y && T != 0) || !down) return MOE_ERR_NULL;
  if (T != 0 && !aligned16(y)) return MOE_ERR_ALIGN;
  const int I = down->K;
  if (I <= 0 || I % 64 != 0) return MOE_ERR_SHAPE;
  if ((s = check_weights(down, E, H, I)) != MOE_OK) return s;
  WView wg, wu;
  if (gate_up) {
    if ((s = check_weights(gate_up, E, 2 * I, H)) != MOE_OK) return s;
    if (wcode(gate_up) != wcode(down)) return MOE_ERR_QUANT;
    wg = view_of(gate_up, 0);
    wu = view_of(gate_up, I);
  } else {
    if (!gate || !up) return MOE_ERR_NULL;
    if (!compatible(gate, up, false)) return MOE_ERR_INCOMPATIBLE;
    // the fused GEMM reads gate and up columns in one layout
    if ((gate->packed_q == nullptr) != (up->packed_q == nullptr)) return MOE_ERR_INCOMPATIBLE;
    if ((s = check_weights(gate, E, I, H)) != MOE_OK) return s;
    if ((s = check_weights(up, E, I, H)) != MOE_OK) return s;
    if (wcode(gate) != wcode(down)) return MOE_ERR_QUANT;
    wg = view_of(gate, 0);
    wu = view_of(up, 0);
  }
  const int bits = wcode(down);  // NVFP4 weights: moe::NVF4
  const int kcap = kcap_of(k);
  const int64_t P = (int64_t)T * kcap;
  const bool gemv_fits = moe::gemv_lanes_chunks(H, bits) <= 4 && moe::gemv_down_fits(I, bits, kcap);
  bool gemv = false;
  if (!(flags & MOE_FLAG_FORCE_MFMA)) gemv = gemv_fits && ((flags & MOE_FLAG_FORCE_GEMV) || P <= kGemvMaxPairs);
  Needs nd;
  nd.batched = !gemv;
  nd.sb_gu = bits != 16 && !(gate_up && gate_up->packed_sb);
  nd.sb_d = bits != 16 && !down->packed_sb;
  const Layout L = layout(T, H, E, kcap, I, flags, nd);
  if (T == 0) return MOE_OK;
  // 5-bit rows on the batched path: two-group (80-byte) stages of both GEMMs
  if (bits == 5 && !gemv && (H % 128 != 0 || I % 128 != 0)) return MOE_ERR_QUANT;
  if (use_scratch) {
    if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  } else {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_ERR_ALIGN;
  }

  // ---- device
  DevProps props;
  if ((s = device_props(&props)) != MOE_OK) return s;
  if (use_scratch && (s = scratch_ptr(&ws)) != MOE_OK) return s;

  uint8_t* W = (uint8_t*)ws;
  float* logits = (taps && taps->logits) ? taps->logits : (float*)(W + L.logits);
  int32_t* idx = (int32_t*)(W + L.idx);
  float* wts = (float*)(W + L.w);
  int32_t* k_used = (int32_t*)(W + L.scal);
  float* entropy = (float*)(W + L.scal + 4);
  int32_t* counts = (int32_t*)(W + L.counts);
  int32_t* offsets = (int32_t*)(W + L.offsets);
  int32_t* perm = (int32_t*)(W + L.perm);
  int32_t* pos = (int32_t*)(W + L.pos);
  uint16_t* h = (uint16_t*)(W + L.h);
  uint16_t* o = (uint16_t*)(W + L.o);
  uint16_t* a16w = (uint16_t*)(W + L.a16);
  float* g32 = (float*)(W + L.g32);
  // bf16 activations reach the fp16 operands as x * 2^-a_t per token
  int32_t* tokexp = dt == MOE_BF16 ? (int32_t*)(W + L.tokexp) : nullptr;
  int32_t* any_scaled = (int32_t*)(W + L.scal + 8);
  float* u32 = (float*)(W + L.u32);
  const bool unfused = (flags & MOE_FLAG_UNFUSED) != 0;
  const int act = (int)dt;
  (void)pos;

  const bool want_sort_taps = taps && (taps->counts || taps->offsets || taps->perm);
  float* pre_tap = taps ? taps->gate_up_preact : nullptr;
  const int k_static = k > 0 ? k : 0;

  plan_begin(st);
  if (gemv) {
    // decode path: with static k the GEMV kernels select the experts from the
    // logits themselves (no separate selection launch)
    HIP_TRY(moe::launch_router_logits(x, router_w, logits, T, H, E, act, ro.health, ro.alpha, st));
    plan_step("router_logits", st);
    moe::GemvRoute rt{logits, E, idx, wts, k_used, entropy, ro.gs};
    if (k <= 0) {
      moe_status s2 = select_impl(logits, T, E, k, ro.gs, idx, wts, k_used, entropy, (float*)(W + L.hent), st);
      if (s2 != MOE_OK) return s2;
      rt.logits = nullptr;
    }
    if (!unfused) {
      HIP_TRY(moe::launch_gemv_up(x, act, rt, k_static, kcap, T, H, I, bits, true, wg, wu, h, nullptr, props.num_cu,
                                  st, pre_tap, tokexp));
      plan_step("gemv_gate_up_swiglu", st);
    } else {
      HIP_TRY(moe::launch_gemv_up(x, act, rt, k_static, kcap, T, H, I, bits, false, wg, wg, nullptr, g32,
                                  props.num_cu, st, nullptr, tokexp));
      plan_step("gemv_gate", st);
      HIP_TRY(moe::launch_gemv_up(x, act, rt, k_static, kcap, T, H, I, bits, false, wu, wu, nullptr, u32,
                                  props.num_cu, st, nullptr, tokexp));
      plan_step("gemv_up", st);
      HIP_TRY(moe::launch_swiglu(g32, u32, h, P, I, false, st, tokexp, nullptr, kcap));
      plan_step("swiglu", st);
      if (pre_tap) {
        HIP_TRY(moe::launch_gather_preact(g32, u32, nullptr, P, I, pre_tap, kcap, k_used, k_static, st));
        plan_step("gather_preact", st);
      }
    }
    // the gate+up kernel wrote the selection: the down kernel reads it
    // instead of selecting again
    moe::GemvRoute rt_down = rt;
    rt_down.logits = nullptr;
    HIP_TRY(moe::launch_gemv_down(h, rt_down, k_static, kcap, T, H, I, bits, view_of(down, 0), y, act, props.num_cu,
                                  st, ro.cap, tokexp));
    plan_step("gemv_down_combine", st);
    if (want_sort_taps) {
      HIP_TRY(moe::launch_sort_pairs(idx, T, kcap, k_used, k_static, E, counts, offsets, perm, pos, st, ro.cap));
      plan_step("sort_pairs", st);
    }
  } else {
    // the selection also clears the flag that the operand conversion raises
    // for scaled bf16 tokens
    if ((s = route_impl(x, dt, T, H, router_w, E, k, ro, idx, wts, k_used, entropy, logits, (float*)(W + L.hent),
                        st, any_scaled)) != MOE_OK)
      return s;
    const int bm = moe::gemm_block_m((int)P, E);
    const int mt = moe::gemm_max_mtiles((int)P, E, bm);
    // the GEMM operand: fp16 activations, 8-element blocks in 4-bit unpack
    // order for affine 4-bit codes (NVFP4 codes unpack in column order),
    // converted in the sort's launch
    const bool perm8 = bits == 4;
    const uint16_t* a16 = (const uint16_t*)x;
    if (perm8 || dt != MOE_F16) {
      HIP_TRY(moe::launch_sort_prep(idx, T, kcap, k_used, k_static, E, counts, offsets, perm, pos, st, ro.cap, x, act,
                                    a16w, H, perm8, tokexp, any_scaled));
      plan_step("sort_pairs_prep_a", st);
      a16 = a16w;
    } else {
      HIP_TRY(moe::launch_sort_pairs(idx, T, kcap, k_used, k_static, E, counts, offsets, perm, pos, st, ro.cap));
      plan_step("sort_pairs", st);
    }
    // the gate and up scales in one packed_sb, up rows inter rows after gate
    // rows (the GEMM reads both halves with one descriptor)
    if (bits != 16 && !(gate_up && gate_up->packed_sb)) {
      uint8_t* sb = W + L.sbgu;
      HIP_TRY(moe::launch_pack_sb(wg.s, wg.b, E, I, H, wg.stride, sb, 2 * I, 0, st, bits == moe::NVF4));
      plan_step("pack_sb_gate", st);
      HIP_TRY(moe::launch_pack_sb(wu.s, wu.b, E, I, H, wu.stride, sb, 2 * I, I, st, bits == moe::NVF4));
      plan_step("pack_sb_up", st);
      wg.sb = sb;
      wu.sb = sb + (size_t)I * 8;
      wg.sb_stride = wu.sb_stride = 2 * I;
    } else if (bits != 16) {
      wu.sb = wg.sb + (size_t)I * 8;  // the fused tensor's packed_sb, up half
    }
    if (!unfused) {
      HIP_TRY(moe::launch_gemm(moe::GEMM_FUSED_SWIGLU, a16, T, perm, counts, offsets, kcap, E, H, I, bits, wg, wu, h,
                               perm8, bm, mt, st, pre_tap, tokexp, any_scaled));
      plan_step("gemm_gate_up_swiglu", st);
    } else {
      HIP_TRY(moe::launch_gemm(moe::GEMM_GATHER_F32, a16, T, perm, counts, offsets, kcap, E, H, I, bits, wg, wg, g32,
                               false, bm, mt, st, nullptr, tokexp, any_scaled));
      plan_step("gemm_gate", st);
      HIP_TRY(moe::launch_gemm(moe::GEMM_GATHER_F32, a16, T, perm, counts, offsets, kcap, E, H, I, bits, wu, wu, u32,
                               false, bm, mt, st, nullptr, tokexp, any_scaled));
      plan_step("gemm_up", st);
      HIP_TRY(moe::launch_swiglu(g32, u32, h, P, I, perm8, st, tokexp, perm, kcap));
      plan_step("swiglu", st);
      if (pre_tap) {
        HIP_TRY(moe::launch_gather_preact(g32, u32, pos, P, I, pre_tap, kcap, k_used, k_static, st));
        plan_step("gather_preact", st);
      }
    }
    WView wd = view_of(down, 0);
    if (bits != 16 && !wd.sb) {
      uint8_t* sb = W + L.sbd;
      HIP_TRY(moe::launch_pack_sb(wd.s, wd.b, E, H, I, wd.stride, sb, H, 0, st, bits == moe::NVF4));
      plan_step("pack_sb_down", st);
      wd.sb = sb;
      wd.sb_stride = H;
    }
    HIP_TRY(moe::launch_gemm(moe::GEMM_ROWS_F16, h, P, perm, counts, offsets, kcap, E, I, H, bits, wd, wd, o, false, bm,
                             mt, st));
    plan_step("gemm_down", st);
    HIP_TRY(moe::launch_combine(o, pos, wts, k_used, k_static, kcap, T, H, y, act, st, tokexp));
    plan_step("combine", st);
  }

  // ---- taps (copies only)
  if (taps) {
    if (taps->topk_idx) HIP_TRY(moe::launch_copy_words(idx, taps->topk_idx, P, st));
    if (taps->topk_w) HIP_TRY(moe::launch_copy_words(wts, taps->topk_w, P, st));
    if (taps->k_used) HIP_TRY(moe::launch_copy_words(k_used, taps->k_used, 1, st));
    if (taps->entropy) HIP_TRY(moe::launch_copy_words(entropy, taps->entropy, 1, st));
    if (taps->counts) HIP_TRY(moe::launch_copy_words(counts, taps->counts, E, st));
    if (taps->offsets) HIP_TRY(moe::launch_copy_words(offsets, taps->offsets, E + 1, st));
    if (taps->perm) HIP_TRY(moe::launch_copy_words(perm, taps->perm, P, st));
    if (taps->h) {
      if (gemv)
        HIP_TRY(moe::launch_gather_rows(h, nullptr, P, I, (uint16_t*)taps->h, kcap, k_used, k_static, false, st));
      else
        HIP_TRY(moe::launch_gather_rows(h, pos, P, I, (uint16_t*)taps->h, kcap, k_used, k_static, bits == 4, st));
    }
  }
  return MOE_OK;
}

}  // namespace

namespace moe {
namespace {
int g_tuning[TUNE_KEYS] = {8, 8, 1 << 30, 1, 2, 2, 1, 8, 1, 2};
}
int tuning(TuneKey key) { return g_tuning[key]; }
void set_tuning(int key, int value) {
  if (key >= 0 && key < TUNE_KEYS && value > 0) g_tuning[key] = value;
}
}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_DTYPE: return "unknown activation dtype";
    case MOE_ERR_ALIGN: return "a pointer is not suitably aligned";
    case MOE_ERR_K: return "k out of range";
    case MOE_ERR_QUANT: return "unsupported quantisation (bits, group size or scale presence)";
    case MOE_ERR_INCOMPATIBLE: return "gate and up cannot be fused";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "no usable gfx950 device is current";
    case MOE_ERR_HIP: return "a HIP call failed";
    case MOE_ERR_INTERNAL: return "internal error";
    case MOE_ERR_OPTION: return "a routing option is out of range";
    case MOE_ERR_SCRATCH:
      return "the call needs more workspace than the allocation-free entry point holds "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1) return 0;
  // logits, then (adaptive k) the per-token entropies
  return align_up((size_t)T * (size_t)E * 4) + (k == MOE_K_ENTROPY ? align_up((size_t)T * 4) : 0);
}

moe_status moe_route(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E, int32_t k,
                     int32_t* topk_idx, float* topk_w, int32_t* k_used, float* entropy, float* logits_out, void* ws,
                     size_t ws_bytes, void* stream) {
  return moe_route_ex(x, dt, T, H, router_w, E, k, nullptr, topk_idx, topk_w, k_used, entropy, logits_out, ws,
                      ws_bytes, stream);
}

moe_status moe_route_ex(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                        int32_t k, const moe_route_opts* opts, int32_t* topk_idx, float* topk_w, int32_t* k_used,
                        float* entropy, float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  try {
    moe_status s = check_router(x, dt, T, H, router_w, E, k);
    if (s != MOE_OK) return s;
    RouteOpt ro;
    if ((s = check_opts(opts, E, k, &ro)) != MOE_OK) return s;
    if (ro.cap) return MOE_ERR_OPTION;  // capacity is a dispatch option: moe_layer_forward_ex only
    if (T == 0) return MOE_OK;
    if (!topk_idx || !topk_w) return MOE_ERR_NULL;
    float* logits = logits_out;
    float* scratch = nullptr;
    if (!logits || ws) {
      if (!ws) return MOE_ERR_WORKSPACE;
      if (ws_bytes < moe_route_workspace_size(T, E, k)) return MOE_ERR_WORKSPACE;
      if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return MOE_ERR_ALIGN;
      if (!logits) logits = (float*)ws;
      if (k == MOE_K_ENTROPY) scratch = (float*)((char*)ws + align_up((size_t)T * (size_t)E * 4));
    }
    DevProps props;
    if ((s = device_props(&props)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    return route_impl(x, dt, T, H, router_w, E, k, ro, topk_idx, topk_w, k_used, entropy, logits, scratch, st);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_topk_from_logits(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                                float* topk_w, int32_t* k_used, float* entropy, void* ws, size_t ws_bytes,
                                void* stream) {
  return moe_topk_from_logits_ex(logits, T, E, k, nullptr, topk_idx, topk_w, k_used, entropy, ws, ws_bytes, stream);
}

moe_status moe_topk_from_logits_ex(const float* logits, int32_t T, int32_t E, int32_t k, const moe_route_opts* opts,
                                   int32_t* topk_idx, float* topk_w, int32_t* k_used, float* entropy, void* ws,
                                   size_t ws_bytes, void* stream) {
  try {
    (void)ws;
    (void)ws_bytes;
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if (T != 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_NULL;
    if (k == MOE_K_ENTROPY) {
      if (E < MOE_K_ENTROPY_CAP) return MOE_ERR_K;
    } else if (k < 1 || k > MOE_MAX_K || k > E) {
      return MOE_ERR_K;
    }
    RouteOpt ro;
    moe_status so = check_opts(opts, E, k, &ro);
    if (so != MOE_OK) return so;
    if (ro.health || ro.cap) return MOE_ERR_OPTION;
    if (T == 0) return MOE_OK;
    DevProps props;
    moe_status s = device_props(&props);
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    if (moe::launch_topk(logits, T, E, k, ro.gs, topk_idx, topk_w, k_used, entropy, nullptr, st) != hipSuccess)
      return MOE_ERR_HIP;
    plan_step(k > 0 ? "topk" : "topk_entropy", st);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, int32_t inter, uint32_t flags) {
  if (T < 0 || H < 0 || E < 1 || inter < 0) return 0;
  return layout(T, H, E, kcap_of(k), inter, flags).total;
}

moe_status moe_layer_forward(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                             int32_t k, const moe_weights* gate_up, const moe_weights* gate, const moe_weights* up,
                             const moe_weights* down, void* y, uint32_t flags, const moe_taps* taps, void* ws,
                             size_t ws_bytes, void* stream) {
  try {
    return forward_impl(x, dt, T, H, router_w, E, k, nullptr, gate_up, gate, up, down, y, flags, taps, ws, ws_bytes,
                        (hipStream_t)stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_layer_forward_ex(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                                int32_t k, const moe_route_opts* opts, const moe_weights* gate_up,
                                const moe_weights* gate, const moe_weights* up, const moe_weights* down, void* y,
                                uint32_t flags, const moe_taps* taps, void* ws, size_t ws_bytes, void* stream) {
  try {
    return forward_impl(x, dt, T, H, router_w, E, k, opts, gate_up, gate, up, down, y, flags, taps, ws, ws_bytes,
                        (hipStream_t)stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_layer_forward_noalloc(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w,
                                     int32_t E, int32_t k, const moe_route_opts* opts, const moe_weights* gate_up,
                                     const moe_weights* gate, const moe_weights* up, const moe_weights* down,
                                     void* y, uint32_t flags, const moe_taps* taps, void* stream) {
  try {
    return forward_impl(x, dt, T, H, router_w, E, k, opts, gate_up, gate, up, down, y, flags, taps, nullptr, 0,
                        (hipStream_t)stream, true);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_load_stats(const int32_t* counts, int32_t E, int32_t* least_used, float* stddev,
                                 void* stream) {
  try {
    if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if (!counts || !least_used || !stddev) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(counts) & 3u) || (reinterpret_cast<uintptr_t>(least_used) & 3u) ||
        (reinterpret_cast<uintptr_t>(stddev) & 3u))
      return MOE_ERR_ALIGN;
    DevProps props;
    moe_status s = device_props(&props);
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    HIP_TRY(moe::launch_load_stats(counts, E, least_used, stddev, st));
    plan_step("load_stats", st);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

size_t moe_packed_sb_bytes(int32_t E, int64_t expert_stride_rows, int32_t K) {
  if (E < 1 || expert_stride_rows < 1 || K < 64 || K % 64 != 0) return 0;
  return (size_t)moe::packed_sb_bytes(E, expert_stride_rows, K);
}

moe_status moe_pack_sb(const moe_weights* w, void* out, void* stream) {
  if (!w || !out) return MOE_ERR_NULL;
  if (w->bits == 16) return MOE_ERR_QUANT;  // packed_sb holds scales and biases
  moe_status s = check_weights(w, w->E, w->N, w->K);
  if (s != MOE_OK) return s;
  if (!aligned16(out)) return MOE_ERR_ALIGN;
  DevProps props;
  if ((s = device_props(&props)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  plan_begin(st);
  HIP_TRY(moe::launch_pack_sb((const uint16_t*)w->scales, (const uint16_t*)w->biases, w->E, w->N, w->K,
                              w->expert_stride_rows, (uint8_t*)out, w->expert_stride_rows, 0, st,
                              w->format == MOE_FMT_NVFP4));
  plan_step("pack_sb", st);
  return MOE_OK;
}

size_t moe_packed_q_bytes(int32_t E, int64_t expert_stride_rows, int32_t K, int32_t bits) {
  if (E < 1 || expert_stride_rows < 32 || expert_stride_rows % 32 != 0 || K < 64 || K % 64 != 0) return 0;
  if (bits != 4 && bits != 5 && bits != 6 && bits != 8 && bits != 16) return 0;
  return (size_t)E * (size_t)moe::packed_q_expert_bytes(expert_stride_rows, K, bits);
}

moe_status moe_pack_q(const moe_weights* w, void* out, void* stream) {
  try {
    if (!w || !out) return MOE_ERR_NULL;
    moe_status s = check_weights(w, w->E, w->N, w->K);
    if (s != MOE_OK) return s;
    if (w->N % 32 != 0 || w->expert_stride_rows % 32 != 0) return MOE_ERR_SHAPE;
    if (!aligned16(out)) return MOE_ERR_ALIGN;
    DevProps props;
    if ((s = device_props(&props)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    HIP_TRY(moe::launch_pack_q((const uint8_t*)w->q, w->E, w->N, w->K, wcode(w), w->expert_stride_rows,
                               (uint8_t*)out, w->expert_stride_rows, st));
    plan_step("pack_q", st);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_fuse_gate_up(const moe_weights* gate, const moe_weights* up, void* q_out, void* s_out, void* b_out,
                            void* stream) {
  try {
    if (!gate || !up || !gate->q || !up->q || !q_out) return MOE_ERR_NULL;
    if (!compatible(gate, up, true)) return MOE_ERR_INCOMPATIBLE;
    moe_status s = check_weights(gate, gate->E, gate->N, gate->K);
    if (s != MOE_OK) return s;
    if ((s = check_weights(up, gate->E, gate->N, gate->K)) != MOE_OK) return s;
    const bool f4 = gate->format == MOE_FMT_NVFP4;
    const bool quant = gate->bits != 16;
    const bool has_b = quant && !f4;  // NVFP4 weights have no biases
    if (quant && !s_out) return MOE_ERR_NULL;
    if (has_b && !b_out) return MOE_ERR_NULL;
    if ((!quant && s_out) || (!has_b && b_out)) return MOE_ERR_QUANT;
    if (!aligned16(q_out) || (quant && !aligned16(s_out)) || (has_b && !aligned16(b_out))) return MOE_ERR_ALIGN;
    DevProps props;
    if ((s = device_props(&props)) != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    const size_t E = (size_t)gate->E, I = (size_t)gate->N;
    const size_t rb = (size_t)gate->K * gate->bits / 8, sb = f4 ? (size_t)gate->K / 16 : (size_t)(gate->K / 64) * 2;
    struct Part {
      void* dst;
      const void* src;
      size_t row, sstride;
    };
    Part parts[6] = {{q_out, gate->q, rb, (size_t)gate->expert_stride_rows},
                     {(uint8_t*)q_out + I * rb, up->q, rb, (size_t)up->expert_stride_rows},
                     {s_out, gate->scales, sb, (size_t)gate->expert_stride_rows},
                     {(uint8_t*)s_out + I * sb, up->scales, sb, (size_t)up->expert_stride_rows},
                     {b_out, gate->biases, sb, (size_t)gate->expert_stride_rows},
                     {(uint8_t*)b_out + I * sb, up->biases, sb, (size_t)up->expert_stride_rows}};
    const int nparts = has_b ? 6 : (quant ? 4 : 2);
    for (int i = 0; i < nparts; ++i) {
      const Part& p = parts[i];
      // E blocks of I rows; destination experts are 2*I rows apart
      if (hipMemcpy2DAsync(p.dst, 2 * I * p.row, p.src, p.sstride * p.row, I * p.row, E, hipMemcpyDeviceToDevice,
                           st) != hipSuccess) {
        (void)hipGetLastError();
        for (size_t e = 0; e < E; ++e)
          if (hipMemcpyAsync((uint8_t*)p.dst + e * 2 * I * p.row, (const uint8_t*)p.src + e * p.sstride * p.row,
                             I * p.row, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return MOE_ERR_HIP;
      }
    }
    plan_step("fuse_gate_up_copy", st);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

void moe_debug_set_events(void* const* events, int32_t n) {
  g_prof.ev = (hipEvent_t const*)events;
  g_prof.n = events ? n : 0;
  g_prof.next = 0;
}

void moe_debug_set_tuning(int32_t key, int32_t value) { moe::set_tuning(key, value); }

moe_status moe_debug_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  try {
    if (!src || !sink) return MOE_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MOE_ERR_ALIGN;
    if (bytes == 0 || bytes % 16 != 0 || bytes >= (size_t(1) << 32)) return MOE_ERR_SHAPE;
    DevProps props;
    moe_status s = device_props(&props);
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    plan_begin(st);
    HIP_TRY(moe::launch_stream_read(src, (uint32_t)bytes, sink, st));
    plan_step("stream_read", st);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

int32_t moe_debug_last_plan(char* buf, size_t buf_bytes) {
  const std::string& p = g_prof.plan;
  if (buf && buf_bytes > 0) {
    size_t n = std::min(buf_bytes - 1, p.size());
    std::memcpy(buf, p.data(), n);
    buf[n] = 0;
  }
  return (int32_t)p.size();
}

}  // extern "C"
