// Host side of the MoE decode C ABI: descriptor validation, layouts, the
// lossless NVFP4 / bf16 packers, the layer handle and its workspace, and the
// launch sequence of one layer call.  Declarations: include/moe_decode.h.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "moe_internal.h"

using moe::MatGeom;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
  MatGeom g13, g2;
  int Er, maxd, n_router_blocks, wpe13, s3;
};

// Full check of a description; fills the kernel plan on success.
int plan_layer(const moe_layer_desc* d, Plan* p) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  const int H = d->hidden, I = d->inter, E = d->n_routed, k = d->top_k, S = d->n_shared;
  if (H <= 0 || I <= 0 || E <= 0 || k <= 0 || S < 0 || d->max_batch <= 0) return MOE_ERR_INVALID_ARG;
  if (d->routed_wtype != MOE_W_NVFP4 && d->routed_wtype != MOE_W_BF16) return MOE_ERR_INVALID_ARG;
  if (d->shared_wtype != MOE_W_NVFP4 && d->shared_wtype != MOE_W_BF16) return MOE_ERR_INVALID_ARG;
  if (d->route != MOE_ROUTE_SIGMOID_TOPK && d->route != MOE_ROUTE_SOFTMAX_SINK) return MOE_ERR_INVALID_ARG;
  if (k > E) return MOE_ERR_INVALID_ARG;
  if (d->prenorm_gamma != nullptr && !(d->rms_eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (d->max_batch > MOE_MAX_BATCH) return MOE_ERR_UNSUPPORTED;
  if (H % 32 || I % 32 || H > 8192 || I > 2048) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_ROUTED || k > MOE_MAX_TOPK || S > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  if (d->routed_wtype == MOE_W_BF16 && d->shared_wtype == MOE_W_NVFP4) return MOE_ERR_UNSUPPORTED;
  if (d->router_bias != nullptr && d->route != MOE_ROUTE_SIGMOID_TOPK) return MOE_ERR_UNSUPPORTED;
  const int Er = E + (d->route == MOE_ROUTE_SOFTMAX_SINK ? S : 0);
  if (Er > MOE_MAX_ROUTED) return MOE_ERR_UNSUPPORTED;
  if (d->prenorm_gamma != nullptr && !aligned16(d->prenorm_gamma)) return MOE_ERR_ALIGNMENT;
  if (d->router_bias != nullptr && (reinterpret_cast<uintptr_t>(d->router_bias) & 3u)) return MOE_ERR_ALIGNMENT;

  if (moe::make_geom(2 * I, H, &p->g13) || moe::make_geom(H, I, &p->g2)) return MOE_ERR_UNSUPPORTED;
  if (p->g2.ns != 1) return MOE_ERR_UNSUPPORTED;
  if (I % p->g13.rpw) return MOE_ERR_UNSUPPORTED;
  const int gate_steps = I / p->g13.rpw;
  const int nrg = moe::kWaves / p->g13.ns;
  if (gate_steps % (moe::kGateSteps * nrg)) return MOE_ERR_UNSUPPORTED;
  p->wpe13 = gate_steps / (moe::kGateSteps * nrg);
  // down kernel: steps per workgroup; its LDS tile holds 8 * s3 * rpw floats per wave
  p->s3 = (p->g2.nsteps % 8 == 0 && p->g2.nsteps / 8 >= 512 && 8 * 8 * p->g2.rpw <= 1024) ? 8 : 2;
  if (8 * p->s3 * p->g2.rpw > 1024) return MOE_ERR_UNSUPPORTED;
  p->Er = Er;
  p->maxd = (d->max_batch * k < E) ? d->max_batch * k : E;
  p->n_router_blocks = (Er + moe::kWaves - 1) / moe::kWaves;
  return MOE_OK;
}

int layout(int wtype, int H, int I, int n, moe_expert_layout* o) {
  if (o == nullptr || H <= 0 || I <= 0 || n < 0 || H % 32 || I % 32) return MOE_ERR_INVALID_ARG;
  memset(o, 0, sizeof(*o));
  const size_t IH = (size_t)I * H;
  if (wtype == MOE_W_NVFP4) {
    o->w13_code_bytes = IH;           // 2I * H / 2
    o->w2_code_bytes = IH / 2;        // H * I / 2
    o->w13_scale_bytes = IH / 8;      // 2I * H / 16
    o->w2_scale_bytes = IH / 16;      // H * I / 16
  } else if (wtype == MOE_W_BF16) {
    o->w13_code_bytes = IH * 4;       // 2I * H * 2
    o->w2_code_bytes = IH * 2;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  o->code_stride = o->w13_code_bytes + o->w2_code_bytes;
  o->code_region_bytes = o->code_stride * (size_t)n;
  o->scale_stride = o->w13_scale_bytes + o->w2_scale_bytes;
  if (wtype == MOE_W_NVFP4) {
    o->tensor_scale_offset = align_up(o->scale_stride * (size_t)n, kAlign);
    o->scale_region_bytes = o->tensor_scale_offset + (size_t)n * 2 * sizeof(float);
  }
  o->shared_scale_offset = align_up(o->code_region_bytes, kAlign);
  o->shared_total_bytes = o->shared_scale_offset + o->scale_region_bytes;
  return MOE_OK;
}

// Matrices the packers accept: a geometry must exist for them.
int pack_geom(int rows, int cols, MatGeom* g) {
  if (rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (moe::make_geom(rows, cols, g)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

struct moe_layer {
  moe_layer_desc d;
  Plan p;
  moe_expert_layout lr, ls;
  int device;
  void* ws;
  size_t ws_bytes;
  unsigned* counter;
  float* logits;
  int* rt_nd;
  int* rt_ids;
  unsigned* rt_mask;
  float* rt_wt;
  int* topk_ids;
  float* topk_w;
  float* shared_c;
  uint16_t* xhat;
  uint16_t* h_routed;
  uint16_t* h_shared;
  int last_batch;
  const void* last_x;
  std::vector<void*> prof;       // profiling events (caller-owned)
  unsigned long long prof_call;
};

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or combination";
    case MOE_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case MOE_ERR_BATCH: return "batch outside [1, max_batch]";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_DEVICE: return "device allocation or query failed";
    case MOE_ERR_STATE: return "no layer call yet on this handle";
    default: return "unknown status";
  }
}

int moe_layer_validate(const moe_layer_desc* desc) {
  Plan p;
  return plan_layer(desc, &p);
}

int moe_expert_layout_query(int wtype, int hidden, int inter, int n_experts, moe_expert_layout* out) {
  return layout(wtype, hidden, inter, n_experts, out);
}

int moe_pack_nvfp4(int rows, int cols, const uint8_t* codes, const uint8_t* scales, uint8_t* codes_out,
                   uint8_t* scales_out) {
  if (!codes || !scales || !codes_out || !scales_out) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  const size_t crow = (size_t)cols / 2, srow = (size_t)cols / 16;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int ri = 0; ri < g.rpw; ++ri)
        for (int j = 0; j < g.cw; ++j) {
          const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
          memcpy(codes_out + moe::code_unit(g, s, t, ri, j) * 16, codes + row * crow + cc * 16, 16);
          memcpy(scales_out + moe::scale_word(g, s, t, ri, j) + 2 * (t & 1), scales + row * srow + cc * 2, 2);
        }
  return MOE_OK;
}

int moe_unpack_nvfp4(int rows, int cols, const uint8_t* codes_packed, const uint8_t* scales_packed,
                     uint8_t* codes, uint8_t* scales) {
  if (!codes || !scales || !codes_packed || !scales_packed) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  const size_t crow = (size_t)cols / 2, srow = (size_t)cols / 16;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int ri = 0; ri < g.rpw; ++ri)
        for (int j = 0; j < g.cw; ++j) {
          const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
          memcpy(codes + row * crow + cc * 16, codes_packed + moe::code_unit(g, s, t, ri, j) * 16, 16);
          memcpy(scales + row * srow + cc * 2, scales_packed + moe::scale_word(g, s, t, ri, j) + 2 * (t & 1), 2);
        }
  return MOE_OK;
}

int moe_pack_bf16(int rows, int cols, const uint16_t* w, uint16_t* w_out) {
  if (!w || !w_out) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int sub = 0; sub < 4; ++sub)
        for (int ri = 0; ri < g.rpw; ++ri)
          for (int j = 0; j < g.cw; ++j) {
            const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
            memcpy(w_out + moe::bf16_unit(g, s, t, sub, ri, j) * 8, w + row * cols + cc * 32 + sub * 8, 16);
          }
  return MOE_OK;
}

int moe_unpack_bf16(int rows, int cols, const uint16_t* w_packed, uint16_t* w) {
  if (!w || !w_packed) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int sub = 0; sub < 4; ++sub)
        for (int ri = 0; ri < g.rpw; ++ri)
          for (int j = 0; j < g.cw; ++j) {
            const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
            memcpy(w + row * cols + cc * 32 + sub * 8, w_packed + moe::bf16_unit(g, s, t, sub, ri, j) * 8, 16);
          }
  return MOE_OK;
}

int moe_layer_create(const moe_layer_desc* desc, moe_layer_t* out) {
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  Plan p;
  if (int st = plan_layer(desc, &p)) return st;
  moe_layer* L = new (std::nothrow) moe_layer();
  if (L == nullptr) return MOE_ERR_DEVICE;
  L->d = *desc;
  L->p = p;
  layout(desc->routed_wtype, desc->hidden, desc->inter, desc->n_routed, &L->lr);
  layout(desc->shared_wtype, desc->hidden, desc->inter, desc->n_shared, &L->ls);
  if (hipGetDevice(&L->device) != hipSuccess) {
    delete L;
    return MOE_ERR_DEVICE;
  }
  const size_t maxB = desc->max_batch, H = desc->hidden, I = desc->inter, k = desc->top_k;
  const size_t S1 = desc->n_shared > 0 ? desc->n_shared : 1, maxd = p.maxd;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  const size_t o_counter = take(sizeof(unsigned));
  const size_t o_logits = take(maxB * p.Er * sizeof(float));
  const size_t o_nd = take(sizeof(int));
  const size_t o_ids = take(maxd * sizeof(int));
  const size_t o_mask = take(maxd * sizeof(unsigned));
  const size_t o_wt = take(maxd * maxB * sizeof(float));
  const size_t o_tid = take(maxB * k * sizeof(int));
  const size_t o_tw = take(maxB * k * sizeof(float));
  const size_t o_c = take(maxB * S1 * sizeof(float));
  const size_t o_xhat = take(desc->prenorm_gamma ? maxB * H * 2 : 16);
  const size_t o_hr = take(maxd * maxB * I * 2);
  const size_t o_hs = take(S1 * maxB * I * 2);
  L->ws_bytes = off;
  if (hipMalloc(&L->ws, L->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete L;
    return MOE_ERR_DEVICE;
  }
  if (hipMemset(L->ws, 0, L->ws_bytes) != hipSuccess) {
    (void)hipFree(L->ws);
    delete L;
    return MOE_ERR_DEVICE;
  }
  char* w = static_cast<char*>(L->ws);
  L->counter = reinterpret_cast<unsigned*>(w + o_counter);
  L->logits = reinterpret_cast<float*>(w + o_logits);
  L->rt_nd = reinterpret_cast<int*>(w + o_nd);
  L->rt_ids = reinterpret_cast<int*>(w + o_ids);
  L->rt_mask = reinterpret_cast<unsigned*>(w + o_mask);
  L->rt_wt = reinterpret_cast<float*>(w + o_wt);
  L->topk_ids = reinterpret_cast<int*>(w + o_tid);
  L->topk_w = reinterpret_cast<float*>(w + o_tw);
  L->shared_c = reinterpret_cast<float*>(w + o_c);
  L->xhat = reinterpret_cast<uint16_t*>(w + o_xhat);
  L->h_routed = reinterpret_cast<uint16_t*>(w + o_hr);
  L->h_shared = reinterpret_cast<uint16_t*>(w + o_hs);
  *out = L;
  return MOE_OK;
}

int moe_layer_destroy(moe_layer_t L) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  int st = MOE_OK;
  if (L->ws != nullptr && hipFree(L->ws) != hipSuccess) st = MOE_ERR_DEVICE;
  delete L;
  return st;
}

}  // extern "C"

namespace {

moe::LayerArgs make_args(const moe_layer* L, const void* x, const void* router_w, const void* expert_packed,
                         const void* scales, const void* shared_w, void* out, int batch) {
  moe::LayerArgs a;
  memset(&a, 0, sizeof(a));
  const moe_layer_desc& d = L->d;
  a.x = static_cast<const uint16_t*>(x);
  a.router_w = static_cast<const uint16_t*>(router_w);
  a.bias = d.router_bias;
  a.gamma = static_cast<const uint16_t*>(d.prenorm_gamma);
  a.r_codes = static_cast<const uint8_t*>(expert_packed);
  a.r_scales = static_cast<const uint8_t*>(scales);
  a.r_tscale = (d.routed_wtype == MOE_W_NVFP4 && scales)
                   ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(scales) + L->lr.tensor_scale_offset)
                   : nullptr;
  a.s_codes = static_cast<const uint8_t*>(shared_w);
  a.s_scales = shared_w ? static_cast<const uint8_t*>(shared_w) + L->ls.shared_scale_offset : nullptr;
  a.s_tscale = (d.shared_wtype == MOE_W_NVFP4 && shared_w)
                   ? reinterpret_cast<const float*>(a.s_scales + L->ls.tensor_scale_offset)
                   : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.counter = L->counter;
  a.logits = L->logits;
  a.rt_nd = L->rt_nd;
  a.rt_ids = L->rt_ids;
  a.rt_mask = L->rt_mask;
  a.rt_wt = L->rt_wt;
  a.topk_ids = L->topk_ids;
  a.topk_w = L->topk_w;
  a.shared_c = L->shared_c;
  a.xhat = L->xhat;
  a.h_routed = L->h_routed;
  a.h_shared = L->h_shared;
  a.B = batch;
  a.maxB = d.max_batch;
  a.H = d.hidden;
  a.I = d.inter;
  a.E = d.n_routed;
  a.k = d.top_k;
  a.S = d.n_shared;
  a.Er = L->p.Er;
  a.maxd = L->p.maxd;
  a.route = d.route;
  a.prenorm = d.prenorm_gamma != nullptr;
  a.residual = d.add_residual != 0;
  a.eps = d.rms_eps;
  a.g13 = L->p.g13;
  a.g2 = L->p.g2;
  a.r_code_stride = L->lr.code_stride;
  a.r_w13_code = L->lr.w13_code_bytes;
  a.r_scale_stride = L->lr.scale_stride;
  a.r_w13_scale = L->lr.w13_scale_bytes;
  a.s_code_stride = L->ls.code_stride;
  a.s_w13_code = L->ls.w13_code_bytes;
  a.s_scale_stride = L->ls.scale_stride;
  a.s_w13_scale = L->ls.w13_scale_bytes;
  a.n_router_blocks = L->p.n_router_blocks;
  a.wpe13 = L->p.wpe13;
  a.s3 = L->p.s3;
  return a;
}

}  // namespace

extern "C" {

int moe_decode_layer(moe_layer_t L, const void* x, const void* router_w, const void* expert_packed,
                     const void* scales, const void* shared_w, void* out, int batch, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = L->d;
  if (batch < 1 || batch > d.max_batch) return MOE_ERR_BATCH;
  if (!x || !router_w || !expert_packed || !out) return MOE_ERR_INVALID_ARG;
  if (d.routed_wtype == MOE_W_NVFP4 && !scales) return MOE_ERR_INVALID_ARG;
  if (d.n_shared > 0 && !shared_w) return MOE_ERR_INVALID_ARG;
  if (x == out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(expert_packed) || !aligned16(out) ||
      (scales && !aligned16(scales)) || (shared_w && !aligned16(shared_w)))
    return MOE_ERR_ALIGNMENT;
  const moe::LayerArgs a = make_args(L, x, router_w, expert_packed, scales, shared_w, out, batch);
  const int tb = batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8;
  void* const* ev = nullptr;
  if (!L->prof.empty()) {
    ev = L->prof.data() + 4 * (L->prof_call % (L->prof.size() / 4));
    ++L->prof_call;
  }
  if (moe::launch_layer(a, tb, d.routed_wtype, d.shared_wtype, stream, ev) != 0) return MOE_ERR_LAUNCH;
  L->last_batch = batch;
  L->last_x = x;
  return MOE_OK;
}

int moe_layer_routing(moe_layer_t L, int32_t* ids, float* w, float* c, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (L->last_batch == 0) return MOE_ERR_STATE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t nk = (size_t)L->last_batch * L->d.top_k, ns = (size_t)L->last_batch * L->d.n_shared;
  if (ids && hipMemcpyAsync(ids, L->topk_ids, nk * sizeof(int), hipMemcpyDeviceToDevice, st) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (w && hipMemcpyAsync(w, L->topk_w, nk * sizeof(float), hipMemcpyDeviceToDevice, st) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (c && ns && hipMemcpyAsync(c, L->shared_c, ns * sizeof(float), hipMemcpyDeviceToDevice, st) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

int moe_layer_set_profiling(moe_layer_t L, void* const* events, int n_events) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (events == nullptr || n_events == 0) {
    L->prof.clear();
    return MOE_OK;
  }
  if (n_events < 4 || n_events % 4) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  L->prof.assign(events, events + n_events);
  L->prof_call = 0;
  return MOE_OK;
}

int moe_layer_debug_h(moe_layer_t L, void* h_routed, void* h_shared, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (L->last_batch == 0) return MOE_ERR_STATE;
  const moe::LayerArgs a = make_args(L, L->last_x, nullptr, nullptr, nullptr, nullptr, nullptr, L->last_batch);
  if (moe::launch_debug_h(a, static_cast<uint16_t*>(h_routed), static_cast<uint16_t*>(h_shared), stream) != 0)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

}  // extern "C"
