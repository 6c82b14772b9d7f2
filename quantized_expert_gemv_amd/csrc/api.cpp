// Host side of the MoE decode C ABI: descriptor validation and the launch
// plan, expert layouts, the lossless NVFP4 / bf16 packers, the layer handle
// and its workspace, and the single launch of one layer call.
// Declarations: include/moe_decode.h.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "moe_internal.h"

using moe::MatGeom;

namespace {

constexpr size_t kAlign = 256;
constexpr unsigned long long kWaitTicks = 20000000ull;   // 0.2 s of the 100 MHz clock
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int tb_of(int batch) { return batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8; }
inline int tb_index(int tb) { return tb == 1 ? 0 : tb == 2 ? 1 : tb == 4 ? 2 : 3; }

struct Plan {
  MatGeom g13, g2;
  int Er, maxd, tbmax;
  moe::FastDiv dv_gs2;
  int spg_max;                 // most down steps a workgroup owns (given G)
  int G;                       // workgroups (0 until the device is known)
  int b1 = 0;                  // batch-1 calls run the role-split kernel (launch_b1)
  int b8 = 0;                  // batch 2-8 calls run the small-batch kernel (launch_b8)
  int lds_act[4], lds_acc[4];  // per token bucket 1, 2, 4, 8
};

// Shape checks that need no device.  Fills the geometry part of the plan.
int plan_shapes(const moe_layer_desc* d, Plan* p) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  const int H = d->hidden, I = d->inter, E = d->n_routed, k = d->top_k, S = d->n_shared;
  if (H <= 0 || I <= 0 || E <= 0 || k <= 0 || S < 0 || d->max_batch <= 0) return MOE_ERR_INVALID_ARG;
  if (d->routed_wtype != MOE_W_NVFP4 && d->routed_wtype != MOE_W_BF16 && d->routed_wtype != MOE_W_2BIT)
    return MOE_ERR_INVALID_ARG;
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
  if (I % (2 * p->g13.rpw)) return MOE_ERR_UNSUPPORTED;                 // whole gate step pairs
  if (p->g13.ns > 1 && (p->g13.rpw != 1 || moe::kFusedWaves % p->g13.ns)) return MOE_ERR_UNSUPPORTED;
  p->tbmax = tb_of(d->max_batch);
  const int qx = moe::fused_qx(H);                                      // router units per thread
  if (qx == 0 || (p->tbmax >= 8 && qx != 1)) return MOE_ERR_UNSUPPORTED;
  p->Er = Er;
  p->maxd = (d->max_batch * k < E) ? d->max_batch * k : E;
  p->G = 0;
  // 2-bit routed experts run on the dedicated kernels of the Flint shape only
  // (batch 1 and batch 2-8)
  if (d->routed_wtype == MOE_W_2BIT)
    return (H == moe::FlintShape::H && I == moe::FlintShape::I && E == moe::FlintShape::E && k == moe::FlintShape::k &&
            S == moe::FlintShape::S && d->shared_wtype == MOE_W_NVFP4 && d->route == MOE_ROUTE_SIGMOID_TOPK)
               ? MOE_OK
               : MOE_ERR_UNSUPPORTED;
  // a kernel variant must exist for every batch bucket the layer may run
  const int shape = moe::fixed_shape_of(H, I, E, k, S, Er, d->routed_wtype, d->shared_wtype);
  for (int tb = 1; tb <= p->tbmax; tb *= 2)
    if (!moe::fused_variant_exists(shape, tb, qx, d->routed_wtype, d->shared_wtype)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Grid and shared-memory plan for G workgroups.
void plan_grid(const moe_layer_desc* d, Plan* p, int G) {
  p->G = G;
  const int nsteps2 = p->g2.nsteps;
  p->spg_max = (nsteps2 + G - 1) / G;
  const int gs2 = d->inter / p->g13.rpw / 2;
  const int ns = p->g13.ns;
  for (int ti = 0; ti < 4; ++ti) {
    const int tb = 1 << ti;
    size_t part = 0;
    if (ns > 1) {
      const int n1 = d->n_shared * gs2, n2 = p->maxd * gs2;
      const int per = ((n1 > n2 ? n1 : n2) + G - 1) / G;
      part = (size_t)per * tb * 4 * ns * sizeof(float);
    }
    const size_t xbytes = (size_t)tb * d->hidden * 2 + part;
    const int nb = d->max_batch < tb ? d->max_batch : tb;
    const size_t hbytes = (size_t)nb * (d->top_k + d->n_shared) * d->inter * 2;
    p->lds_act[ti] = (int)align_up(xbytes > hbytes ? xbytes : hbytes, 16);
    p->lds_acc[ti] = moe::kFusedWaves * tb * p->spg_max * p->g2.rpw * (int)sizeof(float);   // nsub <= waves
  }
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
  } else if (wtype == MOE_W_2BIT) {
    o->w13_code_bytes = IH / 2;       // 2I * H / 4
    o->w2_code_bytes = IH / 4;        // H * I / 4
    o->w13_scale_bytes = IH / 8;
    o->w2_scale_bytes = IH / 16;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  o->code_stride = o->w13_code_bytes + o->w2_code_bytes;
  o->code_region_bytes = o->code_stride * (size_t)n;
  o->scale_stride = o->w13_scale_bytes + o->w2_scale_bytes;
  if (wtype == MOE_W_NVFP4 || wtype == MOE_W_2BIT) {
    o->tensor_scale_offset = align_up(o->scale_stride * (size_t)n, kAlign);
    o->scale_region_bytes = o->tensor_scale_offset + (size_t)n * 2 * sizeof(float);
  }
  o->shared_scale_offset = align_up(o->code_region_bytes, kAlign);
  o->shared_total_bytes = o->shared_scale_offset + o->scale_region_bytes;
  return MOE_OK;
}


// Geometry of a dense GEMV matrix: rows padded up to whole scale-word step
// pairs, one wave step per rpw rows (cols <= 2048: no slices).
int dense_geom(int rows, int cols, MatGeom* g) {
  if (rows <= 0 || rows > (1 << 20) || cols < 32 || cols > 2048 || cols % 32) return -1;
  const int rpw = moe::geom_of(1, cols).rpw;
  const int prows = (rows + 2 * rpw - 1) / (2 * rpw) * (2 * rpw);
  if (moe::make_geom(prows, cols, g) || g->ns != 1) return -1;
  return 0;
}

// Matrices the packers accept: a geometry must exist for them.
int pack_geom(int rows, int cols, MatGeom* g) {
  if (rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (moe::make_geom(rows, cols, g)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// One matrix, canonical <-> kernel layout.  PACK = true moves canonical bytes
// (codes / scales / bf16 words) into the packed buffers, false the reverse.
template <bool PACK>
void move_nvfp4(const MatGeom& g, uint8_t* codes, uint8_t* scales, uint8_t* cp, uint8_t* sp) {
  const size_t crow = (size_t)g.cols / 2, srow = (size_t)g.cols / 16;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int ri = 0; ri < g.rpw; ++ri)
        for (int j = 0; j < g.cw; ++j) {
          const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
          uint8_t* pc = cp + moe::code_unit(g, s, t, ri, j) * 16;
          uint8_t* ps = sp + moe::scale_word(g, s, t, ri, j) + 2 * (t & 1);
          if (PACK) {
            memcpy(pc, codes + row * crow + cc * 16, 16);
            memcpy(ps, scales + row * srow + cc * 2, 2);
          } else {
            memcpy(codes + row * crow + cc * 16, pc, 16);
            memcpy(scales + row * srow + cc * 2, ps, 2);
          }
        }
}
// The 2-bit planes: the NVFP4 geometry with 8-byte code chunks (32 codes of
// 2 bits, in canonical order) and the same scale words.
template <bool PACK>
void move_2bit(const MatGeom& g, uint8_t* codes, uint8_t* scales, uint8_t* cp, uint8_t* sp) {
  const size_t crow = (size_t)g.cols / 4, srow = (size_t)g.cols / 16;
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int ri = 0; ri < g.rpw; ++ri)
        for (int j = 0; j < g.cw; ++j) {
          const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
          uint8_t* pc = cp + moe::code_unit(g, s, t, ri, j) * 8;
          uint8_t* ps = sp + moe::scale_word(g, s, t, ri, j) + 2 * (t & 1);
          if (PACK) {
            memcpy(pc, codes + row * crow + cc * 8, 8);
            memcpy(ps, scales + row * srow + cc * 2, 2);
          } else {
            memcpy(codes + row * crow + cc * 8, pc, 8);
            memcpy(scales + row * srow + cc * 2, ps, 2);
          }
        }
}
template <bool PACK>
void move_bf16(const MatGeom& g, uint16_t* w, uint16_t* wp) {
  for (int s = 0; s < g.ns; ++s)
    for (int t = 0; t < g.nsteps; ++t)
      for (int sub = 0; sub < 4; ++sub)
        for (int ri = 0; ri < g.rpw; ++ri)
          for (int j = 0; j < g.cw; ++j) {
            const size_t row = (size_t)t * g.rpw + ri, cc = (size_t)s * g.cw + j;
            uint16_t* p = wp + moe::bf16_unit(g, s, t, sub, ri, j) * 8;
            uint16_t* c = w + row * g.cols + cc * 32 + sub * 8;
            if (PACK) memcpy(p, c, 16);
            else memcpy(c, p, 16);
          }
}

// The weight type and expert count of one expert set of a layer.
struct SetInfo {
  int wtype, n;
};
int set_info(const moe_layer_desc* d, int set, SetInfo* si) {
  if (d == nullptr || (set != MOE_SET_ROUTED && set != MOE_SET_SHARED)) return MOE_ERR_INVALID_ARG;
  Plan p;
  if (int st = plan_shapes(d, &p)) return st;
  si->wtype = set == MOE_SET_ROUTED ? d->routed_wtype : d->shared_wtype;
  si->n = set == MOE_SET_ROUTED ? d->n_routed : d->n_shared;
  return MOE_OK;
}

// Experts [first, first + count) of a set of n, canonical <-> the set's
// regions (placement 0: code region + scale region; 1: one buffer, the scale
// region at shared_scale_offset).
template <bool PACK>
int move_experts(int wtype, int H, int I, int n, int first, int count, uint8_t* w13, uint8_t* w13s, uint8_t* w2,
                 uint8_t* w2s, float* ts, int placement, uint8_t* code_region, uint8_t* scale_region) {
  moe_expert_layout lay;
  if (int st = layout(wtype, H, I, n, &lay)) return st;
  if (first < 0 || count < 0 || first > n || count > n - first) return MOE_ERR_INVALID_ARG;
  if (placement != 0 && placement != 1) return MOE_ERR_INVALID_ARG;
  if (code_region == nullptr || w13 == nullptr || w2 == nullptr) return MOE_ERR_INVALID_ARG;
  MatGeom g13, g2;
  if (int st = pack_geom(2 * I, H, &g13)) return st;
  if (int st = pack_geom(H, I, &g2)) return st;
  uint8_t* sreg = placement == 1 ? code_region + lay.shared_scale_offset : scale_region;
  const bool scaled = wtype == MOE_W_NVFP4 || wtype == MOE_W_2BIT;
  if (scaled && (w13s == nullptr || w2s == nullptr || sreg == nullptr)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    const size_t e = (size_t)first + i;
    uint8_t* cb = code_region + e * lay.code_stride;
    if (scaled) {
      const size_t per = wtype == MOE_W_NVFP4 ? 2 : 4;   // codes per byte
      const size_t c13 = (size_t)2 * I * H / per, s13 = (size_t)2 * I * H / 16;
      const size_t c2 = (size_t)H * I / per, s2 = (size_t)H * I / 16;
      uint8_t* sb = sreg + e * lay.scale_stride;
      if (wtype == MOE_W_NVFP4) {
        move_nvfp4<PACK>(g13, w13 + i * c13, w13s + i * s13, cb, sb);
        move_nvfp4<PACK>(g2, w2 + i * c2, w2s + i * s2, cb + lay.w13_code_bytes, sb + lay.w13_scale_bytes);
      } else {
        move_2bit<PACK>(g13, w13 + i * c13, w13s + i * s13, cb, sb);
        move_2bit<PACK>(g2, w2 + i * c2, w2s + i * s2, cb + lay.w13_code_bytes, sb + lay.w13_scale_bytes);
      }
      float* tp = reinterpret_cast<float*>(sreg + lay.tensor_scale_offset) + 2 * e;
      if (PACK) {
        tp[0] = ts ? ts[2 * i] : 1.0f;
        tp[1] = ts ? ts[2 * i + 1] : 1.0f;
      } else if (ts) {
        ts[2 * i] = tp[0];
        ts[2 * i + 1] = tp[1];
      }
    } else {
      const size_t n13 = (size_t)2 * I * H, n2 = (size_t)H * I;
      move_bf16<PACK>(g13, reinterpret_cast<uint16_t*>(w13) + i * n13, reinterpret_cast<uint16_t*>(cb));
      move_bf16<PACK>(g2, reinterpret_cast<uint16_t*>(w2) + i * n2,
                      reinterpret_cast<uint16_t*>(cb + lay.w13_code_bytes));
    }
  }
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
  unsigned* epoch;
  unsigned* err;
  unsigned long long* xlog;
  unsigned long long* xh;
  unsigned long long* xx;
  int* topk_ids;
  float* topk_w;
  float* shared_c;
  int last_batch;
  std::vector<void*> prof;       // profiling events (caller-owned)
  unsigned long long prof_call;
  int force_general = 0;          // moe_layer_set_path(MOE_PATH_GENERAL)
};

namespace {

// Byte offsets of the workspace areas of a layer (one allocation, or the
// library's static scratch array for moe_decode_layer_static).
struct WsLayout {
  size_t epoch, err, xlog, xh, xx, tid, tw, c, total;
};

WsLayout ws_layout(const moe_layer_desc* d, const Plan& p) {
  const size_t maxB = d->max_batch, k = d->top_k;
  const size_t S1 = d->n_shared > 0 ? d->n_shared : 1;
  const size_t npairs = maxB * (k + d->n_shared);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  WsLayout w;
  w.epoch = take(sizeof(unsigned));
  w.err = take(sizeof(unsigned));
  w.xlog = take((size_t)p.Er * moe::kLogitLine * 8);
  w.xh = take(npairs * (d->inter / 2) * 8);
  w.xx = take((size_t)(d->hidden / 2) * 8);   // a chain's layer outputs, one token
  w.tid = take(maxB * k * sizeof(int));
  w.tw = take(maxB * k * sizeof(float));
  w.c = take(maxB * S1 * sizeof(float));
  w.total = off;
  return w;
}

void bind_ws(moe_layer* L, void* base, const WsLayout& wl) {
  char* w = static_cast<char*>(base);
  L->ws = base;
  L->epoch = reinterpret_cast<unsigned*>(w + wl.epoch);
  L->err = reinterpret_cast<unsigned*>(w + wl.err);
  L->xlog = reinterpret_cast<unsigned long long*>(w + wl.xlog);
  L->xh = reinterpret_cast<unsigned long long*>(w + wl.xh);
  L->xx = reinterpret_cast<unsigned long long*>(w + wl.xx);
  L->topk_ids = reinterpret_cast<int*>(w + wl.tid);
  L->topk_w = reinterpret_cast<float*>(w + wl.tw);
  L->shared_c = reinterpret_cast<float*>(w + wl.c);
}

// The gate/up item divisor, checked once per divisor value over every item
// index a launch can form (n < 2^22; the method is exact for n < 2^31).
// Checked divisors are remembered in a fixed table (no allocation).
bool fastdiv_checked(uint32_t d, moe::FastDiv* out) {
  static std::mutex mu;
  static uint32_t done[64];
  static int ndone = 0;
  const moe::FastDiv dv = moe::make_fastdiv(d);
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < ndone; ++i)
      if (done[i] == d) {
        *out = dv;
        return true;
      }
  }
  for (uint32_t n = 0; n < (1u << 22); ++n)
    if (moe::fastdiv(n, dv) != n / d) return false;
  std::lock_guard<std::mutex> g(mu);
  if (ndone < 64) done[ndone++] = d;
  *out = dv;
  return true;
}

// Grid of the launch on `device`: a power of two of workgroups (work splits
// by shifts), at most one per router row (each publishes a logit, which is
// how workgroup 0 knows every workgroup has read the call counter), at most
// two rows each, and never more than can be resident together.
int plan_device(const moe_layer_desc* desc, Plan* pp, int device) {
  Plan& p = *pp;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  const int rwt = desc->routed_wtype, swt = desc->shared_wtype;
  if (rwt == MOE_W_2BIT) {
    // only the dedicated kernels take 2-bit routed experts: batch 1 and, for
    // a layer that may run more tokens, batch 2-8
    int occ1 = 0, occ8 = 0;
    p.b1 = cus >= moe::kB1Workgroups && moe::b1_occupancy(&occ1) == 0 && occ1 >= 1;
    p.b8 = cus >= moe::kB1Workgroups && moe::b8_occupancy(&occ8) == 0 && occ8 >= 1;
    (void)hipGetLastError();
    if (!p.b1 || (desc->max_batch > 1 && !p.b8)) return MOE_ERR_UNSUPPORTED;
    plan_grid(desc, &p, moe::kB1Workgroups);
    return MOE_OK;
  }
  int cap = p.Er < cus ? p.Er : cus;
  int G = 1;
  while (2 * G <= cap) G *= 2;
  plan_grid(desc, &p, G);
  const int shape = moe::fixed_shape_of(desc->hidden, desc->inter, desc->n_routed, desc->top_k, desc->n_shared, p.Er,
                                        rwt, swt);
  for (int tb = 1; tb <= p.tbmax; tb *= 2) {
    int occ = 0;
    const int ti = tb_index(tb);
    if (moe::fused_occupancy(shape, tb, moe::fused_qx(desc->hidden), rwt, swt, p.lds_act[ti] + p.lds_acc[ti], &occ) != 0 ||
        occ < 1) {
      (void)hipGetLastError();
      return MOE_ERR_UNSUPPORTED;
    }
    while (G > occ * cus) G /= 2;
  }
  if (2 * G < p.Er) return MOE_ERR_UNSUPPORTED;
  plan_grid(desc, &p, G);
  const int gs2 = desc->inter / p.g13.rpw / 2;
  if (moe::kFusedWaves / p.g13.ns > gs2) return MOE_ERR_UNSUPPORTED;
  if (!fastdiv_checked((uint32_t)gs2, &p.dv_gs2)) return MOE_ERR_UNSUPPORTED;
  // Batch 1 of the Flint shape with NVFP4 experts and the sigmoid router runs
  // the role-split kernel when all of its workgroups fit on the device at once.
  p.b1 = p.b8 = 0;
  int occ1 = 0, occ8 = 0;
  if (shape == 1 && rwt == MOE_W_NVFP4 && desc->route == MOE_ROUTE_SIGMOID_TOPK && cus >= moe::kB1Workgroups) {
    if (moe::b1_occupancy(&occ1) == 0 && occ1 >= 1) p.b1 = 1;
    if (moe::b8_occupancy(&occ8) == 0 && occ8 >= 1) p.b8 = 1;
  }
  (void)hipGetLastError();
  return MOE_OK;
}

}  // namespace

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
  return plan_shapes(desc, &p);
}

int moe_expert_layout_query(const moe_layer_desc* desc, int set, moe_expert_layout* out) {
  SetInfo si;
  if (int st = set_info(desc, set, &si)) return st;
  return layout(si.wtype, desc->hidden, desc->inter, si.n, out);
}

int moe_pack_nvfp4(int rows, int cols, const uint8_t* codes, const uint8_t* scales, uint8_t* codes_out,
                   uint8_t* scales_out) {
  if (!codes || !scales || !codes_out || !scales_out) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  move_nvfp4<true>(g, const_cast<uint8_t*>(codes), const_cast<uint8_t*>(scales), codes_out, scales_out);
  return MOE_OK;
}

int moe_unpack_nvfp4(int rows, int cols, const uint8_t* codes_packed, const uint8_t* scales_packed,
                     uint8_t* codes, uint8_t* scales) {
  if (!codes || !scales || !codes_packed || !scales_packed) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  move_nvfp4<false>(g, codes, scales, const_cast<uint8_t*>(codes_packed), const_cast<uint8_t*>(scales_packed));
  return MOE_OK;
}

int moe_dense_layout_query(int rows, int cols, moe_dense_layout* o) {
  MatGeom g;
  if (o == nullptr || dense_geom(rows, cols, &g)) return MOE_ERR_INVALID_ARG;
  memset(o, 0, sizeof(*o));
  o->rows = rows;
  o->cols = cols;
  o->packed_rows = g.rows;
  o->code_bytes = (size_t)g.rows * cols / 2;
  o->scale_bytes = (size_t)g.rows * cols / 16;
  o->tensor_scale_offset = align_up(o->scale_bytes, kAlign);
  o->scale_region_bytes = o->tensor_scale_offset + kAlign;
  return MOE_OK;
}

int moe_pack_dense(int rows, int cols, const void* codes, const void* scales, float tensor_scale,
                   void* code_region, void* scale_region) {
  MatGeom g;
  if (!codes || !scales || !code_region || !scale_region || dense_geom(rows, cols, &g)) return MOE_ERR_INVALID_ARG;
  // the rows past `rows` are zero codes with zero scales
  const size_t crow = (size_t)cols / 2, srow = (size_t)cols / 16;
  std::vector<uint8_t> c((size_t)g.rows * crow, 0), s((size_t)g.rows * srow, 0);
  memcpy(c.data(), codes, (size_t)rows * crow);
  memcpy(s.data(), scales, (size_t)rows * srow);
  uint8_t* sr = static_cast<uint8_t*>(scale_region);
  move_nvfp4<true>(g, c.data(), s.data(), static_cast<uint8_t*>(code_region), sr);
  moe_dense_layout lay;
  (void)moe_dense_layout_query(rows, cols, &lay);
  memset(sr + lay.scale_bytes, 0, lay.scale_region_bytes - lay.scale_bytes);
  memcpy(sr + lay.tensor_scale_offset, &tensor_scale, sizeof(float));
  return MOE_OK;
}

int moe_unpack_dense(int rows, int cols, const void* code_region, const void* scale_region, void* codes,
                     void* scales, float* tensor_scale) {
  MatGeom g;
  if (!codes || !scales || !code_region || !scale_region || dense_geom(rows, cols, &g)) return MOE_ERR_INVALID_ARG;
  const size_t crow = (size_t)cols / 2, srow = (size_t)cols / 16;
  std::vector<uint8_t> c((size_t)g.rows * crow), s((size_t)g.rows * srow);
  move_nvfp4<false>(g, c.data(), s.data(), const_cast<uint8_t*>(static_cast<const uint8_t*>(code_region)),
                    const_cast<uint8_t*>(static_cast<const uint8_t*>(scale_region)));
  memcpy(codes, c.data(), (size_t)rows * crow);
  memcpy(scales, s.data(), (size_t)rows * srow);
  if (tensor_scale) {
    moe_dense_layout lay;
    (void)moe_dense_layout_query(rows, cols, &lay);
    memcpy(tensor_scale, static_cast<const uint8_t*>(scale_region) + lay.tensor_scale_offset, sizeof(float));
  }
  return MOE_OK;
}

int moe_dense_gemv(int rows, int cols, const void* code_region, const void* scale_region, const void* x, void* y,
                   int batch, void* stream) {
  MatGeom g;
  if (!code_region || !scale_region || !x || !y || dense_geom(rows, cols, &g)) return MOE_ERR_INVALID_ARG;
  if (batch < 1 || batch > MOE_MAX_BATCH) return MOE_ERR_BATCH;
  if (!aligned16(code_region) || !aligned16(scale_region) || !aligned16(x) || !aligned16(y)) return MOE_ERR_ALIGNMENT;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* yb = static_cast<const uint8_t*>(y);
  const size_t xn = (size_t)batch * cols * 2, yn = (size_t)batch * rows * 2;
  if (xb < yb + yn && yb < xb + xn) return MOE_ERR_INVALID_ARG;
  moe_dense_layout lay;
  (void)moe_dense_layout_query(rows, cols, &lay);
  moe::DenseArgs a;
  a.codes = static_cast<const uint8_t*>(code_region);
  a.scales = static_cast<const uint8_t*>(scale_region);
  a.tscale = reinterpret_cast<const float*>(a.scales + lay.tensor_scale_offset);
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.rows = rows;
  a.B = batch;
  a.g = g;
  return moe::launch_dense(a, stream) == 0 ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_pack_bf16(int rows, int cols, const uint16_t* w, uint16_t* w_out) {
  if (!w || !w_out) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  move_bf16<true>(g, const_cast<uint16_t*>(w), w_out);
  return MOE_OK;
}

int moe_unpack_bf16(int rows, int cols, const uint16_t* w_packed, uint16_t* w) {
  if (!w || !w_packed) return MOE_ERR_INVALID_ARG;
  MatGeom g;
  if (int st = pack_geom(rows, cols, &g)) return st;
  move_bf16<false>(g, w, const_cast<uint16_t*>(w_packed));
  return MOE_OK;
}

int moe_requant_2bit(int rows, int cols, const uint8_t* codes, const uint8_t* scales, uint8_t* codes2,
                     uint8_t* scales2) {
#pragma clang fp contract(off)
  if (!codes || !scales || !codes2 || !scales2 || rows <= 0 || cols <= 0 || cols % 16) return MOE_ERR_INVALID_ARG;
  static const double kE2m1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  static const double kLevel[4] = {-4.0, -1.0, 1.0, 4.0};
  const auto e4m3 = [](int b) {
    const int e = (b >> 3) & 15, m = b & 7;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return (b & 0x80) ? -mag : mag;
  };
  double cand[0x7F];
  for (int sb = 0; sb < 0x7F; ++sb) cand[sb] = e4m3(sb);
  const size_t nb = (size_t)cols / 16;
  for (size_t r = 0; r < (size_t)rows; ++r) {
    for (size_t b = 0; b < nb; ++b) {
      double v[16];
      const double bs = e4m3(scales[r * nb + b]);
      for (int i = 0; i < 16; ++i) {
        const size_t c = b * 16 + i;
        const int code = (codes[r * (cols / 2) + c / 2] >> (4 * (c & 1))) & 15;
        const double m = (code & 8) ? -kE2m1[code & 7] : kE2m1[code & 7];
        v[i] = m * bs;
      }
      double best = INFINITY;
      int best_sb = 0;
      uint8_t best_q[16] = {0};
      for (int sb = 0; sb < 0x7F; ++sb) {
        const double sc = cand[sb];
        uint8_t q[16];
        double err = 0.0;
        for (int i = 0; i < 16; ++i) {
          const bool neg = std::signbit(v[i]);
          const bool big = sc > 0.0 && 2.0 * fabs(v[i]) > 5.0 * sc;
          q[i] = neg ? (big ? 0 : 1) : (big ? 3 : 2);
          const double rec = kLevel[q[i]] * sc;
          const double d = v[i] - rec;
          const double dd = d * d;
          err = err + dd;
        }
        if (err < best) {
          best = err;
          best_sb = sb;
          memcpy(best_q, q, 16);
        }
      }
      scales2[r * nb + b] = (uint8_t)best_sb;
      for (int j = 0; j < 4; ++j)
        codes2[r * (cols / 4) + b * 4 + j] =
            (uint8_t)(best_q[4 * j] | (best_q[4 * j + 1] << 2) | (best_q[4 * j + 2] << 4) | (best_q[4 * j + 3] << 6));
    }
  }
  return MOE_OK;
}

int moe_pack_experts(const moe_layer_desc* desc, int set, int first, int count, const void* w13,
                     const void* w13_scales, const void* w2, const void* w2_scales, const float* tensor_scales,
                     void* region, void* scale_region) {
  SetInfo si;
  if (int st = set_info(desc, set, &si)) return st;
  return move_experts<true>(si.wtype, desc->hidden, desc->inter, si.n, first, count,
                            static_cast<uint8_t*>(const_cast<void*>(w13)),
                            static_cast<uint8_t*>(const_cast<void*>(w13_scales)),
                            static_cast<uint8_t*>(const_cast<void*>(w2)),
                            static_cast<uint8_t*>(const_cast<void*>(w2_scales)), const_cast<float*>(tensor_scales),
                            set == MOE_SET_SHARED ? 1 : 0, static_cast<uint8_t*>(region),
                            static_cast<uint8_t*>(scale_region));
}

int moe_unpack_experts(const moe_layer_desc* desc, int set, int first, int count, const void* region,
                       const void* scale_region, void* w13, void* w13_scales, void* w2, void* w2_scales,
                       float* tensor_scales) {
  SetInfo si;
  if (int st = set_info(desc, set, &si)) return st;
  return move_experts<false>(si.wtype, desc->hidden, desc->inter, si.n, first, count,
                             static_cast<uint8_t*>(w13), static_cast<uint8_t*>(w13_scales), static_cast<uint8_t*>(w2),
                             static_cast<uint8_t*>(w2_scales), tensor_scales, set == MOE_SET_SHARED ? 1 : 0,
                             static_cast<uint8_t*>(const_cast<void*>(region)),
                             static_cast<uint8_t*>(const_cast<void*>(scale_region)));
}

int moe_layer_create(const moe_layer_desc* desc, moe_layer_t* out) {
  if (out == nullptr) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  Plan p;
  if (int st = plan_shapes(desc, &p)) return st;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  if (int st = plan_device(desc, &p, device)) return st;
  moe_layer* L = new (std::nothrow) moe_layer();
  if (L == nullptr) return MOE_ERR_DEVICE;
  L->d = *desc;
  L->p = p;
  L->device = device;
  (void)moe_expert_layout_query(desc, MOE_SET_ROUTED, &L->lr);
  (void)moe_expert_layout_query(desc, MOE_SET_SHARED, &L->ls);
  const WsLayout wl = ws_layout(desc, p);
  L->ws_bytes = wl.total;
  if (hipMalloc(&L->ws, L->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete L;
    return MOE_ERR_DEVICE;
  }
  // zero words carry tag 0, which no call uses (tags start at 1)
  if (hipMemset(L->ws, 0, L->ws_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(L->ws);
    delete L;
    return MOE_ERR_DEVICE;
  }
  bind_ws(L, L->ws, wl);
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

moe::FusedArgs make_args(const moe_layer* L, const void* x, const void* router_w, const void* expert_packed,
                         const void* scales, const void* shared_w, void* out, int batch) {
  moe::FusedArgs a;
  memset(&a, 0, sizeof(a));
  const moe_layer_desc& d = L->d;
  a.x = static_cast<const uint16_t*>(x);
  a.router_w = static_cast<const uint16_t*>(router_w);
  a.bias = d.router_bias;
  a.gamma = static_cast<const uint16_t*>(d.prenorm_gamma);
  a.r_codes = static_cast<const uint8_t*>(expert_packed);
  a.r_scales = static_cast<const uint8_t*>(scales);
  a.r_tscale = ((d.routed_wtype == MOE_W_NVFP4 || d.routed_wtype == MOE_W_2BIT) && scales)
                   ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(scales) + L->lr.tensor_scale_offset)
                   : nullptr;
  a.s_codes = static_cast<const uint8_t*>(shared_w);
  a.s_scales = shared_w ? static_cast<const uint8_t*>(shared_w) + L->ls.shared_scale_offset : nullptr;
  a.s_tscale = (d.shared_wtype == MOE_W_NVFP4 && shared_w)
                   ? reinterpret_cast<const float*>(a.s_scales + L->ls.tensor_scale_offset)
                   : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.epoch = L->epoch;
  a.err = L->err;
  a.xlog = L->xlog;
  a.xh = L->xh;
  a.topk_ids = L->topk_ids;
  a.topk_w = L->topk_w;
  a.shared_c = L->shared_c;
  a.B = batch;
  a.H = d.hidden;
  a.I = d.inter;
  a.E = d.n_routed;
  a.k = d.top_k;
  a.S = d.n_shared;
  a.Er = L->p.Er;
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
  a.G = L->p.G;
  a.log2G = 0;
  while ((1 << a.log2G) < a.G) ++a.log2G;
  a.dv_gs2 = L->p.dv_gs2;
  const int ti = tb_index(tb_of(batch));
  a.lds_act = L->p.lds_act[ti];
  a.lds_acc = L->p.lds_acc[ti];
  a.spg_max = L->p.spg_max;
  a.wait_ticks = kWaitTicks;
  return a;
}

// One layer call.
int launch_layer(const moe_layer* L, const moe::FusedArgs& a, void* stream) {
  if (!L->force_general) {
    if (a.B == 1 && L->p.b1) {
      moe::B1Args b;
      b.a = a;
      b.xx = L->xx;
      b.n = 1;
      b.L[0] = moe::chain_layer_of(a);
      b.r2bit = L->d.routed_wtype == MOE_W_2BIT;
      return moe::launch_b1(b, stream);
    }
    if (a.B >= 2 && L->p.b8) return moe::launch_b8(a, a.B, L->d.routed_wtype == MOE_W_2BIT, stream);
  }
  return moe::launch_fused(a, tb_of(a.B), L->d.routed_wtype, L->d.shared_wtype, stream);
}

// Argument checks of one layer call (both entry points).
int check_call(const moe_layer_desc& d, const void* x, const void* router_w, const void* expert_packed,
               const void* scales, const void* shared_w, const void* out, int batch) {
  if (batch < 1 || batch > d.max_batch) return MOE_ERR_BATCH;
  if (!x || !router_w || !expert_packed || !out) return MOE_ERR_INVALID_ARG;
  if ((d.routed_wtype == MOE_W_NVFP4 || d.routed_wtype == MOE_W_2BIT) && !scales) return MOE_ERR_INVALID_ARG;
  if (d.n_shared > 0 && !shared_w) return MOE_ERR_INVALID_ARG;
  if (x == out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(expert_packed) || !aligned16(out) ||
      (scales && !aligned16(scales)) || (shared_w && !aligned16(shared_w)))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

// Plans of handle-less calls, per (device, layer shape), in a fixed table.
bool cached_plan(const moe_layer_desc* d, int device, Plan* p) {
  struct Key {
    int device, H, I, E, k, S, maxb, rwt, swt, route;
    bool operator==(const Key& o) const {
      return device == o.device && H == o.H && I == o.I && E == o.E && k == o.k && S == o.S && maxb == o.maxb &&
             rwt == o.rwt && swt == o.swt && route == o.route;
    }
  };
  constexpr int kSlots = 16;
  static std::mutex mu;
  static Key keys[kSlots];
  static Plan plans[kSlots];
  static int used = 0, next = 0;
  const Key key{device, d->hidden, d->inter, d->n_routed, d->top_k, d->n_shared, d->max_batch,
                d->routed_wtype, d->shared_wtype, d->route};
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
      if (keys[i] == key) {
        *p = plans[i];
        return true;
      }
  }
  if (plan_device(d, p, device) != MOE_OK) return false;
  std::lock_guard<std::mutex> g(mu);
  keys[next] = key;
  plans[next] = *p;
  next = (next + 1) % kSlots;
  if (used < kSlots) ++used;
  return true;
}

}  // namespace

extern "C" {

// ---- prefill / large batch ----

namespace {

bool prefill_supported(const moe_layer_desc& d, const Plan& p) {
  // the router GEMM takes 256 columns per pass, the expert GEMMs stage K in
  // slices of min(256, K) columns
  const auto slice_ok = [](int n) { return n % 256 == 0 || n == 64 || n == 128; };   // power-of-two slices
  return (d.routed_wtype == MOE_W_NVFP4 || d.routed_wtype == MOE_W_2BIT) &&
         (d.n_shared == 0 || d.shared_wtype == MOE_W_NVFP4) &&
         d.route == MOE_ROUTE_SIGMOID_TOPK && d.hidden <= moe::kPfMaxH && d.hidden % 256 == 0 &&
         d.inter % 64 == 0 && slice_ok(d.hidden) && slice_ok(d.inter) && d.n_routed <= moe::kPfMaxE &&
         d.n_routed % 16 == 0 && p.g13.ns == 1 && p.g2.ns == 1;
}

// Token counts the prefill takes: 1 .. MOE_PREFILL_MAX_TOKENS, and few enough
// that every element offset into the sorted intermediate rows ((top_k +
// n_shared) rows per token, `inter` wide) fits 32 bits (the GEMMs stage rows
// by 32-bit element offsets).
bool prefill_tokens_ok(const moe_layer_desc& d, int tokens) {
  return tokens >= 1 && tokens <= MOE_PREFILL_MAX_TOKENS &&
         (uint64_t)tokens * (uint64_t)(d.top_k + d.n_shared) * (uint64_t)d.inter < (1ull << 32);
}

struct PfLayout {
  size_t xhat, logits, ids, wts, counts, offs, toff, perm, inv, h, y, total;
};

PfLayout pf_layout(const moe_layer_desc& d, int T) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  const size_t Tk = (size_t)T * d.top_k, rows = Tk + (size_t)T * d.n_shared;
  const size_t ng = (size_t)d.n_routed + d.n_shared + 1;
  PfLayout w;
  w.xhat = take(d.prenorm_gamma ? (size_t)T * d.hidden * 2 : 0);
  w.logits = take((size_t)T * d.n_routed * 4);
  w.ids = take(Tk * 4);
  w.wts = take(Tk * 4);
  w.counts = take((size_t)d.n_routed * 5 * 4);   // per expert: its pairs, then each counting wave's share
  w.offs = take(ng * 4);
  w.toff = take(ng * 4);
  w.perm = take(Tk * 4);
  w.inv = take(Tk * 4);
  w.h = take(rows * d.inter * 2);
  w.y = take(rows * d.hidden * 4);
  w.total = off;
  return w;
}

}  // namespace

int moe_prefill_workspace_bytes(moe_layer_t L, int tokens, size_t* bytes) {
  if (L == nullptr || bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = 0;
  if (!prefill_supported(L->d, L->p)) return MOE_ERR_UNSUPPORTED;
  if (!prefill_tokens_ok(L->d, tokens)) return MOE_ERR_BATCH;
  *bytes = pf_layout(L->d, tokens).total;
  return MOE_OK;
}

int moe_prefill_layer(moe_layer_t L, const void* x, const void* router_w, const void* expert_packed,
                      const void* scales, const void* shared_w, void* out, int tokens, void* workspace,
                      size_t workspace_bytes, int32_t* topk_ids, float* topk_w, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = L->d;
  if (!prefill_supported(d, L->p)) return MOE_ERR_UNSUPPORTED;
  if (!prefill_tokens_ok(d, tokens)) return MOE_ERR_BATCH;
  if (!x || !router_w || !expert_packed || !scales || !out || !workspace) return MOE_ERR_INVALID_ARG;
  if (d.n_shared > 0 && !shared_w) return MOE_ERR_INVALID_ARG;
  const size_t xbytes = (size_t)tokens * d.hidden * 2;
  const char *xb = static_cast<const char*>(x), *ob = static_cast<const char*>(out);
  if (xb < ob + xbytes && ob < xb + xbytes) return MOE_ERR_INVALID_ARG;   // out overlaps x
  const PfLayout wl = pf_layout(d, tokens);
  if (workspace_bytes < wl.total) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(expert_packed) || !aligned16(scales) ||
      !aligned16(out) || !aligned16(workspace) || (shared_w && !aligned16(shared_w)) ||
      (reinterpret_cast<uintptr_t>(topk_ids) & 3u) || (reinterpret_cast<uintptr_t>(topk_w) & 3u))
    return MOE_ERR_ALIGNMENT;
  const moe::FusedArgs f = make_args(L, x, router_w, expert_packed, scales, shared_w, out, 1);
  moe::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.x = f.x;
  a.out = f.out;
  a.router_w = f.router_w;
  a.bias = f.bias;
  a.gamma = f.gamma;
  a.eps = f.eps;
  a.prenorm = f.prenorm;
  a.residual = f.residual;
  a.r_codes = f.r_codes;
  a.r_scales = f.r_scales;
  a.r_tscale = f.r_tscale;
  a.s_codes = f.s_codes;
  a.s_scales = f.s_scales;
  a.s_tscale = f.s_tscale;
  a.r_code_stride = f.r_code_stride;
  a.r_w13_code = f.r_w13_code;
  a.r_scale_stride = f.r_scale_stride;
  a.r_w13_scale = f.r_w13_scale;
  a.s_code_stride = f.s_code_stride;
  a.s_w13_code = f.s_w13_code;
  a.s_scale_stride = f.s_scale_stride;
  a.s_w13_scale = f.s_w13_scale;
  a.T = tokens;
  a.H = d.hidden;
  a.I = d.inter;
  a.E = d.n_routed;
  a.k = d.top_k;
  a.S = d.n_shared;
  a.g13 = L->p.g13;
  a.g2 = L->p.g2;
  a.r2bit = d.routed_wtype == MOE_W_2BIT;
  char* w = static_cast<char*>(workspace);
  a.xhat = reinterpret_cast<uint16_t*>(w + wl.xhat);
  a.logits = reinterpret_cast<float*>(w + wl.logits);
  a.ids = reinterpret_cast<int*>(w + wl.ids);
  a.wts = reinterpret_cast<float*>(w + wl.wts);
  a.counts = reinterpret_cast<int*>(w + wl.counts);
  a.offs = reinterpret_cast<int*>(w + wl.offs);
  a.tile_off = reinterpret_cast<int*>(w + wl.toff);
  a.perm = reinterpret_cast<int*>(w + wl.perm);
  a.inv = reinterpret_cast<int*>(w + wl.inv);
  a.h = reinterpret_cast<uint16_t*>(w + wl.h);
  a.y = reinterpret_cast<float*>(w + wl.y);
  a.out_ids = topk_ids;
  a.out_w = topk_w;
  return moe::launch_prefill(a, stream) == 0 ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_decode_layer(moe_layer_t L, const void* x, const void* router_w, const void* expert_packed,
                     const void* scales, const void* shared_w, void* out, int batch, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = L->d;
  if (int st = check_call(d, x, router_w, expert_packed, scales, shared_w, out, batch)) return st;
  const moe::FusedArgs a = make_args(L, x, router_w, expert_packed, scales, shared_w, out, batch);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!L->prof.empty()) {
    void* const* ev = L->prof.data() + 2 * (L->prof_call % (L->prof.size() / 2));
    ++L->prof_call;
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[0]), st);
    const int r = launch_layer(L, a, stream);
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[1]), st);
    if (r != 0) return MOE_ERR_LAUNCH;
  } else if (launch_layer(L, a, stream) != 0) {
    return MOE_ERR_LAUNCH;
  }
  L->last_batch = batch;
  return MOE_OK;
}

int moe_decode_layer_static(const moe_layer_desc* desc, const void* x, const void* router_w,
                            const void* expert_packed, const void* scales, const void* shared_w, void* out,
                            int batch, unsigned* err_flags, void* stream) {
  Plan p;
  if (int st = plan_shapes(desc, &p)) return st;
  const WsLayout wl = ws_layout(desc, p);
  if (wl.total > moe::kStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
  if (int st = check_call(*desc, x, router_w, expert_packed, scales, shared_w, out, batch)) return st;
  if (err_flags != nullptr && (reinterpret_cast<uintptr_t>(err_flags) & 3u)) return MOE_ERR_ALIGNMENT;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  void* base = moe::static_scratch(device);
  if (base == nullptr) return MOE_ERR_DEVICE;
  if (!cached_plan(desc, device, &p)) return MOE_ERR_UNSUPPORTED;
  moe_layer L;                      // on the stack: no workspace of its own
  L.d = *desc;
  L.p = p;
  L.device = device;
  (void)moe_expert_layout_query(desc, MOE_SET_ROUTED, &L.lr);
  (void)moe_expert_layout_query(desc, MOE_SET_SHARED, &L.ls);
  bind_ws(&L, base, wl);
  if (err_flags != nullptr) L.err = err_flags;
  const moe::FusedArgs a = make_args(&L, x, router_w, expert_packed, scales, shared_w, out, batch);
  if (launch_layer(&L, a, stream) != 0) return MOE_ERR_LAUNCH;
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
  if (n_events < 2 || n_events % 2) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  L->prof.assign(events, events + n_events);
  L->prof_call = 0;
  return MOE_OK;
}

int moe_decode_chain(const moe_layer_t* layers, int n_layers, const void* x, const void* const* router_w,
                     const void* const* expert_packed, const void* const* scales, const void* const* shared_w,
                     void* out, int batch, void* stream) {
  if (layers == nullptr || n_layers < 1 || n_layers > MOE_MAX_CHAIN || !router_w || !expert_packed || !scales ||
      !shared_w)
    return MOE_ERR_INVALID_ARG;
  const moe_layer* L0 = layers[0];
  if (L0 == nullptr) return MOE_ERR_INVALID_ARG;
  if (batch != 1) return MOE_ERR_UNSUPPORTED;
  if (!L0->p.b1 || L0->force_general) return MOE_ERR_UNSUPPORTED;
  const moe_layer_desc& d0 = L0->d;
  if (d0.routed_wtype != MOE_W_NVFP4) return MOE_ERR_UNSUPPORTED;   // the chain kernel reads NVFP4 experts
  moe::B1Args b;
  b.r2bit = 0;
  b.xx = L0->xx;
  b.n = n_layers;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer* Ll = layers[l];
    if (Ll == nullptr) return MOE_ERR_INVALID_ARG;
    const moe_layer_desc& d = Ll->d;
    if (d.hidden != d0.hidden || d.inter != d0.inter || d.n_routed != d0.n_routed || d.top_k != d0.top_k ||
        d.n_shared != d0.n_shared || d.routed_wtype != d0.routed_wtype || d.shared_wtype != d0.shared_wtype ||
        d.route != d0.route || Ll->device != L0->device || !Ll->p.b1)
      return MOE_ERR_UNSUPPORTED;
    if (int st = check_call(d, x, router_w[l], expert_packed[l], scales[l], shared_w[l], out, batch)) return st;
    const moe::FusedArgs a = make_args(Ll, x, router_w[l], expert_packed[l], scales[l], shared_w[l], out, batch);
    if (l == 0) b.a = a;
    b.L[l] = moe::chain_layer_of(a);
  }
  if (moe::launch_b1(b, stream) != 0) return MOE_ERR_LAUNCH;
  for (int l = 0; l < n_layers; ++l) layers[l]->last_batch = batch;
  return MOE_OK;
}

int moe_layer_set_path(moe_layer_t L, int path, int* active) {
  if (L == nullptr || (path != MOE_PATH_AUTO && path != MOE_PATH_GENERAL)) return MOE_ERR_INVALID_ARG;
  if (path == MOE_PATH_GENERAL && L->d.routed_wtype == MOE_W_2BIT) return MOE_ERR_UNSUPPORTED;   // no general kernel
  L->force_general = path == MOE_PATH_GENERAL;
  if (active) *active = ((L->p.b1 || L->p.b8) && !L->force_general) ? MOE_PATH_DEDICATED : MOE_PATH_GENERAL;
  return MOE_OK;
}

int moe_layer_debug_h(moe_layer_t L, void* h_routed, void* h_shared, void* stream) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (L->last_batch == 0) return MOE_ERR_STATE;
  const moe::FusedArgs a = make_args(L, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, L->last_batch);
  if (moe::launch_fused_debug_h(a, static_cast<uint16_t*>(h_routed), static_cast<uint16_t*>(h_shared), stream) != 0)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

int moe_layer_error(moe_layer_t L, unsigned* flags, int clear) {
  if (L == nullptr || flags == nullptr) return MOE_ERR_INVALID_ARG;
  if (hipMemcpy(flags, L->err, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  if (clear && *flags != 0u && hipMemset(L->err, 0, sizeof(unsigned)) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

int moe_layer_reset(moe_layer_t L) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess || hipMemset(L->ws, 0, L->ws_bytes) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  L->last_batch = 0;
  return MOE_OK;
}

int moe_layer_grid(moe_layer_t L, int* workgroups, int* lds_bytes) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  const int ti = tb_index(L->p.tbmax);
  if (workgroups) *workgroups = L->p.G;
  if (lds_bytes) *lds_bytes = L->p.lds_act[ti] + L->p.lds_acc[ti];
  return MOE_OK;
}

}  // extern "C"
