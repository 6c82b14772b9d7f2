// HIP kernels of the small-batch MoE decode layer for MI355X (gfx950, CDNA4).
//
// One layer call is three kernels on one stream:
//   k1_router_shared : router GEMV (+ pre-norm prologue) and, in the same grid,
//                      the shared experts' gate/up GEMV with SiLU*up (they do
//                      not depend on routing).
//   k2_gateup        : every workgroup first computes the routing from the
//                      logits (top-k, weights, the union of the selected
//                      experts across the batch; workgroup 0 also stores it for
//                      kernel 3), then the gate/up GEMV of its selected routed
//                      expert, SiLU*up epilogue, h in bf16 to the workspace.
//   k3_down          : down GEMV of every selected and shared expert with the
//                      weighted combine fused in; each workgroup owns a tile of
//                      output rows and sums the experts in a fixed order
//                      (deterministic, no atomics), adds the residual, rounds
//                      once to bf16.
// Flint page ("From 1,096 kernels to 346"): the router and expert GEMVs read
// only the selected experts' weights, and routing and the combine are fused
// into the neighbouring GEMV kernels.
//
// GEMV core: a wavefront lane owns a 32-element chunk of a weight row per
// step (one 128-bit load of e2m1 codes, or four of bf16) plus two e4m3 block
// scales, converts the codes to bf16 pairs in registers
// (v_cvt_scalef32_pk_bf16_fp4) and accumulates with v_dot2_f32_bf16 against
// the activation chunk it holds in VGPRs; the two 16-element block partial
// sums are scaled by their e4m3 scales (v_cvt_f32_fp8) in fp32.  Lane
// partial sums are reduced across the lanes of a row with cross-lane
// shuffles.  The NVFP4 value is e2m1 x e4m3 block scale x fp32 tensor scale
// ("Frontier MoE on consumer Blackwell (SM120)", section "GLM-5.2").

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

enum { WT_NVFP4 = 0, WT_BF16 = 1 };

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// sum_i w[i] . x[i] over the 8 bf16 pairs [OFF, OFF+8), as two independent
// 4-long dot2 chains added at the end (shorter dependency chains).
template <int OFF>
__device__ __forceinline__ float dot8(const uint32_t* w, const uint32_t* x) {
  float pa = dot2(w[OFF + 0], x[OFF + 0], 0.f);
  float pb = dot2(w[OFF + 1], x[OFF + 1], 0.f);
  pa = dot2(w[OFF + 2], x[OFF + 2], pa);
  pb = dot2(w[OFF + 3], x[OFF + 3], pb);
  pa = dot2(w[OFF + 4], x[OFF + 4], pa);
  pb = dot2(w[OFF + 5], x[OFF + 5], pb);
  pa = dot2(w[OFF + 6], x[OFF + 6], pa);
  pb = dot2(w[OFF + 7], x[OFF + 7], pb);
  return pa + pb;
}

// Two e2m1 codes (byte SEL of v; low nibble = lower element) -> bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t fp4pair(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL));
}

// 32 e2m1 codes in canonical order -> 16 bf16 pairs (pair i = elements 2i, 2i+1).
__device__ __forceinline__ void decode_chunk(const uint4& c, uint32_t w[16]) {
  w[0] = fp4pair<0>(c.x);  w[1] = fp4pair<1>(c.x);  w[2] = fp4pair<2>(c.x);  w[3] = fp4pair<3>(c.x);
  w[4] = fp4pair<0>(c.y);  w[5] = fp4pair<1>(c.y);  w[6] = fp4pair<2>(c.y);  w[7] = fp4pair<3>(c.y);
  w[8] = fp4pair<0>(c.z);  w[9] = fp4pair<1>(c.z);  w[10] = fp4pair<2>(c.z); w[11] = fp4pair<3>(c.z);
  w[12] = fp4pair<0>(c.w); w[13] = fp4pair<1>(c.w); w[14] = fp4pair<2>(c.w); w[15] = fp4pair<3>(c.w);
}

// e4m3 byte SEL of v -> fp32.
template <int SEL>
__device__ __forceinline__ float e4m3f(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, SEL);
}

// DPP lane permutes (gfx9 encodings): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror (lane i <- 7-i within 8), row_mirror (lane i <- 15-i within 16).
#define MOE_DPP_XOR1 0xB1
#define MOE_DPP_XOR2 0x4E
#define MOE_DPP_HALF_MIRROR 0x141
#define MOE_DPP_MIRROR 0x140

__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_XOR1, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_XOR2, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_HALF_MIRROR, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_MIRROR, 0xF, 0xF, false));
  }
}

// Value of lane i ^ 16 / lane i ^ 32 (gfx950 v_permlane16_swap / v_permlane32_swap
// with both operands equal: the two results hold the lane's own value and
// its partner's, in an order that depends on the half, so their sum / max
// combines a lane with its partner in every lane).
__device__ __forceinline__ float add_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ unsigned max_x16(unsigned v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((unsigned)r[0], (unsigned)r[1]);
}
__device__ __forceinline__ unsigned max_x32(unsigned v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((unsigned)r[0], (unsigned)r[1]);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
// Each step adds the value of a partner lane from the other half of the
// group, so every lane of a group ends with the same, order-fixed sum.
__device__ __forceinline__ float lane_reduce(float v, int width) {
  if (width >= 2) v += dpp_f(v, 0);
  if (width >= 4) v += dpp_f(v, 1);
  if (width >= 8) v += dpp_f(v, 2);
  if (width >= 16) v += dpp_f(v, 3);
  if (width >= 32) v = add_x16(v);
  if (width >= 64) v = add_x32(v);
  return v;
}

// Max of a 32-bit unsigned key over the wavefront, returned uniform.
__device__ __forceinline__ unsigned wave_umax(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_XOR1, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_XOR2, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_HALF_MIRROR, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_MIRROR, 0xF, 0xF, false));
  v = max_x32(max_x16(v));
  return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

// Sum over the wavefront, returned uniform (fixed order).
__device__ __forceinline__ float wave_fsum(float v) {
  v = lane_reduce(v, 64);
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key);
// both zeros map to the same key and NaN maps to 0, below every number.
__device__ __forceinline__ unsigned fkey(float f) {
  if (f != f) return 0u;
  const unsigned u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unkey(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void unpack4(const uint4& v, uint32_t* d) {
  d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
}

// ---------------------------------------------------------------------------
// activations
// ---------------------------------------------------------------------------

// Pre-norm: 1/sqrt(mean(x_b^2) + eps) for every token of the batch, into
// s_rn[b].  Whole workgroup; ends with a barrier.
__device__ void block_rms(const LayerArgs& a, float* s_rn, float* s_red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nunits = a.H / 8;
  for (int b = 0; b < a.B; ++b) {
    float s = 0.f;
    for (int u = tid; u < nunits; u += kThreads) {
      uint32_t d[4];
      unpack4(ld16(a.x + (size_t)b * a.H + u * 8), d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = bf16lo(d[i]), hi = bf16hi(d[i]);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
      }
    }
    s = lane_reduce(s, 64);
    if (lane == 0) s_red[wave * MOE_MAX_BATCH + b] = s;
  }
  __syncthreads();
  if (tid < a.B) {
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += s_red[w * MOE_MAX_BATCH + tid];
    s_rn[tid] = 1.0f / sqrtf(s / (float)a.H + a.eps);
  }
  __syncthreads();
}

// xhat pair = bf16(x * rn * gamma) elementwise on a packed bf16 pair.
__device__ __forceinline__ uint32_t norm_pair(uint32_t xv, uint32_t gv, float rn) {
  const float lo = (bf16lo(xv) * rn) * bf16lo(gv);
  const float hi = (bf16hi(xv) * rn) * bf16hi(gv);
  return f2bf(lo) | (f2bf(hi) << 16);
}

// The 32-element activation chunk starting at column col0 for every token in
// `mask`, as 16 bf16 pairs per token.  rn != null applies the pre-norm.
template <int TB>
__device__ __forceinline__ void load_act(uint32_t (&xr)[TB][16], const uint16_t* act, int H, int col0,
                                         unsigned mask, const float* rn, const uint16_t* gamma) {
  // every load is issued before any is used: rows of tokens outside `mask`
  // are redirected to the first token of the mask and zeroed afterwards
  const int b0 = __builtin_ctz(mask | 0x80000000u);
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int bb = ((mask >> b) & 1u) ? b : b0;
    const uint16_t* p = act + (size_t)bb * H + col0;
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(ld16(p + 8 * q), &xr[b][4 * q]);
  }
#pragma unroll
  for (int b = 0; b < TB; ++b)
    if (!((mask >> b) & 1u))
#pragma unroll
      for (int i = 0; i < 16; ++i) xr[b][i] = 0u;
  if (rn != nullptr) {
    uint32_t gr[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(ld16(gamma + col0 + 8 * q), &gr[4 * q]);
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if ((mask >> b) & 1u) {
        const float r = rn[b];
#pragma unroll
        for (int i = 0; i < 16; ++i) xr[b][i] = norm_pair(xr[b][i], gr[i], r);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gate/up GEMV with SiLU*up epilogue (shared experts in k1, routed in k2)
// ---------------------------------------------------------------------------

// First activation column of this lane's chunk in the gate/up GEMV.
__device__ __forceinline__ int gateup_col0(const MatGeom& g) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane % g.lpr;
  const int jj = (j < g.cw) ? j : 0;      // idle lanes read a valid chunk
  return ((wave % g.ns) * g.cw + jj) * 32;
}

// One workgroup: kWaves wavefronts.  Wave w takes slice w % ns of the rows
// and row group w / ns; each wave covers kGateSteps gate steps and the same
// number of up steps (rows I apart).  h[b][r] = SiLU(g13 * gate) * (g13 * up)
// rounded to bf16, written to h_out[b * I + r].
template <int TB, int WT>
__device__ void gateup_block(const LayerArgs& a, const uint8_t* codes, const uint8_t* scales, float g13,
                            int item, const uint32_t (&xr)[TB][16], unsigned mask, uint16_t* h_out,
                            float* s_part) {
  const MatGeom& g = a.g13;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % g.ns, rg = wave / g.ns, nrg = kWaves / g.ns;
  const int ri = lane / g.lpr, j = lane % g.lpr;
  const bool active = j < g.cw;
  const int t0 = (item * nrg + rg) * kGateSteps;
  const int gate_steps = a.I / g.rpw;

  float acc[TB][2][kGateSteps];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int st = 0; st < kGateSteps; ++st) acc[b][q][st] = 0.f;

  // 1. this wave's weight loads (HBM)
  uint4 cq[2][kGateSteps];        // nvfp4 codes
  uint32_t sw[2];                 // nvfp4 scale words
  uint4 cb[2][kGateSteps][4];     // bf16 weights
  if (active) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = t0 + q * gate_steps;
      if constexpr (WT == WT_NVFP4) {
#pragma unroll
        for (int st = 0; st < kGateSteps; ++st) cq[q][st] = ld16(codes + code_unit(g, slice, t + st, ri, j) * 16);
        sw[q] = *reinterpret_cast<const uint32_t*>(scales + scale_word(g, slice, t, ri, j));
      } else {
#pragma unroll
        for (int st = 0; st < kGateSteps; ++st)
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
            cb[q][st][sub] = ld16(codes + bf16_unit(g, slice, t + st, sub, ri, j) * 16);
      }
    }
  }
  // 2. compute
  if (active) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int st = 0; st < kGateSteps; ++st) {
        uint32_t w[16];
        float s0 = 1.f, s1 = 1.f;
        if constexpr (WT == WT_NVFP4) {
          s0 = (st == 0) ? e4m3f<0>(sw[q]) : e4m3f<2>(sw[q]);
          s1 = (st == 0) ? e4m3f<1>(sw[q]) : e4m3f<3>(sw[q]);
          decode_chunk(cq[q][st], w);
        } else {
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) unpack4(cb[q][st][sub], &w[4 * sub]);
        }
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          if ((mask >> b) & 1u) {
            const float p0 = dot8<0>(w, xr[b]);
            const float p1 = dot8<8>(w, xr[b]);
            acc[b][q][st] = (WT == WT_NVFP4) ? fmaf(p1, s1, p0 * s0) : p0 + p1;
          }
        }
      }
    }
  }

  // reduce the lanes of each row
#pragma unroll
  for (int b = 0; b < TB; ++b)
    if ((mask >> b) & 1u)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int st = 0; st < kGateSteps; ++st) acc[b][q][st] = lane_reduce(acc[b][q][st], g.lpr);

  if (g.ns > 1) {
    // rows are split over ns waves: combine the slices in slice order
    float* mine = s_part + wave * (TB * 2 * kGateSteps);
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int st = 0; st < kGateSteps; ++st) mine[(b * 2 + q) * kGateSteps + st] = acc[b][q][st];
    }
    __syncthreads();
    if (slice != 0) return;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int st = 0; st < kGateSteps; ++st) {
          float v = 0.f;
          for (int s = 0; s < g.ns; ++s)
            v += s_part[(rg * g.ns + s) * (TB * 2 * kGateSteps) + (b * 2 + q) * kGateSteps + st];
          acc[b][q][st] = v;
        }
  }

  if (j == 0) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if ((mask >> b) & 1u) {
#pragma unroll
        for (int st = 0; st < kGateSteps; ++st) {
          const float gt = acc[b][0][st] * g13;
          const float up = acc[b][1][st] * g13;
          const float h = gt / (1.0f + __expf(-gt)) * up;
          const int r = (t0 + st) * g.rpw + ri;
          h_out[(size_t)b * a.I + r] = (uint16_t)f2bf(h);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// routing, recomputed by every workgroup of k2 from the router logits
// ---------------------------------------------------------------------------

struct RouteSmem {
  unsigned mask[MOE_MAX_ROUTED];                       // token mask per expert
  unsigned ckey[MOE_MAX_BATCH][kWaves * MOE_MAX_TOPK]; // per-wave candidates (keys), wave-major
  int cexp[MOE_MAX_BATCH][kWaves * MOE_MAX_TOPK];      // and their experts
  float wmax[MOE_MAX_BATCH][kWaves];                   // sink: per-wave max logit
  float wsum[MOE_MAX_BATCH][kWaves];                   //       and sum of exp(l - max)
  int sel[MOE_MAX_BATCH][MOE_MAX_TOPK];                // selected experts, selection order
  float selw[MOE_MAX_BATCH][MOE_MAX_TOPK];             // their combine weights
  float shc[MOE_MAX_BATCH][MOE_MAX_SHARED];            // shared-expert coefficients
  int ids[MOE_MAX_BATCH * MOE_MAX_TOPK];               // distinct experts, ascending
  unsigned dmask[MOE_MAX_BATCH * MOE_MAX_TOPK];
  int cnt[kWaves];
  int nd;
};

// Routing from the router logits, computed by a whole workgroup.
//
// Top-k per token in two stages.  (1) Wave w holds experts
// [64 w p, 64 (w+1) p) (p = 1 or 2 per lane, consecutive), keys = order-
// preserving integers of the fp32 logits (experts past E and NaN logits get
// key 0), and picks its local top-k in k rounds: the largest lane head over
// the wave, ties to the lowest lane, which is the lowest expert because
// lanes hold consecutive experts.  (2) One wave ranks the 4k candidates:
// a candidate's rank counts the candidates with a larger key, plus those
// with an equal key that come earlier (lower wave, or earlier pick of the
// same wave, i.e. lower expert index).  Ranks below k are the selection, in
// order.  Then the routing weights, and the ascending list of distinct
// selected experts with their token masks.  Ends with a barrier.
__device__ void route_block(const LayerArgs& a, RouteSmem& sm) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int p = (a.Er > 256) ? 2 : 1;
  const int e0i = (wave * 64 + lane) * p;
  for (int e = tid; e < a.E; e += kThreads) sm.mask[e] = 0u;
  // all logits of all tokens issued before any is used (clamped addresses)
  float lv[MOE_MAX_BATCH][2];
#pragma unroll
  for (int b = 0; b < MOE_MAX_BATCH; ++b) {
    const float* lg = a.logits + (size_t)min(b, a.B - 1) * a.Er;
    lv[b][0] = lg[min(e0i, a.Er - 1)];
    lv[b][1] = lg[min(e0i + 1, a.Er - 1)];
  }

#pragma unroll
  for (int b = 0; b < MOE_MAX_BATCH; ++b) {
    if (b >= a.B) break;
    unsigned k0 = (e0i < a.E) ? fkey(lv[b][0]) : 0u;
    unsigned k1 = (p == 2 && e0i + 1 < a.E) ? fkey(lv[b][1]) : 0u;
    int x0 = e0i, x1 = e0i + 1;
    if (k1 > k0) {
      const unsigned tk = k0; k0 = k1; k1 = tk;
      const int te = x0; x0 = x1; x1 = te;
    }
    if (p == 1) { k1 = 0u; x1 = 0x7fffffff; }
    for (int r = 0; r < a.k; ++r) {
      const unsigned m = wave_umax(k0);
      const int win = __builtin_ctzll(__ballot(k0 == m));
      const int e_sel = __builtin_amdgcn_readlane(x0, win);
      if (lane == 0) {
        sm.ckey[b][wave * a.k + r] = m;
        sm.cexp[b][wave * a.k + r] = e_sel;
      }
      if (lane == win) { k0 = k1; x0 = x1; k1 = 0u; x1 = 0x7fffffff; }
    }
    if (a.route == MOE_ROUTE_SOFTMAX_SINK) {
      const bool v0 = e0i < a.Er, v1 = (p == 2) && (e0i + 1 < a.Er);
      float mx = fmaxf(v0 ? lv[b][0] : -INFINITY, v1 ? lv[b][1] : -INFINITY);
      mx = unkey(wave_umax(fkey(mx)));
      float sv = (v0 ? expf(lv[b][0] - mx) : 0.f) + (v1 ? expf(lv[b][1] - mx) : 0.f);
      sv = wave_fsum(sv);
      if (lane == 0) {
        sm.wmax[b][wave] = mx;
        sm.wsum[b][wave] = sv;
      }
    }
  }
  __syncthreads();

  const int nc = kWaves * a.k;
  for (int b = wave; b < a.B; b += kWaves) {
    const unsigned ki = (lane < nc) ? sm.ckey[b][lane] : 0u;
    int ei = (lane < nc) ? sm.cexp[b][lane] : 0;
    int rank = 0;
    for (int jc = 0; jc < nc; ++jc) {
      const unsigned kj = (unsigned)__builtin_amdgcn_readlane((int)ki, jc);
      rank += (kj > ki || (kj == ki && jc < lane)) ? 1 : 0;
    }
    const bool sel = lane < nc && rank < a.k;
    ei = min(max(ei, 0), a.E - 1);          // in range whatever the inputs
    float mx = 0.f, z = 1.f;
    if (a.route == MOE_ROUTE_SOFTMAX_SINK) {
      mx = fmaxf(fmaxf(sm.wmax[b][0], sm.wmax[b][1]), fmaxf(sm.wmax[b][2], sm.wmax[b][3]));
      z = 0.f;
      for (int w = 0; w < kWaves; ++w) z += sm.wsum[b][w] * expf(sm.wmax[b][w] - mx);
    }
    const float l = unkey(ki);
    float v = 0.f;
    if (sel) v = (a.route == MOE_ROUTE_SOFTMAX_SINK) ? expf(l - mx) / z : 1.0f / (1.0f + expf(-l));
    float w = v;
    if (a.route != MOE_ROUTE_SOFTMAX_SINK) w = v / wave_fsum(v);
    if (sel) {
      sm.sel[b][rank] = ei;
      sm.selw[b][rank] = w;
      atomicOr(&sm.mask[ei], 1u << b);
    }
    if (lane < a.S)
      sm.shc[b][lane] = (a.route == MOE_ROUTE_SOFTMAX_SINK)
                            ? expf(a.logits[(size_t)b * a.Er + a.E + lane] - mx) / z : 1.0f;
  }
  __syncthreads();

  // compaction: distinct experts in ascending order
  int base_pos = 0;
  for (int base = 0; base < a.E; base += kThreads) {
    const int e = base + tid;
    const unsigned mk = (e < a.E) ? sm.mask[e] : 0u;
    const bool flag = mk != 0u;
    const unsigned long long bal = __ballot(flag);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sm.cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base_pos;
    for (int w = 0; w < wave; ++w) off += sm.cnt[w];
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += sm.cnt[w];
    if (flag) {
      sm.ids[off + below] = e;
      sm.dmask[off + below] = mk;
    }
    base_pos += tot;
    __syncthreads();
  }
  if (tid == 0) sm.nd = base_pos;
  __syncthreads();
}

// The routing of this call, for the down kernel and the readback hooks.
// rt_wt holds each (slot, token) combine weight already multiplied by the
// expert's W2 tensor scale.
template <int WTR>
__device__ void write_route_table(const LayerArgs& a, const RouteSmem& sm) {
  const int tid = threadIdx.x;
  if (tid == 0) a.rt_nd[0] = sm.nd;
  for (int d = tid; d < sm.nd; d += kThreads) {
    const int e = sm.ids[d];
    const unsigned mk = sm.dmask[d];
    const float g2 = (WTR == WT_NVFP4) ? a.r_tscale[2 * e + 1] : 1.0f;
    a.rt_ids[d] = e;
    a.rt_mask[d] = mk;
    for (int b = 0; b < a.maxB; ++b) {
      float w = 0.f;
      if (b < a.B && ((mk >> b) & 1u))
        for (int r = 0; r < a.k; ++r)
          if (sm.sel[b][r] == e) w = sm.selw[b][r];
      a.rt_wt[d * a.maxB + b] = w * g2;
    }
  }
  for (int i = tid; i < a.B * a.k; i += kThreads) {
    a.topk_ids[i] = sm.sel[i / a.k][i % a.k];
    a.topk_w[i] = sm.selw[i / a.k][i % a.k];
  }
  for (int i = tid; i < a.B * a.S; i += kThreads) a.shared_c[i] = sm.shc[i / a.S][i % a.S];
}

// ---------------------------------------------------------------------------
// kernel 1: router GEMV (+ routing) and shared experts' gate/up
// ---------------------------------------------------------------------------

// Router: wave per router row; lane owns 16 B units u = pass*256 + it*64 + lane
// of the row (8 bf16 each), so every load instruction covers 1 KB contiguous.
template <int TB>
__device__ void router_part(const LayerArgs& a, const float* s_rn) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + wave;
  const bool has_row = row < a.Er;
  const int nunits = a.H / 8;
  const bool write_xhat = a.prenorm && blockIdx.x == 0 && wave == 0;
  float acc[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) acc[b] = 0.f;

  for (int base = 0; base < nunits; base += 256) {
    uint4 wv[4];
    uint32_t xr[TB][4][4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = base + it * 64 + lane;
      if (has_row && u < nunits) wv[it] = ld16(a.router_w + (size_t)row * a.H + u * 8);
      else wv[it] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = base + it * 64 + lane;
      const bool ok = u < nunits;
      uint32_t gr[4] = {0u, 0u, 0u, 0u};
      if (ok && a.prenorm) unpack4(ld16(a.gamma + u * 8), gr);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if (ok && b < a.B) {
          unpack4(ld16(a.x + (size_t)b * a.H + u * 8), xr[b][it]);
          if (a.prenorm) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[b][it][i] = norm_pair(xr[b][it][i], gr[i], s_rn[b]);
            if (write_xhat)
              *reinterpret_cast<uint4*>(a.xhat + (size_t)b * a.H + u * 8) =
                  make_uint4(xr[b][it][0], xr[b][it][1], xr[b][it][2], xr[b][it][3]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[b][it][i] = 0u;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint32_t w4[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[b] = dot2(w4[i], xr[b][it][i], acc[b]);
    }
  }

  if (has_row) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if (b < a.B) {
        const float v = lane_reduce(acc[b], 64);
        if (lane == 0) {
          const float bias = (a.bias != nullptr && row < a.E) ? a.bias[row] : 0.f;
          a.logits[(size_t)b * a.Er + row] = v + bias;
        }
      }
    }
  }

}

template <int TB, int WTS>
__global__ __launch_bounds__(kThreads) void k1_router_shared(LayerArgs a) {
  __shared__ float s_rn[MOE_MAX_BATCH];
  __shared__ float s_red[kWaves * MOE_MAX_BATCH];
  __shared__ float s_part[kWaves * TB * 2 * kGateSteps];
  if (a.prenorm) block_rms(a, s_rn, s_red);
  if ((int)blockIdx.x < a.n_router_blocks) {
    router_part<TB>(a, s_rn);
    return;
  }
  const int sb = blockIdx.x - a.n_router_blocks;
  const int s = sb / a.wpe13, item = sb % a.wpe13;
  const uint8_t* codes = a.s_codes + (size_t)s * a.s_code_stride;
  const uint8_t* scales = (WTS == WT_NVFP4) ? a.s_scales + (size_t)s * a.s_scale_stride : nullptr;
  const float g13 = (WTS == WT_NVFP4) ? a.s_tscale[2 * s] : 1.0f;
  const unsigned mask = (1u << a.B) - 1u;
  uint32_t xr[TB][16];
  load_act<TB>(xr, a.x, a.H, gateup_col0(a.g13), mask, a.prenorm ? s_rn : nullptr, a.gamma);
  gateup_block<TB, WTS>(a, codes, scales, g13, item, xr, mask, a.h_shared + (size_t)s * a.maxB * a.I, s_part);
}

// ---------------------------------------------------------------------------
// kernel 2: gate/up of the selected routed experts
// ---------------------------------------------------------------------------

template <int TB, int WTR>
__global__ __launch_bounds__(kThreads) void k2_gateup(LayerArgs a) {
  __shared__ float s_part[kWaves * TB * 2 * kGateSteps];
  __shared__ RouteSmem sm;
  // activations of every token: issued together with the logits loads
  uint32_t xr[TB][16];
  load_act<TB>(xr, a.prenorm ? a.xhat : a.x, a.H, gateup_col0(a.g13), (1u << a.B) - 1u, nullptr, nullptr);
  route_block(a, sm);
  if (blockIdx.x == 0) write_route_table<WTR>(a, sm);
  const int d = blockIdx.x / a.wpe13, item = blockIdx.x % a.wpe13;
  if (d >= sm.nd) return;  // fewer distinct experts than the grid allows for
  const int e = sm.ids[d];
  if (e < 0 || e >= a.E) return;
  const unsigned mask = sm.dmask[d];
#pragma unroll
  for (int b = 0; b < TB; ++b)
    if (!((mask >> b) & 1u))
#pragma unroll
      for (int i = 0; i < 16; ++i) xr[b][i] = 0u;
  const uint8_t* codes = a.r_codes + (size_t)e * a.r_code_stride;
  const uint8_t* scales = (WTR == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride : nullptr;
  const float g13 = (WTR == WT_NVFP4) ? a.r_tscale[2 * e] : 1.0f;
  gateup_block<TB, WTR>(a, codes, scales, g13, item, xr, mask, a.h_routed + (size_t)d * a.maxB * a.I, s_part);
}

// ---------------------------------------------------------------------------
// kernel 3: down GEMV + weighted combine (+ residual)
// ---------------------------------------------------------------------------

// Weight and activation registers of one down-GEMV item.
template <int TB, int WT, int S3>
struct DownRegs {
  uint4 c[WT == WT_NVFP4 ? S3 : 4 * S3];
  uint32_t sw[S3 / 2];
  uint32_t hr[TB][16];
};

template <int TB, int WT, int S3, typename Item>
__device__ __forceinline__ void down_load(DownRegs<TB, WT, S3>& r, const Item& d, const MatGeom& g, int t0,
                                          int ri, int j, int I) {
  if constexpr (WT == WT_NVFP4) {
#pragma unroll
    for (int st = 0; st < S3; ++st) r.c[st] = ld16(d.codes + code_unit(g, 0, t0 + st, ri, j) * 16);
#pragma unroll
    for (int p = 0; p < S3 / 2; ++p)
      r.sw[p] = *reinterpret_cast<const uint32_t*>(d.scales + scale_word(g, 0, t0 + 2 * p, ri, j));
  } else {
#pragma unroll
    for (int st = 0; st < S3; ++st)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) r.c[4 * st + sub] = ld16(d.codes + bf16_unit(g, 0, t0 + st, sub, ri, j) * 16);
  }
  const int b0 = __builtin_ctz(d.mask | 0x80000000u);
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int bb = ((d.mask >> b) & 1u) ? b : b0;
    const uint16_t* p = d.h + (size_t)bb * I + j * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(ld16(p + 8 * q), &r.hr[b][4 * q]);
  }
}

// acc[b][st] += wf[b] * (W2 h_b)[rows of step t0+st]   (lane partial sums)
template <int TB, int WT, int S3>
__device__ __forceinline__ void down_compute(const DownRegs<TB, WT, S3>& r, unsigned mask, const float (&wf)[TB],
                                             float (&acc)[TB][S3]) {
#pragma unroll
  for (int st = 0; st < S3; ++st) {
    uint32_t w[16];
    float s0 = 1.f, s1 = 1.f;
    if constexpr (WT == WT_NVFP4) {
      s0 = (st & 1) ? e4m3f<2>(r.sw[st / 2]) : e4m3f<0>(r.sw[st / 2]);
      s1 = (st & 1) ? e4m3f<3>(r.sw[st / 2]) : e4m3f<1>(r.sw[st / 2]);
      decode_chunk(r.c[st], w);
    } else {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) unpack4(r.c[4 * st + sub], &w[4 * sub]);
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if ((mask >> b) & 1u) {
        float v;
        if constexpr (WT == WT_NVFP4) {
          v = fmaf(dot8<8>(w, r.hr[b]), s1, dot8<0>(w, r.hr[b]) * s0);
        } else {
          v = dot8<0>(w, r.hr[b]) + dot8<8>(w, r.hr[b]);
        }
        acc[b][st] = fmaf(v, wf[b], acc[b][st]);
      }
    }
  }
}

template <int TB, int WT, int S3, typename Item>
__device__ __forceinline__ void down_one(const Item& d, const MatGeom& g, int t0, int ri, int j, int I,
                                         const float (&wf)[TB], float (&acc)[TB][S3]) {
  DownRegs<TB, WT, S3> r;
  down_load<TB, WT, S3>(r, d, g, t0, ri, j, I);
  down_compute<TB, WT, S3>(r, d.mask, wf, acc);
}

// Two items with all their loads issued before either is computed.
template <int TB, int WT1, int WT2, int S3, typename Item>
__device__ __forceinline__ void down_pair(const Item& d1, const Item& d2, const MatGeom& g, int t0, int ri, int j,
                                          int I, const float (&wf1)[TB], const float (&wf2)[TB],
                                          float (&acc)[TB][S3]) {
  DownRegs<TB, WT1, S3> r1;
  DownRegs<TB, WT2, S3> r2;
  down_load<TB, WT1, S3>(r1, d1, g, t0, ri, j, I);
  down_load<TB, WT2, S3>(r2, d2, g, t0, ri, j, I);
  down_compute<TB, WT1, S3>(r1, d1.mask, wf1, acc);
  down_compute<TB, WT2, S3>(r2, d2.mask, wf2, acc);
}

// One item of the down kernel: an expert (shared experts first, then the
// routed slots in ascending expert order) with its token mask, per-token
// combine weights (times the W2 tensor scale) and activations.
struct DownItem {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* h;
  unsigned mask;
  int slot;       // index into the per-slot weight table (shared: -1 - s)
};

template <int TB, int WTR, int WTS, int S3>
__global__ __launch_bounds__(kThreads) void k3_down(LayerArgs a) {
  __shared__ float s_red[kWaves * 1024];
  __shared__ int s_ids[MOE_MAX_BATCH * MOE_MAX_TOPK];
  __shared__ unsigned s_mask[MOE_MAX_BATCH * MOE_MAX_TOPK];
  __shared__ float s_wf[MOE_MAX_BATCH * MOE_MAX_TOPK * MOE_MAX_BATCH];
  __shared__ float s_cf[MOE_MAX_SHARED * MOE_MAX_BATCH];
  __shared__ int s_nd;
  const MatGeom& g = a.g2;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ri = lane / g.lpr, j = lane % g.lpr;
  const bool active = j < g.cw;
  const int t0 = blockIdx.x * S3;

  // the routing table in one round trip
  if (tid == 0) s_nd = a.rt_nd[0];
  for (int d = tid; d < a.maxd; d += kThreads) {
    s_ids[d] = a.rt_ids[d];
    s_mask[d] = a.rt_mask[d];
  }
  for (int i = tid; i < a.maxd * a.maxB; i += kThreads) s_wf[i] = a.rt_wt[i];
  for (int i = tid; i < a.S * a.B; i += kThreads) {
    const int s = i / a.B, b = i % a.B;
    const float g2 = (WTS == WT_NVFP4) ? a.s_tscale[2 * s + 1] : 1.0f;
    s_cf[s * MOE_MAX_BATCH + b] = a.shared_c[b * a.S + s] * g2;
  }
  __syncthreads();
  const int nd = s_nd;
  const int nitems = a.S + nd;

  float acc[TB][S3];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int st = 0; st < S3; ++st) acc[b][st] = 0.f;

  auto item_of = [&](int it) {
    DownItem d;
    if (it < a.S) {
      d.codes = a.s_codes + (size_t)it * a.s_code_stride + a.s_w13_code;
      d.scales = (WTS == WT_NVFP4) ? a.s_scales + (size_t)it * a.s_scale_stride + a.s_w13_scale : nullptr;
      d.h = a.h_shared + (size_t)it * a.maxB * a.I;
      d.mask = (1u << a.B) - 1u;
      d.slot = -1 - it;
    } else {
      const int sl = it - a.S;
      const int e = min(max(s_ids[sl], 0), a.E - 1);
      d.codes = a.r_codes + (size_t)e * a.r_code_stride + a.r_w13_code;
      d.scales = (WTR == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride + a.r_w13_scale : nullptr;
      d.h = a.h_routed + (size_t)sl * a.maxB * a.I;
      d.mask = s_mask[sl];
      d.slot = sl;
    }
    return d;
  };
  auto weights_of = [&](const DownItem& d, float (&wf)[TB]) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const bool on = (d.mask >> b) & 1u;
      wf[b] = !on ? 0.f : (d.slot >= 0 ? s_wf[d.slot * a.maxB + b] : s_cf[(-1 - d.slot) * MOE_MAX_BATCH + b]);
    }
  };

  if (active) {
    // wave w takes items w, w+4, w+8, ...; at small batch two items are in
    // flight at a time (their loads issued before either is computed), at
    // larger batch the activation registers allow one
    constexpr int kInFlight = (TB <= 2 && (S3 == 2 || (WTR == WT_NVFP4 && WTS == WT_NVFP4))) ? 2 : 1;
    for (int it = wave; it < nitems; it += kInFlight * kWaves) {
      const int it2 = it + kWaves;
      const DownItem d1 = item_of(it);
      float wf1[TB];
      weights_of(d1, wf1);
      if (kInFlight == 1 || it2 >= nitems) {
        if (it < a.S) down_one<TB, WTS, S3>(d1, g, t0, ri, j, a.I, wf1, acc);
        else down_one<TB, WTR, S3>(d1, g, t0, ri, j, a.I, wf1, acc);
        continue;
      }
      const DownItem d2 = item_of(it2);
      float wf2[TB];
      weights_of(d2, wf2);
      if (it2 < a.S) down_pair<TB, WTS, WTS, S3>(d1, d2, g, t0, ri, j, a.I, wf1, wf2, acc);
      else if (it < a.S) down_pair<TB, WTS, WTR, S3>(d1, d2, g, t0, ri, j, a.I, wf1, wf2, acc);
      else down_pair<TB, WTR, WTR, S3>(d1, d2, g, t0, ri, j, a.I, wf1, wf2, acc);
    }
  }

  const int rpw = g.rpw;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (b < a.B) {
#pragma unroll
      for (int st = 0; st < S3; ++st) {
        const float v = lane_reduce(acc[b][st], g.lpr);
        if (j == 0) s_red[((wave * TB + b) * S3 + st) * rpw + ri] = v;
      }
    }
  }
  __syncthreads();
  const int nout = a.B * S3 * rpw;
  for (int idx = tid; idx < nout; idx += kThreads) {
    const int b = idx / (S3 * rpw), rem = idx % (S3 * rpw);
    const int st = rem / rpw, r_in = rem % rpw;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += s_red[((w * TB + b) * S3 + st) * rpw + r_in];
    const int row = (t0 + st) * rpw + r_in;
    if (a.residual) v += bf16lo(a.x[(size_t)b * a.H + row]);
    a.out[(size_t)b * a.H + row] = (uint16_t)f2bf(v);
  }
}

// ---------------------------------------------------------------------------
// test hook: gather h of the last call in selection order
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_debug_h(LayerArgs a, uint16_t* h_r, uint16_t* h_s) {
  const int pair = blockIdx.x;
  const uint16_t* src = nullptr;
  uint16_t* dst = nullptr;
  if (pair < a.B * a.k) {
    const int b = pair / a.k;
    const int e = a.topk_ids[pair];
    const int nd = a.rt_nd[0];
    int d = -1;
    for (int i = 0; i < nd; ++i)
      if (a.rt_ids[i] == e) d = i;
    if (d < 0 || h_r == nullptr) return;
    src = a.h_routed + ((size_t)d * a.maxB + b) * a.I;
    dst = h_r + (size_t)pair * a.I;
  } else {
    const int p = pair - a.B * a.k;
    const int b = p / a.S, s = p % a.S;
    if (h_s == nullptr) return;
    src = a.h_shared + ((size_t)s * a.maxB + b) * a.I;
    dst = h_s + (size_t)p * a.I;
  }
  for (int i = threadIdx.x; i < a.I; i += kThreads) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

static inline void mark(void* const* ev, int i, hipStream_t st) {
  if (ev != nullptr) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), st);
}

template <int TB, int WTR, int WTS, int S3>
static int launch_impl(const LayerArgs& a, hipStream_t st, void* const* ev) {
  const int g1 = a.n_router_blocks + a.S * a.wpe13;
  const int nd_max = (a.B * a.k < a.E) ? a.B * a.k : a.E;
  const int g2 = nd_max * a.wpe13;
  const int g3 = a.g2.nsteps / S3;
  mark(ev, 0, st);
  hipLaunchKernelGGL((k1_router_shared<TB, WTS>), dim3(g1), dim3(kThreads), 0, st, a);
  mark(ev, 1, st);
  hipLaunchKernelGGL((k2_gateup<TB, WTR>), dim3(g2), dim3(kThreads), 0, st, a);
  mark(ev, 2, st);
  hipLaunchKernelGGL((k3_down<TB, WTR, WTS, S3>), dim3(g3), dim3(kThreads), 0, st, a);
  mark(ev, 3, st);
  return (int)hipGetLastError();
}

template <int TB, int WTR, int WTS>
static int launch_s3(const LayerArgs& a, hipStream_t st, void* const* ev) {
  if (a.s3 == 8) return launch_impl<TB, WTR, WTS, 8>(a, st, ev);
  return launch_impl<TB, WTR, WTS, 2>(a, st, ev);
}

template <int TB>
static int launch_wt(const LayerArgs& a, int rwt, int swt, hipStream_t st, void* const* ev) {
  if (rwt == WT_NVFP4 && swt == WT_NVFP4) return launch_s3<TB, WT_NVFP4, WT_NVFP4>(a, st, ev);
  if (rwt == WT_BF16 && swt == WT_BF16) return launch_s3<TB, WT_BF16, WT_BF16>(a, st, ev);
  if (rwt == WT_NVFP4 && swt == WT_BF16) return launch_s3<TB, WT_NVFP4, WT_BF16>(a, st, ev);
  return (int)hipErrorInvalidValue;
}

int launch_layer(const LayerArgs& a, int tb, int rwt, int swt, void* stream, void* const* ev4) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so it is not reported as ours
  switch (tb) {
    case 1: return launch_wt<1>(a, rwt, swt, st, ev4);
    case 2: return launch_wt<2>(a, rwt, swt, st, ev4);
    case 4: return launch_wt<4>(a, rwt, swt, st, ev4);
    case 8: return launch_wt<8>(a, rwt, swt, st, ev4);
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_debug_h(const LayerArgs& a, uint16_t* h_r, uint16_t* h_s, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int n = a.B * a.k + a.B * a.S;
  hipLaunchKernelGGL(k_debug_h, dim3(n), dim3(kThreads), 0, st, a, h_r, h_s);
  return (int)hipGetLastError();
}

}  // namespace moe
