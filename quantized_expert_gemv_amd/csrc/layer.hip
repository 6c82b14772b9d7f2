// Single-launch small-batch MoE decode layer for MI355X (gfx950, CDNA4).
//
// One launch computes the whole layer (router GEMV, routing, gate/up GEMV with
// SiLU*up, down GEMV with the weighted combine).  The Flint page ("From 1,096
// kernels to 346") runs the layer as a chain of kernels that load their
// weights early and fuse routing and the combine into the neighbouring GEMVs;
// here the chain is one grid of G workgroups, all resident at once, that hand
// data to each other through tagged words in device memory:
//
//   phase 1  every workgroup: its router row(s) -> publish logits; the shared
//            experts' gate/up rows (they do not depend on routing) -> publish
//            their SiLU*up activations
//   routing  every workgroup gathers all logits and computes the same top-k,
//            routing weights and the union of the batch's selected experts
//   phase 2  every workgroup: its slice of the selected experts' gate/up rows
//            -> publish SiLU*up activations; the down-GEMV weights this
//            workgroup needs later are already loading
//   phase 3  every workgroup gathers all activations and computes its output
//            rows: down GEMV of every selected and shared expert, summed in a
//            fixed order with the combine weights (+ residual), one bf16
//            rounding
//
// Tagged words (8 bytes): value in the low half, the call's tag in the high
// half, written and read with agent-scope atomic stores/loads.  A reader polls
// until the tag matches, so each word carries its own validity; no fences or
// barriers cross workgroups.  Every wait is bounded by a deadline: a grid whose
// workgroups are not all resident ends with an error bit set instead of
// hanging.
//
// GEMV tiles: a wavefront lane owns a 32-element chunk of a weight row per
// wave step: 16 bytes of e2m1 codes (or 64 bytes of bf16) plus the chunk's two
// e4m3 block scales.  Codes become bf16 pairs in registers
// (v_cvt_scalef32_pk_bf16_fp4), each 16-element block's partial dot
// (v_dot2_f32_bf16) is scaled by its e4m3 scale, the tensor scale is applied
// per row.  NVFP4 = e2m1 x e4m3 block-16 scale x fp32 tensor scale
// ("Frontier MoE on consumer Blackwell (SM120)", section "GLM-5.2").

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

typedef unsigned long long u64;
constexpr int NW = kFusedWaves;
constexpr int NT = kFusedThreads;
constexpr int kMaxD = MOE_MAX_BATCH * MOE_MAX_TOPK;

// ---------------------------------------------------------------------------
// tagged words
// ---------------------------------------------------------------------------

__device__ __forceinline__ u64 clock100() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ void publish(u64* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 peek(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread polls its words i = tid + NT*q (q < NB per round) of a set of n
// tagged words until their tags equal `tag`, then hands (i, value) to sink.
// addr(i) gives word i's address.  Past the deadline the error bit is set and
// the remaining words are taken as they are.
template <int NB, typename Addr, typename Sink>
__device__ __forceinline__ void gather(int n, uint32_t tag, u64 deadline, unsigned* err, unsigned bit, Addr&& addr,
                                       Sink&& sink) {
  const int tid = threadIdx.x;
  for (int base = 0; base < n; base += NB * NT) {
    u64 v[NB];
    unsigned pend = 0;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = base + q * NT + tid;
      v[q] = peek(addr(i < n ? i : 0));
      if (i < n) pend |= 1u << q;
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if ((pend >> q) & 1u)
        if ((uint32_t)(v[q] >> 32) == tag) pend &= ~(1u << q);
    while (pend != 0u) {
      if (clock100() > deadline) {
        __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((pend >> q) & 1u) v[q] = peek(addr(base + q * NT + tid));
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((pend >> q) & 1u)
          if ((uint32_t)(v[q] >> 32) == tag) pend &= ~(1u << q);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = base + q * NT + tid;
      if (i < n) sink(i, (uint32_t)v[q]);
    }
  }
}

// ---------------------------------------------------------------------------
// shared-memory state
// ---------------------------------------------------------------------------

struct Smem {
  unsigned emask[MOE_MAX_ROUTED];             // tokens that selected expert e
  int slot[MOE_MAX_ROUTED];                   // slot d of a selected expert
  int sel[MOE_MAX_BATCH][MOE_MAX_TOPK];       // per token, selection order
  float selw[MOE_MAX_BATCH][MOE_MAX_TOPK];    // routing weights
  float shc[MOE_MAX_BATCH][MOE_MAX_SHARED];   // shared-expert coefficients
  int ids[kMaxD];                             // distinct selected experts, ascending
  unsigned dmask[kMaxD];                      // their token masks
  int poff[kMaxD];                            // first activation pair of slot d
  float pw[kMaxPairs];                        // combine weight x W2 tensor scale, per pair
  float red[NW][2][MOE_MAX_BATCH];            // router / norm partial sums
  float rn[MOE_MAX_BATCH];                    // 1/rms per token
  int cnt[NW];
  int nd;
  uint32_t tag;
};

// ---------------------------------------------------------------------------
// weight tiles: one lane's share of one wave step
// ---------------------------------------------------------------------------

template <int WT> struct Tile;
template <> struct Tile<WT_NVFP4> { uint4 c; uint32_t sw; };
template <> struct Tile<WT_BF16> { uint4 c[4]; };

// Loads the lane's chunk of (slice s, step t) of a packed matrix.
template <int WT>
__device__ __forceinline__ void tile_load(Tile<WT>& tl, const uint8_t* codes, const uint8_t* scales,
                                          const MatGeom& g, int s, int t, int ri, int j) {
  if constexpr (WT == WT_NVFP4) {
    tl.c = ld16(codes + code_unit(g, s, t, ri, j) * 16);
    tl.sw = *reinterpret_cast<const uint32_t*>(scales + scale_word(g, s, t, ri, j));
  } else {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) tl.c[sub] = ld16(codes + bf16_unit(g, s, t, sub, ri, j) * 16);
  }
}

// sum over the lane's 32 weights of w * act (act: 16 bf16 pairs); NVFP4 block
// scales of step t are the bytes 2(t&1), 2(t&1)+1 of the scale word.
template <int WT>
__device__ __forceinline__ float tile_dot(const Tile<WT>& tl, int t, const uint32_t (&act)[16]) {
  uint32_t w[16];
  if constexpr (WT == WT_NVFP4) {
    decode_chunk(tl.c, w);
    const uint32_t sp = (t & 1) ? (tl.sw >> 16) : tl.sw;
    return fmaf(dot8<8>(w, act), e4m3f<1>(sp), dot8<0>(w, act) * e4m3f<0>(sp));
  } else {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) unpack4(tl.c[sub], &w[4 * sub]);
    return dot8<0>(w, act) + dot8<8>(w, act);
  }
}

// 32 bf16 activations (16 pairs) at p (16-byte aligned, shared memory).
__device__ __forceinline__ void lds_chunk(const uint16_t* p, uint32_t (&a)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack4(q[i], &a[4 * i]);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------
// experts of a gate/up phase
// ---------------------------------------------------------------------------

// Gate/up item j of a phase = (expert slot j / gs2, step pair j % gs2): gate
// steps 2 t2, 2 t2 + 1 and the up steps gate_steps later.  Its SiLU*up values
// for row-in-step ri go to activation word t2 * rpw + ri of each token's pair.
struct ItemSet {
  int shared;          // 1: shared experts (slot = shared index), 0: routed slots
  int n;               // number of items
  int lo, hi;          // this workgroup's block of items
};

struct ExpertRef {
  const uint8_t* codes;
  const uint8_t* scales;
  float g13;
  unsigned mask;
  int pair0;           // pair of the first token of the mask (routed) / token 0 (shared)
};

template <int WT>
__device__ __forceinline__ ExpertRef expert_ref(const FusedArgs& a, const Smem& s, int shared, int slot) {
  ExpertRef r;
  if (shared) {
    r.codes = a.s_codes + (size_t)slot * a.s_code_stride;
    r.scales = (WT == WT_NVFP4) ? a.s_scales + (size_t)slot * a.s_scale_stride : nullptr;
    r.g13 = (WT == WT_NVFP4) ? a.s_tscale[2 * slot] : 1.0f;
    r.mask = (1u << a.B) - 1u;
    r.pair0 = a.B * a.k + slot * a.B;
  } else {
    const int e = min(max(s.ids[slot], 0), a.E - 1);
    r.codes = a.r_codes + (size_t)e * a.r_code_stride;
    r.scales = (WT == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride : nullptr;
    r.g13 = (WT == WT_NVFP4) ? a.r_tscale[2 * e] : 1.0f;
    r.mask = s.dmask[slot];
    r.pair0 = s.poff[slot];
  }
  return r;
}

// Pair index of token b in an expert's mask.
__device__ __forceinline__ int pair_of(const ExpertRef& r, int shared, int b) {
  return shared ? r.pair0 + b : r.pair0 + __popc(r.mask & ((1u << b) - 1u));
}

// Gate/up items of one workgroup when a weight row fits one wave step (ns = 1):
// each wave takes items lo + wave, lo + wave + NW, ... on its own; a tile is
// one (gate|up, step) of an item, P tiles are in flight.
// xr: this lane's activation chunk per token.
template <int TB, int WT, int P, typename Mid>
__device__ __forceinline__ void gateup_solo(const FusedArgs& a, const Smem& s, const ItemSet& set, const uint32_t (&xr)[TB][16],
                            uint32_t tag, Mid&& mid) {
  static_assert(P % 4 == 0, "a pipeline round must hold whole items");
  const MatGeom& g = a.g13;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ri = lane / g.lpr, jj = lane % g.lpr;
  const bool active = jj < g.cw;
  const int jc = active ? jj : 0;
  const int gate_steps = a.I / g.rpw, gs2 = gate_steps / 2;
  const int first = set.lo + wave;
  const int nmine = (set.hi > first) ? (set.hi - first + NW - 1) / NW : 0;
  const int ntiles = 4 * nmine;
  const int I2 = a.I / 2;

  auto tile_step = [&](int tau, int& item) {
    item = first + (tau >> 2) * NW;
    const int q = (tau >> 1) & 1, st = tau & 1;
    return q * gate_steps + 2 * (item % gs2) + st;
  };
  auto load = [&](Tile<WT>& tl, int tau) {
    int item;
    const int t = tile_step(tau, item);
    const ExpertRef r = expert_ref<WT>(a, s, set.shared, item / gs2);
    tile_load<WT>(tl, r.codes, r.scales, g, 0, t, ri, jc);
  };

  float acc[TB][4];
  Tile<WT> buf[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < ntiles) load(buf[p], p);
  mid();
  for (int base = 0; base < ntiles; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int tau = base + p;
      if (tau < ntiles) {
        int item;
        const int t = tile_step(tau, item);
        const ExpertRef r = expert_ref<WT>(a, s, set.shared, item / gs2);
#pragma unroll
        for (int b = 0; b < TB; ++b)
          if ((r.mask >> b) & 1u) acc[b][p & 3] = active ? tile_dot<WT>(buf[p], t, xr[b]) : 0.f;
        if (tau + P < ntiles) load(buf[p], tau + P);
        if ((p & 3) == 3) {
          // item complete: reduce the lanes of each row, SiLU*up, publish
          const int t2 = item % gs2;
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if ((r.mask >> b) & 1u) {
              float v[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) v[c] = lane_reduce(acc[b][c], g.lpr);
              if (jj == 0) {
                const float h0 = silu_mul(v[0] * r.g13, v[2] * r.g13);
                const float h1 = silu_mul(v[1] * r.g13, v[3] * r.g13);
                const int pr = pair_of(r, set.shared, b);
                publish(a.xh + (size_t)pr * I2 + t2 * g.rpw + ri, f2bf(h0) | (f2bf(h1) << 16), tag);
              }
            }
          }
        }
      }
    }
  }
}

// Gate/up items when a row spans ns > 1 wave steps (slices): the ns waves of a
// group take the same items, wave w handling slice w % ns; lane-reduced
// partial sums meet in shared memory, and after one barrier the workgroup
// combines them in slice order, applies SiLU*up and publishes.
// part: TB * 4 * ns floats per item of the workgroup's block.
template <int TB, int WT, int P, typename Mid>
__device__ __forceinline__ void gateup_group(const FusedArgs& a, const Smem& s, const ItemSet& set, const uint32_t (&xr)[TB][16],
                             float* part, uint32_t tag, Mid&& mid) {
  static_assert(P % 4 == 0, "a pipeline round must hold whole items");
  const MatGeom& g = a.g13;   // here rpw = 1, lpr = 64
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ns = g.ns, ngr = NW / ns, grp = wave / ns, sl = wave % ns;
  const bool active = lane < g.cw;
  const int jc = active ? lane : 0;
  const int gate_steps = a.I, gs2 = gate_steps / 2;
  const int first = set.lo + grp;
  const int nmine = (set.hi > first) ? (set.hi - first + ngr - 1) / ngr : 0;
  const int ntiles = 4 * nmine;
  const int I2 = a.I / 2;

  auto tile_step = [&](int tau, int& item) {
    item = first + (tau >> 2) * ngr;
    const int q = (tau >> 1) & 1, st = tau & 1;
    return q * gate_steps + 2 * (item % gs2) + st;
  };
  auto load = [&](Tile<WT>& tl, int tau) {
    int item;
    const int t = tile_step(tau, item);
    const ExpertRef r = expert_ref<WT>(a, s, set.shared, item / gs2);
    tile_load<WT>(tl, r.codes, r.scales, g, sl, t, 0, jc);
  };

  Tile<WT> buf[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < ntiles) load(buf[p], p);
  mid();
  for (int base = 0; base < ntiles; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int tau = base + p;
      if (tau < ntiles) {
        int item;
        const int t = tile_step(tau, item);
        const ExpertRef r = expert_ref<WT>(a, s, set.shared, item / gs2);
        float v[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b)
          if ((r.mask >> b) & 1u) v[b] = active ? tile_dot<WT>(buf[p], t, xr[b]) : 0.f;
        if (tau + P < ntiles) load(buf[p], tau + P);
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          if ((r.mask >> b) & 1u) {
            const float sum = lane_reduce(v[b], 64);
            if (lane == 0) part[(((item - set.lo) * TB + b) * 4 + (p & 3)) * ns + sl] = sum;
          }
        }
      }
    }
  }
  __syncthreads();
  const int nitems = set.hi - set.lo;
  for (int idx = threadIdx.x; idx < nitems * TB; idx += NT) {
    const int il = idx / TB, b = idx % TB;
    const int item = set.lo + il;
    const ExpertRef r = expert_ref<WT>(a, s, set.shared, item / gs2);
    if (!((r.mask >> b) & 1u)) continue;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = 0.f;
      for (int q = 0; q < ns; ++q) acc += part[((il * TB + b) * 4 + c) * ns + q];
      v[c] = acc;
    }
    const float h0 = silu_mul(v[0] * r.g13, v[2] * r.g13);
    const float h1 = silu_mul(v[1] * r.g13, v[3] * r.g13);
    publish(a.xh + (size_t)pair_of(r, set.shared, b) * I2 + item % gs2, f2bf(h0) | (f2bf(h1) << 16), tag);
  }
}

// This lane's activation chunk(s) from the x region of shared memory.
template <int TB>
__device__ __forceinline__ void load_xr(const FusedArgs& a, const uint16_t* xs, uint32_t (&xr)[TB][16]) {
  const MatGeom& g = a.g13;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int col;
  if (g.ns == 1) {
    const int jj = lane % g.lpr;
    col = (jj < g.cw ? jj : 0) * 32;
  } else {
    col = ((wave % g.ns) * g.cw + (lane < g.cw ? lane : 0)) * 32;
  }
#pragma unroll
  for (int b = 0; b < TB; ++b) lds_chunk(xs + (size_t)min(b, a.B - 1) * a.H + col, xr[b]);
}

// mid() runs once the phase's first tiles are loading.
template <int TB, int WT, int P, typename Mid>
__device__ __forceinline__ void gateup_phase(const FusedArgs& a, const Smem& s, const ItemSet& set,
                                             const uint32_t (&xr)[TB][16], float* part, uint32_t tag, Mid&& mid) {
  if (a.g13.ns == 1) gateup_solo<TB, WT, P>(a, s, set, xr, tag, mid);
  else gateup_group<TB, WT, P>(a, s, set, xr, part, tag, mid);
}

// ---------------------------------------------------------------------------
// routing (every workgroup, from the gathered logits)
// ---------------------------------------------------------------------------

// Key for selection: order-preserving integer of the logit; NaN ranks below
// every number (key 1) and a taken expert gets key 0.
__device__ __forceinline__ unsigned sel_key(float f) {
  const unsigned k = fkey(f);
  return k == 0u ? 1u : k;
}

// Top-k per token (wave b % NW takes token b; lane l holds experts
// [l m, l m + m)), routing weights, shared coefficients; then the distinct
// selected experts in ascending order with their token masks, the pair
// offsets and the combine weight of every pair.  Ends with a barrier.
template <int WTR, int WTS>
__device__ __forceinline__ void route(const FusedArgs& a, Smem& s, const float* lg /* [B][Er] */) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < a.E; e += NT) s.emask[e] = 0u;
  __syncthreads();
  const int m = (a.E + 63) / 64;   // <= 8
  for (int b = wave; b < a.B; b += NW) {
    const float* l = lg + (size_t)b * a.Er;
    unsigned key[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane * m + i;
      key[i] = (i < m && e < a.E) ? sel_key(l[e]) : 0u;
    }
    float my_l = 0.f;   // lane r keeps the logit of the r-th selection
    for (int r = 0; r < a.k; ++r) {
      unsigned lm = key[0];
      int li = 0;
#pragma unroll
      for (int i = 1; i < 8; ++i)
        if (key[i] > lm) { lm = key[i]; li = i; }
      const unsigned M = wave_umax(lm);
      const int win = __builtin_ctzll(__ballot(lm == M));
      const int wi = __builtin_amdgcn_readlane(li, win);
      const int e_sel = min(win * m + wi, a.E - 1);
      if (lane == win) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i == wi) key[i] = 0u;
      }
      if (lane == r) my_l = unkey(M);
      if (lane == 0) {
        s.sel[b][r] = e_sel;
        atomicOr(&s.emask[e_sel], 1u << b);
      }
    }
    if (a.route == MOE_ROUTE_SOFTMAX_SINK) {
      float mx = -INFINITY;
      for (int e = lane; e < a.Er; e += 64) mx = fmaxf(mx, l[e]);
      mx = unkey(wave_umax(fkey(mx)));
      float z = 0.f;
      for (int e = lane; e < a.Er; e += 64) z += __expf(l[e] - mx);
      z = wave_fsum(z);
      if (lane < a.k) s.selw[b][lane] = __expf(my_l - mx) / z;
      if (lane < a.S) s.shc[b][lane] = __expf(l[a.E + lane] - mx) / z;
    } else {
      const float sg = (lane < a.k) ? 1.0f / (1.0f + __expf(-my_l)) : 0.f;
      const float sum = wave_fsum(sg);
      if (lane < a.k) s.selw[b][lane] = sg / sum;
      if (lane < a.S) s.shc[b][lane] = 1.0f;
    }
  }
  __syncthreads();

  // distinct experts, ascending
  int base_pos = 0;
  for (int base = 0; base < a.E; base += NT) {
    const int e = base + tid;
    const unsigned mk = (e < a.E) ? s.emask[e] : 0u;
    const bool flag = mk != 0u;
    const unsigned long long bal = __ballot(flag);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s.cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base_pos, tot = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += s.cnt[w];
      tot += s.cnt[w];
    }
    if (flag) {
      s.ids[off + below] = e;
      s.dmask[off + below] = mk;
      s.slot[e] = off + below;
    }
    base_pos += tot;
    __syncthreads();
  }
  const int nd = base_pos;
  // pair offsets: exclusive prefix of the mask popcounts (wave 0, two slots a lane)
  if (wave == 0) {
    const int c0 = (lane < nd) ? __popc(s.dmask[lane]) : 0;
    const int c1 = (lane + 64 < nd) ? __popc(s.dmask[lane + 64]) : 0;
    int i0 = c0, i1 = c1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t0 = __shfl_up(i0, d), t1 = __shfl_up(i1, d);
      if (lane >= d) { i0 += t0; i1 += t1; }
    }
    const int tot0 = __shfl(i0, 63);
    if (lane < nd) s.poff[lane] = i0 - c0;
    if (lane + 64 < nd) s.poff[lane + 64] = tot0 + i1 - c1;
    if (lane == 0) s.nd = nd;
  }
  __syncthreads();
  // combine weight of every pair (x W2 tensor scale)
  for (int i = tid; i < a.B * a.k; i += NT) {
    const int b = i / a.k, r = i % a.k;
    const int e = s.sel[b][r];
    const int d = s.slot[e];
    const int p = s.poff[d] + __popc(s.dmask[d] & ((1u << b) - 1u));
    const float g2 = (WTR == WT_NVFP4) ? a.r_tscale[2 * e + 1] : 1.0f;
    s.pw[p] = s.selw[b][r] * g2;
    if (blockIdx.x == 0) a.pair_of[i] = p;
  }
  for (int i = tid; i < a.B * a.S; i += NT) {
    const int sh = i / a.B, b = i % a.B;
    const float g2 = (WTS == WT_NVFP4) ? a.s_tscale[2 * sh + 1] : 1.0f;
    s.pw[a.B * a.k + i] = s.shc[b][sh] * g2;
  }
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.B * a.k; i += NT) {
      a.topk_ids[i] = s.sel[i / a.k][i % a.k];
      a.topk_w[i] = s.selw[i / a.k][i % a.k];
    }
    for (int i = tid; i < a.B * a.S; i += NT) a.shared_c[i] = s.shc[i / a.S][i % a.S];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// down GEMV + combine
// ---------------------------------------------------------------------------

// Down item j of this workgroup = (expert j / spg, step t_lo + j % spg); experts
// in order: shared 0..S-1, then routed slots 0..nd-1.  Wave w takes items
// w, w + NW, ...  acc: [NW][TB][spg * rpw] partial sums in shared memory.
template <int TB, int WTR, int WTS, int P>
struct DownPhase {
  const FusedArgs& a;
  const Smem& s;
  int t_lo, spg, nitems, ntiles, ri, jj, jc;
  bool active;
  Tile<WTR> bufr[P];
  Tile<WTS> bufs[(WTR == WTS) ? 1 : P];   // same types: shared tiles use bufr

  __device__ __forceinline__ DownPhase(const FusedArgs& a_, const Smem& s_, int t_lo_, int spg_)
      : a(a_), s(s_), t_lo(t_lo_), spg(spg_) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    ri = lane / a.g2.lpr;
    jj = lane % a.g2.lpr;
    active = jj < a.g2.cw;
    jc = active ? jj : 0;
    nitems = (a.S + s.nd) * spg;
    ntiles = (nitems > wave) ? (nitems - wave + NW - 1) / NW : 0;
  }
  __device__ __forceinline__ int item_of(int tau) const { return (threadIdx.x >> 6) + tau * NW; }
  __device__ __forceinline__ void load(int p, int tau) {
    const int item = item_of(tau);
    const int ex = item / spg, t = t_lo + item % spg;
    if (ex < a.S) {
      const uint8_t* c = a.s_codes + (size_t)ex * a.s_code_stride + a.s_w13_code;
      const uint8_t* sc = (WTS == WT_NVFP4) ? a.s_scales + (size_t)ex * a.s_scale_stride + a.s_w13_scale : nullptr;
      if constexpr (WTR == WTS) tile_load<WTR>(bufr[p], c, sc, a.g2, 0, t, ri, jc);
      else tile_load<WTS>(bufs[p], c, sc, a.g2, 0, t, ri, jc);
    } else {
      const int e = min(max(s.ids[ex - a.S], 0), a.E - 1);
      const uint8_t* c = a.r_codes + (size_t)e * a.r_code_stride + a.r_w13_code;
      const uint8_t* sc = (WTR == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride + a.r_w13_scale : nullptr;
      tile_load<WTR>(bufr[p], c, sc, a.g2, 0, t, ri, jc);
    }
  }
  // Issue the first P tiles (before the activations exist).
  __device__ __forceinline__ void prime() {
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (p < ntiles) load(p, p);
  }
  // hs: activations [pairs][I] bf16 in shared memory.
  __device__ __forceinline__ void run(const uint16_t* hs, float* acc) {
    const int wave = threadIdx.x >> 6;
    const int rows = spg * a.g2.rpw;
    for (int base = 0; base < ntiles; base += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int tau = base + p;
        if (tau < ntiles) {
          const int item = item_of(tau);
          const int ex = item / spg, tl = item % spg, t = t_lo + tl;
          unsigned mask;
          int pair0;
          bool sh = ex < a.S;
          if (sh) {
            mask = (1u << a.B) - 1u;
            pair0 = a.B * a.k + ex * a.B;
          } else {
            mask = s.dmask[ex - a.S];
            pair0 = s.poff[ex - a.S];
          }
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if ((mask >> b) & 1u) {
              const int pr = sh ? pair0 + b : pair0 + __popc(mask & ((1u << b) - 1u));
              uint32_t hv[16];
              lds_chunk(hs + (size_t)pr * a.I + jc * 32, hv);
              float v = 0.f;
              if (active) {
                if constexpr (WTR == WTS) v = tile_dot<WTR>(bufr[p], t, hv);
                else v = sh ? tile_dot<WTS>(bufs[p], t, hv) : tile_dot<WTR>(bufr[p], t, hv);
              }
              v = lane_reduce(v, a.g2.lpr);
              if (jj == 0) acc[(wave * TB + b) * rows + tl * a.g2.rpw + ri] += s.pw[pr] * v;
            }
          }
          if (tau + P < ntiles) load(p, tau + P);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Units (16 bytes of a row) per thread in the router phase: H <= 256 * QX * 8.
template <int TB> constexpr int fused_qx() { return TB >= 8 ? 1 : 4; }

template <int TB, int WTR, int WTS>
__global__ __launch_bounds__(NT) void k_fused_layer(FusedArgs a) {
  constexpr int QX = fused_qx<TB>();
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ Smem s;
  __shared__ float lg[TB * MOE_MAX_ROUTED];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int w = blockIdx.x, G = a.G;
  const u64 deadline = clock100() + a.wait_ticks;
  uint16_t* act = reinterpret_cast<uint16_t*>(dyn);                 // x (phases 1-2), h (phase 3)
  float* part = reinterpret_cast<float*>(dyn + (size_t)TB * a.H * 2); // gate/up partials (ns > 1)
  float* acc = reinterpret_cast<float*>(dyn + a.lds_act);            // down partial sums

  // ---- phase 1 loads: call counter, router rows, x (+ gamma) -------------
  if (tid == 0) s.tag = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int U = a.H / 8;                       // 16-byte units per row
  const int QU = (U + NT - 1) / NT;            // <= QX (the plan checks H)
  const int nrr = (w + G < a.Er) ? 2 : 1;      // router rows of this workgroup
  uint4 rw[2][QX], xv[TB][QX], gv[QX];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int u = min(tid + q * NT, U - 1);
      const int row = min(w + rr * G, a.Er - 1);
      if (q < QU && rr < nrr) rw[rr][q] = ld16(a.router_w + (size_t)row * a.H + u * 8);
    }
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int u = min(tid + q * NT, U - 1);
      if (q < QU) xv[b][q] = ld16(a.x + (size_t)min(b, a.B - 1) * a.H + u * 8);
    }
  if (a.prenorm) {
#pragma unroll
    for (int q = 0; q < QX; ++q)
      if (q < QU) gv[q] = ld16(a.gamma + (size_t)min(tid + q * NT, U - 1) * 8);
  }

  // ---- pre-norm: xhat = bf16(x / rms(x) * gamma) -----------------------------
  if (a.prenorm) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < QX; ++q) {
        if (q < QU && tid + q * NT < U) {
          const uint32_t d[4] = {xv[b][q].x, xv[b][q].y, xv[b][q].z, xv[b][q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = bf16lo(d[i]), hi = bf16hi(d[i]);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
          }
        }
      }
      ss = lane_reduce(ss, 64);
      if (lane == 0) s.red[wave][0][b] = ss;
    }
    __syncthreads();
    if (tid < TB) {
      float ss = 0.f;
      for (int q = 0; q < NW; ++q) ss += s.red[q][0][tid];
      s.rn[tid] = 1.0f / sqrtf(ss / (float)a.H + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const float rn = s.rn[b];
#pragma unroll
      for (int q = 0; q < QX; ++q) {
        if (q < QU) {
          uint4& v = xv[b][q];
          v.x = norm_pair(v.x, gv[q].x, rn);
          v.y = norm_pair(v.y, gv[q].y, rn);
          v.z = norm_pair(v.z, gv[q].z, rn);
          v.w = norm_pair(v.w, gv[q].w, rn);
        }
      }
    }
  }
  // x (or xhat) into shared memory for the gate/up tiles
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int u = tid + q * NT;
      if (q < QU && u < U && b < a.B) *reinterpret_cast<uint4*>(act + (size_t)b * a.H + u * 8) = xv[b][q];
    }

  // ---- router GEMV -> publish logits -------------------------------------------
  {
    float racc[2][TB];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        float v = 0.f;
        if (rr < nrr) {
#pragma unroll
          for (int q = 0; q < QX; ++q) {
            if (q < QU && tid + q * NT < U) {
              v = dot2(rw[rr][q].x, xv[b][q].x, v);
              v = dot2(rw[rr][q].y, xv[b][q].y, v);
              v = dot2(rw[rr][q].z, xv[b][q].z, v);
              v = dot2(rw[rr][q].w, xv[b][q].w, v);
            }
          }
        }
        racc[rr][b] = (rr < nrr) ? lane_reduce(v, 64) : 0.f;
      }
    if (lane == 0)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int b = 0; b < TB; ++b) s.red[wave][rr][b] = racc[rr][b];
  }
  __syncthreads();
  const uint32_t tag = s.tag;
  if (tid < nrr * a.B) {
    const int rr = tid / a.B, b = tid % a.B;
    const int row = w + rr * G;
    float v = 0.f;
    for (int q = 0; q < NW; ++q) v += s.red[q][rr][b];
    if (a.bias != nullptr && row < a.E) v += a.bias[row];
    publish(a.xlog + (size_t)row * kLogitLine + b, __float_as_uint(v), tag);
  }

  // ---- shared experts' gate/up (routing-independent) ----------------------------
  uint32_t xr[TB][16];
  load_xr<TB>(a, act, xr);
  const int gs2 = a.I / a.g13.rpw / 2;
  {
    ItemSet set;
    set.shared = 1;
    set.n = a.S * gs2;
    set.lo = (int)((long long)set.n * w / G);
    set.hi = (int)((long long)set.n * (w + 1) / G);
    gateup_phase<TB, WTS, (WTS == WT_NVFP4 ? 8 : 4)>(a, s, set, xr, part, tag, [] {});
  }

  // ---- routing --------------------------------------------------------------------
  gather<4>(a.Er * a.B, tag, deadline, a.err, kErrLogitWait,
            [&](int i) { return a.xlog + (size_t)(i / a.B) * kLogitLine + (i % a.B); },
            [&](int i, uint32_t v) { lg[(i % a.B) * a.Er + i / a.B] = __uint_as_float(v); });
  __syncthreads();
  if (w == 0 && tid == 0) __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  route<WTR, WTS>(a, s, lg);

  // ---- phase 2: selected experts' gate/up; the down weights start loading -----------
  const int nsteps2 = a.g2.nsteps;
  const int t_lo = (int)((long long)nsteps2 * w / G);
  const int t_hi = (int)((long long)nsteps2 * (w + 1) / G);
  DownPhase<TB, WTR, WTS, (WTR == WT_NVFP4 && WTS == WT_NVFP4) ? 6 : 3> down(a, s, t_lo, t_hi - t_lo);
  {
    ItemSet set;
    set.shared = 0;
    set.n = s.nd * gs2;
    set.lo = (int)((long long)set.n * w / G);
    set.hi = (int)((long long)set.n * (w + 1) / G);
    gateup_phase<TB, WTR, (WTR == WT_NVFP4 ? 8 : 4)>(a, s, set, xr, part, tag, [&] { down.prime(); });
  }

  // ---- phase 3: gather activations, down GEMV + combine -------------------------------
  const int rows = (t_hi - t_lo) * a.g2.rpw;
  for (int i = tid; i < NW * TB * rows; i += NT) acc[i] = 0.f;
  __syncthreads();   // every wave is done with x before h overwrites it
  const int I2 = a.I / 2;
  const int npairs = a.B * (a.k + a.S);
  {
    const int rpw = a.g13.rpw;
    gather<8>(npairs * I2, tag, deadline, a.err, kErrActWait, [&](int i) { return a.xh + i; },
              [&](int i, uint32_t v) {
                const int pr = i / I2, q = i % I2;
                const int t2 = q / rpw, ri = q % rpw;
                const int r0 = 2 * t2 * rpw + ri;
                act[(size_t)pr * a.I + r0] = (uint16_t)(v & 0xffffu);
                act[(size_t)pr * a.I + r0 + rpw] = (uint16_t)(v >> 16);
              });
  }
  __syncthreads();
  down.run(act, acc);
  __syncthreads();
  for (int i = tid; i < a.B * rows; i += NT) {
    const int b = i / rows, r = i % rows;
    float v = 0.f;
    for (int q = 0; q < NW; ++q) v += acc[(q * TB + b) * rows + r];
    const int row = t_lo * a.g2.rpw + r;
    if (a.residual) v += bf16lo(a.x[(size_t)b * a.H + row]);
    a.out[(size_t)b * a.H + row] = (uint16_t)f2bf(v);
  }
}

// Test hook: the SiLU*up activations of the last call, from the tagged words.
// h_r [B][k][I] in selection order, h_s [B][S][I].
__global__ __launch_bounds__(NT) void k_fused_debug_h(FusedArgs a, const int* pair_of_sel, uint16_t* h_r,
                                                      uint16_t* h_s) {
  const int row = blockIdx.x;   // 0 .. B*k + B*S - 1
  int pr;
  uint16_t* dst;
  if (row < a.B * a.k) {
    pr = pair_of_sel[row];
    dst = h_r ? h_r + (size_t)row * a.I : nullptr;
  } else {
    const int p = row - a.B * a.k, b = p / a.S, sh = p % a.S;
    pr = a.B * a.k + sh * a.B + b;
    dst = h_s ? h_s + (size_t)p * a.I : nullptr;
  }
  if (dst == nullptr || pr < 0) return;
  const int I2 = a.I / 2, rpw = a.g13.rpw;
  for (int q = threadIdx.x; q < I2; q += NT) {
    const u64 v = peek(a.xh + (size_t)pr * I2 + q);
    const int t2 = q / rpw, ri = q % rpw, r0 = 2 * t2 * rpw + ri;
    dst[r0] = (uint16_t)(v & 0xffffu);
    dst[r0 + rpw] = (uint16_t)((v >> 16) & 0xffffu);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <int TB, int WTR, int WTS>
static const void* fused_fn() {
  return reinterpret_cast<const void*>(&k_fused_layer<TB, WTR, WTS>);
}

template <int TB>
static const void* fused_fn_wt(int rwt, int swt) {
  if (rwt == WT_NVFP4 && swt == WT_NVFP4) return fused_fn<TB, WT_NVFP4, WT_NVFP4>();
  if (rwt == WT_BF16 && swt == WT_BF16) return fused_fn<TB, WT_BF16, WT_BF16>();
  if (rwt == WT_NVFP4 && swt == WT_BF16) return fused_fn<TB, WT_NVFP4, WT_BF16>();
  return nullptr;
}

static const void* fused_kernel(int tb, int rwt, int swt) {
  switch (tb) {
    case 1: return fused_fn_wt<1>(rwt, swt);
    case 2: return fused_fn_wt<2>(rwt, swt);
    case 4: return fused_fn_wt<4>(rwt, swt);
    case 8: return fused_fn_wt<8>(rwt, swt);
    default: return nullptr;
  }
}

int fused_occupancy(int tb, int rwt, int swt, int lds_bytes, int* blocks_per_cu) {
  const void* f = fused_kernel(tb, rwt, swt);
  if (f == nullptr) return (int)hipErrorInvalidValue;
  if (lds_bytes > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, NT, lds_bytes);
}

int launch_fused(const FusedArgs& a, int tb, int rwt, int swt, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const void* f = fused_kernel(tb, rwt, swt);
  if (f == nullptr) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();  // clear a stale error so it is not reported as ours
  void* args[] = {const_cast<FusedArgs*>(&a)};
  return (int)hipLaunchKernel(f, dim3(a.G), dim3(NT), args, (size_t)fused_lds_bytes(a), st);
}

int launch_fused_debug_h(const FusedArgs& a, const int* pair_of_sel, uint16_t* h_r, uint16_t* h_s, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int n = a.B * a.k + a.B * a.S;
  hipLaunchKernelGGL(k_fused_debug_h, dim3(n), dim3(NT), 0, st, a, pair_of_sel, h_r, h_s);
  return (int)hipGetLastError();
}

}  // namespace moe
