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
//            experts' gate/up tiles (they do not depend on routing) start
//            loading
//   routing  every workgroup gathers all logits and computes the same top-k,
//            routing weights and the union of the batch's selected experts
//   phase 2  every workgroup: its slice of the shared and the selected
//            experts' gate/up rows -> publish SiLU*up activations; the
//            down-GEMV weights this workgroup needs later are already loading
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

#include <mutex>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

// ---------------------------------------------------------------------------
// shared-memory state
// ---------------------------------------------------------------------------

struct Smem {
  float tsr[MOE_MAX_ROUTED][2];               // routed tensor scales (W13, W2)
  float tss[MOE_MAX_SHARED][2];               // shared tensor scales
  unsigned emask[MOE_MAX_ROUTED];             // tokens that selected expert e
  int slotmap[MOE_MAX_ROUTED];                // slot of a selected expert
  int sel[MOE_MAX_BATCH][MOE_MAX_TOPK];       // per token, selection order
  float selw[MOE_MAX_BATCH][MOE_MAX_TOPK];    // routing weights
  float shc[MOE_MAX_BATCH][MOE_MAX_SHARED];   // shared-expert coefficients
  int ids[kMaxD];                             // expert in slot d
  float xg[kMaxD];                            // its W13 tensor scale
  unsigned dmask[kMaxD];                      // its token mask
  uint32_t pr[kMaxD][2];                      // selection rank r of token b for slot d, byte b
  float pw[kMaxPairs];                        // combine weight x W2 tensor scale, per pair
  float red[NW][2][MOE_MAX_BATCH];            // router / norm partial sums
  float rn[MOE_MAX_BATCH];                    // 1/rms per token
  int nd;
  uint32_t tag;
  float kpart[8][4][NW];                      // batch-1 split-K gate/up partials [item][row][wave]
};

// Activation pairs: routed pair of token b's r-th selection = b k + r;
// shared expert s of token b = B k + s B + b.

// The routing's tables, spread over the lanes of every wave (entry i in lane
// i % 64 of register i / 64) and read with v_readlane: a uniform index then
// costs a few cycles instead of a shared-memory round trip.
struct SlotTab {
  uint32_t id[2], mask[2], g13[2], prlo[2], prhi[2];   // per slot
  uint32_t pw[3];                                      // per pair
  __device__ __forceinline__ void load(const Smem& s, int lane) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      id[h] = (uint32_t)s.ids[d];
      mask[h] = s.dmask[d];
      g13[h] = __float_as_uint(s.xg[d]);
      prlo[h] = s.pr[d][0];
      prhi[h] = s.pr[d][1];
    }
#pragma unroll
    for (int h = 0; h < 3; ++h) pw[h] = __float_as_uint(s.pw[min(lane + 64 * h, kMaxPairs - 1)]);
  }
  // Lookups read other lanes, so they run only in wave-uniform control flow
  // (all lanes active): inside lane-conditional code the inactive lanes of a
  // register, or of the compiler's copy of it, hold no defined value.  Each
  // register is read at lane i % 64 and the scalars are selected afterwards;
  // a conditional on the array itself would become an indexed access, which
  // puts the table in scratch memory.
  __device__ __forceinline__ static uint32_t rl(uint32_t v, int i) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, i & 63);
  }
  __device__ __forceinline__ static uint32_t pick2(const uint32_t (&v)[2], int i) {
    const uint32_t a0 = rl(v[0], i), a1 = rl(v[1], i);
    return i >= 64 ? a1 : a0;
  }
  // clamped to a valid expert (an unsigned min, which stays on the scalar unit)
  __device__ __forceinline__ int expert(int d, int E) const { return (int)min(pick2(id, d), (uint32_t)(E - 1)); }
  __device__ __forceinline__ unsigned tokens(int d) const { return pick2(mask, d); }
  __device__ __forceinline__ float w13(int d) const { return __uint_as_float(pick2(g13, d)); }
  __device__ __forceinline__ int rank(int d, int b) const {
    const uint32_t wd = (b < 4) ? pick2(prlo, d) : pick2(prhi, d);
    return (int)((wd >> (8 * (b & 3))) & 0xffu);
  }
  __device__ __forceinline__ float weight(int pr) const {
    const uint32_t a0 = rl(pw[0], pr), a1 = rl(pw[1], pr), a2 = rl(pw[2], pr);
    return __uint_as_float(pr >= 128 ? a2 : (pr >= 64 ? a1 : a0));
  }
};

// ---------------------------------------------------------------------------
// weight tiles
// ---------------------------------------------------------------------------

// This lane's place in one wave step of a packed matrix: byte offsets of its
// 16-byte code unit and 4-byte scale word inside a step, and the step strides.
struct LaneGeo {
  uint32_t su16, su4;   // bytes of one step's code units / scale words (per scale pair)
  int nsteps;
  uint32_t c_off, s_off;
  int ri, jj, jc;
  bool active;
};

// ns == 1: a step covers rpw rows of lpr lanes; ns > 1: one row, lane = chunk.
__device__ __forceinline__ LaneGeo lane_geo(const MatGeom g, int lane) {
  LaneGeo L;
  L.su16 = (uint32_t)g.su * 16u;
  L.su4 = (uint32_t)g.su * 4u;
  L.nsteps = g.nsteps;
  if (g.ns == 1) {
    L.ri = lane / g.lpr;
    L.jj = lane % g.lpr;
    L.active = L.jj < g.cw;
  } else {
    L.ri = 0;
    L.jj = lane;
    L.active = lane < g.cw;
  }
  L.jc = L.active ? L.jj : 0;
  const uint32_t u = (uint32_t)(L.ri * g.cw + L.jc);
  L.c_off = u * 16u;
  L.s_off = u * 4u;
  return L;
}

// `dummy` when dm, else `real`, computed without a branch (a branch would
// duplicate the load that uses it and make the loads in flight depend on
// data, which costs a full wait for every load before the copy).
__device__ __forceinline__ const uint8_t* pick(bool dm, const uint8_t* real, const uint8_t* dummy) {
  const uintptr_t m = (uintptr_t)0 - (uintptr_t)dm;
  return reinterpret_cast<const uint8_t*>((uintptr_t)real ^ (((uintptr_t)real ^ (uintptr_t)dummy) & m));
}

// Byte offset of expert (or shared expert) e in a region of the given stride:
// 32-bit arithmetic for a fixed shape, whose regions the host checks to be
// below 4 GiB.
template <class A>
__device__ __forceinline__ size_t expert_off(int e, size_t stride) {
  if constexpr (std::is_base_of<DynShape, A>::value) return (size_t)e * stride;
  else return (size_t)((uint32_t)e * (uint32_t)stride);
}

// Wave-uniform NVFP4 byte offsets of (slice sl, step t): code units, and the
// scale words shared by steps t & ~1 and t | 1.  A lane adds L.c_off / L.s_off.
__device__ __forceinline__ uint32_t code_step(const LaneGeo& L, int sl, int t) {
  return (uint32_t)(sl * L.nsteps + t) * L.su16;
}
__device__ __forceinline__ uint32_t scale_step(const LaneGeo& L, int sl, int t) {
  return (uint32_t)(sl * (L.nsteps >> 1) + (t >> 1)) * L.su4;
}
// BF16 unit `sub` (elements 8 sub .. 8 sub + 7 of a lane's chunk) of (sl, t).
__device__ __forceinline__ uint32_t bf16_step(const LaneGeo& L, int sl, int t, int sub) {
  return (uint32_t)((sl * L.nsteps + t) * 4 + sub) * L.su16;
}

// One lane's share of one wave step of a packed matrix.
template <int WT> struct Tile;
template <> struct Tile<WT_NVFP4> { uint4 c; uint32_t sw; };
template <> struct Tile<WT_BF16> { uint4 c[4]; };

// Loads the lane's chunk of (slice sl, step t).  A dummy load reads the first
// bytes of `dummy` instead (same instructions, so the number of loads in flight
// never depends on data; the value is unused).
template <int WT>
__device__ __forceinline__ void tile_load(Tile<WT>& tl, const uint8_t* codes, const uint8_t* scales,
                                          const LaneGeo& L, int sl, int t, bool dm, const uint8_t* dummy) {
  const uint32_t lm = dm ? 0u : ~0u;
  if constexpr (WT == WT_NVFP4) {
    tl.c = ld16o(pick(dm, codes + code_step(L, sl, t), dummy), L.c_off & lm);
    tl.sw = ld32o(pick(dm, scales + scale_step(L, sl, t), dummy), L.s_off & lm);
  } else {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) tl.c[sub] = ld16o(pick(dm, codes + bf16_step(L, sl, t, sub), dummy), L.c_off & lm);
  }
}

__device__ __forceinline__ float chunk_dot_bf16(const uint4 (&c)[4], const uint32_t (&act)[16]) {
  uint32_t w[16];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) unpack4(c[sub], &w[4 * sub]);
  return dot8<0>(w, act) + dot8<8>(w, act);
}
template <int WT>
__device__ __forceinline__ float tile_dot(const Tile<WT>& tl, int t, const uint32_t (&act)[16]) {
  if constexpr (WT == WT_NVFP4) return chunk_dot_fp4(tl.c, (t & 1) ? (tl.sw >> 16) : tl.sw, act);
  else return chunk_dot_bf16(tl.c, act);
}

// The four tiles of one gate/up item (gate steps 2t2, 2t2+1, up steps
// gate_steps + 2t2, +1) for one slice; NVFP4 scale words pair the two steps.
template <int WT> struct Quad;
template <> struct Quad<WT_NVFP4> { uint4 c[4]; uint32_t sw[2]; };
template <> struct Quad<WT_BF16> { uint4 c[4][4]; };

template <int WT>
__device__ __forceinline__ void quad_load(Quad<WT>& q, const uint8_t* codes, const uint8_t* scales, const LaneGeo& L,
                                          int sl, int gate_steps, int t2, bool dm, const uint8_t* dummy) {
  const uint32_t lm = dm ? 0u : ~0u;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = u * gate_steps + 2 * t2;
    if constexpr (WT == WT_NVFP4) {
      const uint8_t* cb = pick(dm, codes + code_step(L, sl, t), dummy);
      q.c[2 * u] = ld16o(cb, L.c_off & lm);
      q.c[2 * u + 1] = ld16o(cb + (dm ? 0u : L.su16), L.c_off & lm);
      q.sw[u] = ld32o(pick(dm, scales + scale_step(L, sl, t), dummy), L.s_off & lm);
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
          q.c[2 * u + st][sub] = ld16o(pick(dm, codes + bf16_step(L, sl, t + st, sub), dummy), L.c_off & lm);
    }
  }
}

// v = (gate st0, gate st1, up st0, up st1) lane partial dots.
template <int WT>
__device__ __forceinline__ void quad_dot(const Quad<WT>& q, const uint32_t (&x)[16], float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (WT == WT_NVFP4) v[i] = chunk_dot_fp4(q.c[i], (i & 1) ? (q.sw[i >> 1] >> 16) : q.sw[i >> 1], x);
    else v[i] = chunk_dot_bf16(q.c[i], x);
  }
}

// ---------------------------------------------------------------------------
// gate/up phases
// ---------------------------------------------------------------------------

// Gate/up items: item j = (slot j / gs2, step pair j % gs2) of the phase's n
// items.  With more than one token, workgroup w takes items w, w + G, w + 2G,
// ... (its m-th item is w + mG): every workgroup gets the same mix of experts,
// and an expert chosen by many tokens (more work per item) does not load one
// workgroup only.  With one token every item costs the same, and workgroup w
// takes the block [nw/G, n(w+1)/G) (its m-th item is nw/G + m): a wave's
// items then lie in one or two experts.
// With one wave step per row (ns = 1) wave g takes the workgroup's items
// m = g, g + NW, ... on its own and publishes their SiLU*up words; with ns > 1
// the ns waves of a group share items, wave w taking slice w % ns, and after
// one barrier the workgroup combines the slices in order.  PI items are
// loading at a time.
template <int TB, int WT>
constexpr bool kSkipRefills = TB <= 2 && WT == WT_NVFP4;

template <int TB, int WT, int PI>
struct GateUp {
  Quad<WT> q[PI];
  int qslot[PI], qt2[PI], qm[PI];
  int shared, cnt, gs2, gate_steps;   // cnt: the workgroup's items
  int j0, lgj;                          // the workgroup's m-th item is j0 + (m << lgj)
  int ns, grp, ngr, lg_ngr, sl;
  int nmine, nloaded, cslot, ct2, cm;   // this wave's item count, items loaded, next item (slot, pair, m)
  int dslot, dt2;                       // next item of the wave: + dslot slots, + dt2 pairs
  unsigned tmask;                       // tokens this wave computes (shared items at batch 4-8)
  LaneGeo L;

  // Everything that does not depend on the routing.
  template <class A>
  __device__ __forceinline__ void init(const A& a, const LaneGeo& lg13, int shared_) {
    const int wave = wave_id();
    L = lg13;
    shared = shared_;
    gate_steps = a.I / a.g13.rpw;
    gs2 = gate_steps >> 1;
    ns = a.g13.ns;
    ngr = NW / ns;
    lg_ngr = (ngr == 4) ? 2 : (ngr == 2) ? 1 : 0;
    grp = wave / ns;
    sl = wave - grp * ns;
    // shared items (at most a few per workgroup) go to the last groups, which
    // never hold more routed items than the first ones
    if (shared) grp = ngr - 1 - grp;
    tmask = ~0u;
    if (shared && TB >= 4 && ns == 1) {
      // A shared item carries every token (several routed items' work): each
      // wave takes every shared item of the workgroup for its tokens b = wave
      // (mod NW) only, so the waves stay balanced.
      tmask = 0x11111111u << wave;
      grp = 0;
      ngr = 1;
      lg_ngr = 0;
    }
  }
  // The phase's item count n.
  template <class A>
  __device__ __forceinline__ void set_items(const A& a, int n) {
    const int w = blockIdx.x;
    if constexpr (TB == 1) {
      j0 = (int)(((uint32_t)n * w) >> a.log2G);
      cnt = (int)(((uint32_t)n * (w + 1)) >> a.log2G) - j0;
      lgj = 0;
    } else {
      j0 = w;
      cnt = (n > w) ? ((n - 1 - w) >> a.log2G) + 1 : 0;
      lgj = a.log2G;
    }
    nmine = (cnt > grp) ? ((cnt - 1 - grp) >> lg_ngr) + 1 : 0;
    nloaded = 0;
    cm = grp;
    const uint32_t first = (uint32_t)j0 + ((uint32_t)grp << lgj);
    cslot = (int)fastdiv(first, a.dv_gs2);
    ct2 = (int)first - cslot * gs2;
    const uint32_t stepj = (uint32_t)ngr << lgj;
    dslot = (int)fastdiv(stepj, a.dv_gs2);
    dt2 = (int)stepj - dslot * gs2;
  }
  template <class A>
  __device__ __forceinline__ void bases(const A& a, const SlotTab& tb, int slot, const uint8_t*& c,
                                        const uint8_t*& sc) const {
    if (shared) {
      // a layer without shared experts has no shared buffer: x stands in (its
      // items are all dummies, whose loads read x anyway)
      const int sh = min(slot, MOE_MAX_SHARED - 1);
      c = (a.s_codes ? a.s_codes : reinterpret_cast<const uint8_t*>(a.x)) + expert_off<A>(sh, a.s_code_stride);
      sc = (a.s_scales ? a.s_scales : reinterpret_cast<const uint8_t*>(a.x)) + expert_off<A>(sh, a.s_scale_stride);
    } else {
      const int e = tb.expert(min(slot, kMaxD - 1), a.E);
      c = a.r_codes + expert_off<A>(e, a.r_code_stride);
      sc = (WT == WT_NVFP4) ? a.r_scales + expert_off<A>(e, a.r_scale_stride) : reinterpret_cast<const uint8_t*>(a.x);
    }
  }
  // Loads the next item of this wave, or a dummy once they are all loaded.
  template <class A>
  __device__ __forceinline__ void load_next(const A& a, const SlotTab& tb, int p) {
    const bool dm = nloaded >= nmine;
    const uint8_t *c, *sc;
    bases(a, tb, cslot, c, sc);
    quad_load<WT>(q[p], c, sc, L, sl, gate_steps, ct2, dm, reinterpret_cast<const uint8_t*>(a.x));
    qslot[p] = cslot;
    qt2[p] = ct2;
    qm[p] = cm;
    if (!dm) {
      ++nloaded;
      cm += ngr;
      cslot += dslot;
      ct2 += dt2;
      if (ct2 >= gs2) {   // dt2 < gs2
        ct2 -= gs2;
        ++cslot;
      }
    }
  }
  template <class A>
  __device__ __forceinline__ void prime(const A& a, const SlotTab& tb) {
    // a wave with no item of the phase reads none of its buffers (every step
    // is dead), so it issues nothing: no address arithmetic on the scalar
    // unit the CU's waves share, no dummy loads
    if (nmine == 0) return;
#pragma unroll
    for (int p = 0; p < PI; ++p) load_next(a, tb, p);
  }
  // One token's share of an item: dot products, lane reduction, then the
  // SiLU*up word (ns == 1) or the slice partials (ns > 1).  v holds the four
  // lane partials (gate t, gate t+1, up t, up t+1).
  template <class A>
  __device__ __forceinline__ void finish_token(const A& a, const SlotTab& tb, float (&v)[4], int slot, int t2, int m,
                                               int b, float g13, bool lead, float* part, uint32_t tag) const {
    if (!L.active) v[0] = v[1] = v[2] = v[3] = 0.f;
    if (ns == 1) {
      // the table lookup is a cross-lane read: it stays out of the
      // lane-conditional code below, where other lanes are inactive
      const int pr = shared ? a.B * a.k + slot * a.B + b : b * a.k + tb.rank(slot, b);
      const int lpr = a.g13.lpr;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = group_sum(v[c], lpr);
      if (lead) {
        const float h0 = silu_mul(v[0] * g13, v[2] * g13);
        const float h1 = silu_mul(v[1] * g13, v[3] * g13);
        publish(a.xh + (size_t)pr * (a.I / 2) + t2 * a.g13.rpw + L.ri, pack_bf16x2(h0, h1), tag);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sum = group_sum(v[c], 64);
        if (lead) part[((m * TB + b) * 4 + c) * ns + sl] = sum;
      }
    }
  }
  // Item in buffer p (live: a real item of this wave).  RELOAD: refill the
  // buffer with the wave's next item (a dummy past the end) once it is read.
  template <bool RELOAD, int XR, class A>
  __device__ __forceinline__ void step(const A& a, const Smem& s, const SlotTab& tb, const uint32_t (&xr)[XR][16],
                                       const uint16_t* xs, int xcol, float* part, uint32_t tag, int p, bool live,
                                       bool lead) {
    const int slot = qslot[p], t2 = qt2[p];
    const unsigned mask = shared ? ((1u << a.B) - 1u) & tmask : tb.tokens(min(slot, kMaxD - 1));
    const float g13 = shared ? ((WT == WT_NVFP4) ? s.tss[min(slot, MOE_MAX_SHARED - 1)][0] : 1.0f)
                             : tb.w13(min(slot, kMaxD - 1));
    if constexpr (XR == TB) {
      float v[TB][4];
      if (live) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
          if ((mask >> b) & 1u) quad_dot<WT>(q[p], xr[b], v[b]);
      }
      // The buffer is free only now.  Its reload is unconditional (a dummy
      // past the end) and kept below the reads: a conditional or hoisted
      // reload would make the compiler copy registers and wait for every
      // load in flight.
      __asm__ volatile("" ::: "memory");   // also keeps items from being interleaved
      if constexpr (RELOAD) load_next(a, tb, p);
      if (live) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
          if ((mask >> b) & 1u) finish_token(a, tb, v[b], slot, t2, qm[p], b, g13, lead, part, tag);
      }
    } else {
      if (live) {
        for (unsigned m = mask; m != 0u; m &= m - 1u) {   // uniform loop over the item's tokens
          const int b = __builtin_ctz(m);
          uint32_t xb[16];
          lds_chunk(xs + (size_t)b * a.H + xcol, xb);
          float v[4];
          quad_dot<WT>(q[p], xb, v);
          finish_token(a, tb, v, slot, t2, qm[p], b, g13, lead, part, tag);
        }
      }
      __asm__ volatile("" ::: "memory");
      if constexpr (RELOAD) load_next(a, tb, p);
    }
  }
  // xr: the tokens' activation chunks in registers (TB <= 2); otherwise each
  // token's chunk is read from shared memory (xs + b H + xcol) per item, which
  // leaves registers for more items in flight.  part: TB * 4 * ns floats per
  // item of the block (ns > 1 only).
  // xr: the tokens' activation chunks in registers (TB <= 2); otherwise each
  // token's chunk is read from shared memory (xs + b H + xcol) per item, which
  // leaves registers for more items in flight.  part: TB * 4 * ns floats per
  // item of the workgroup (ns > 1 only).
  template <int XR, class A>
  __device__ __forceinline__ void run(const A& a, const Smem& s, const SlotTab& tb, const uint32_t (&xr)[XR][16],
                                      const uint16_t* xs, int xcol, float* part, uint32_t tag) {
    const bool lead = L.jj == ((ns == 1) ? a.g13.lpr - 1 : 63);
    // Small batches: when every item of the wave is already loading, skip the
    // refills (a second copy of the loop; larger batches keep one copy, which
    // the register allocator handles better there).
    if (kSkipRefills<TB, WT> && nmine <= PI) {
#pragma unroll
      for (int p = 0; p < PI; ++p) step<false>(a, s, tb, xr, xs, xcol, part, tag, p, p < nmine, lead);
    } else {
      for (int base = 0; base < nmine; base += PI) {
#pragma unroll
        for (int p = 0; p < PI; ++p) step<true>(a, s, tb, xr, xs, xcol, part, tag, p, base + p < nmine, lead);
      }
    }
    if (ns > 1) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < cnt * TB; idx += NT) {
        const int m = idx / TB, b = idx - m * TB;
        const int j = j0 + (m << lgj), slot = (int)fastdiv((uint32_t)j, a.dv_gs2), t2 = j - slot * gs2;
        const unsigned mask = shared ? (1u << a.B) - 1u : s.dmask[min(slot, kMaxD - 1)];
        if (!((mask >> b) & 1u)) continue;
        const float g13 = shared ? ((WT == WT_NVFP4) ? s.tss[min(slot, MOE_MAX_SHARED - 1)][0] : 1.0f)
                                 : s.xg[min(slot, kMaxD - 1)];
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float acc = 0.f;
          for (int u = 0; u < ns; ++u) acc += part[((m * TB + b) * 4 + c) * ns + u];
          v[c] = acc;
        }
        const float h0 = silu_mul(v[0] * g13, v[2] * g13);
        const float h1 = silu_mul(v[1] * g13, v[3] * g13);
        const int pr = shared ? a.B * a.k + slot * a.B + b
                              : b * a.k + (int)((s.pr[slot][b >> 2] >> (8 * (b & 3))) & 0xffu);
        publish(a.xh + (size_t)pr * (a.I / 2) + t2, pack_bf16x2(h0, h1), tag);
      }
      // the partials are read: a following pass may overwrite them
      __syncthreads();
    }
  }
};

// Batch 1, shapes whose gate/up rows span one 64-lane wave step (rpw = 1):
// every wave takes every item of the workgroup over its quarter of the
// hidden dimension, so six selected items and one shared item cost each wave
// the same instead of two items on some waves and one on others.  Lane l
// holds row l / 16 of the item (gate t, gate t + 1, up t, up t + 1; t = 2 t2)
// at chunk 16 w + l % 16: one 16-byte load per item, the same lane offset for
// every item, and a 16-lane sum; the four quarters meet in shared memory and
// are summed in wave order.  KS shared and KR selected items per workgroup.
template <int KS, int KR>
struct SplitK {
  uint4 c[KS + KR];
  uint32_t sw[KS + KR];
  int js, jr;                 // first shared / selected item of the workgroup
  uint32_t off_c, off_s;      // this lane's code / scale-word byte offsets
  int row, gate_steps;

  template <class A>
  __device__ __forceinline__ void init(const A& a, const LaneGeo& L) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int w = blockIdx.x;
    gate_steps = a.I / a.g13.rpw;
    js = (int)(((uint32_t)(a.S * (gate_steps >> 1)) * w) >> a.log2G);
    jr = (int)(((uint32_t)(a.k * (gate_steps >> 1)) * w) >> a.log2G);
    row = lane >> 4;
    const uint32_t chunk = (uint32_t)(16 * wave + (lane & 15));
    off_c = chunk * 16u + ((row & 1) ? L.su16 : 0u) + ((row >> 1) ? (uint32_t)gate_steps * L.su16 : 0u);
    off_s = chunk * 4u + ((row >> 1) ? (uint32_t)(gate_steps >> 1) * L.su4 : 0u);
  }
  template <class A>
  __device__ __forceinline__ void load_item(const A& a, int m, const uint8_t* cb, const uint8_t* sb, int t2,
                                            const LaneGeo& L) {
    c[m] = ld16o(cb + (uint32_t)(2 * t2) * L.su16, off_c);
    sw[m] = ld32o(sb + (uint32_t)t2 * L.su4, off_s);
  }
  template <class A>
  __device__ __forceinline__ void load_shared(const A& a, const LaneGeo& L) {
    const int gs2 = gate_steps >> 1;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      const int j = js + m, sh = j / gs2, t2 = j - sh * gs2;
      load_item(a, m, a.s_codes + expert_off<A>(sh, a.s_code_stride), a.s_scales + expert_off<A>(sh, a.s_scale_stride),
                t2, L);
    }
  }
  template <class A>
  __device__ __forceinline__ void load_routed(const A& a, const SlotTab& tb, const LaneGeo& L) {
    const int gs2 = gate_steps >> 1;
#pragma unroll
    for (int m = 0; m < KR; ++m) {
      const int j = jr + m, slot = j / gs2, t2 = j - slot * gs2;
      const int e = tb.expert(min(slot, kMaxD - 1), a.E);
      load_item(a, KS + m, a.r_codes + expert_off<A>(e, a.r_code_stride),
                a.r_scales + expert_off<A>(e, a.r_scale_stride), t2, L);
    }
  }
  // Dot products, quarter sums into shared memory, then (after a barrier)
  // one thread per item adds the quarters and publishes the SiLU*up word.
  template <class A>
  __device__ __forceinline__ void run(const A& a, Smem& s, const uint16_t* xs, uint32_t tag) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    uint32_t xk[16];
    lds_chunk(xs + (16 * wave + (lane & 15)) * 32, xk);
    // all items' sums first, then one lane-conditional block of stores: a
    // store per item under its own condition would keep the items apart
    float v[KS + KR];
#pragma unroll
    for (int m = 0; m < KS + KR; ++m) {
      const uint32_t sp = (row & 1) ? (sw[m] >> 16) : sw[m];
      v[m] = group_sum(chunk_dot_fp4(c[m], sp, xk), 16);
    }
    if ((lane & 15) == 15) {
#pragma unroll
      for (int m = 0; m < KS + KR; ++m) s.kpart[m][row][wave] = v[m];
    }
    __syncthreads();
    const int m = threadIdx.x;
    if (m < KS + KR) {
      const int gs2 = gate_steps >> 1;
      float q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < NW; ++u) acc += s.kpart[m][r][u];
        q[r] = acc;
      }
      int pr, t2;
      float g13;
      if (m < KS) {
        const int j = js + m, sh = j / gs2;
        t2 = j - sh * gs2;
        pr = a.k + sh;
        g13 = s.tss[min(sh, MOE_MAX_SHARED - 1)][0];
      } else {
        const int j = jr + m - KS, slot = j / gs2;
        t2 = j - slot * gs2;
        pr = (int)(s.pr[min(slot, kMaxD - 1)][0] & 0xffu);
        g13 = s.xg[min(slot, kMaxD - 1)];
      }
      const float h0 = silu_mul(q[0] * g13, q[2] * g13);
      const float h1 = silu_mul(q[1] * g13, q[3] * g13);
      publish(a.xh + (size_t)pr * (a.I / 2) + t2, pack_bf16x2(h0, h1), tag);
    }
  }
};

// Whether a variant runs SplitK, and its item counts with 256 workgroups
// (the kernel checks the grid size at run time).
template <class A, int TB, int WTR, int WTS, bool DYN = std::is_base_of<DynShape, A>::value>
struct SplitKPlan {
  static constexpr bool on = false;
  static constexpr int KS = 1, KR = 1;
};
template <class A, int TB, int WTR, int WTS>
struct SplitKPlan<A, TB, WTR, WTS, false> {
  static constexpr int KS = A::S * (A::I / 2) / 256, KR = A::k * (A::I / 2) / 256;
  static constexpr bool on = TB == 1 && WTR == WT_NVFP4 && WTS == WT_NVFP4 && A::g13.ns == 1 && A::g13.rpw == 1 &&
                             A::g13.lpr == 64 && A::S >= 1 && (A::S * (A::I / 2)) % 256 == 0 &&
                             (A::k * (A::I / 2)) % 256 == 0 && KS + KR <= 8;
};

// This lane's column (element offset) of the activation row for the gate/up
// tiles, and the chunks of the first XR tokens from the x region of shared memory.
template <class A>
__device__ __forceinline__ int x_col(const A& a, const LaneGeo& L) {
  return ((a.g13.ns == 1) ? L.jc : (wave_id() % a.g13.ns) * a.g13.cw + L.jc) * 32;
}
template <int XR, class A>
__device__ __forceinline__ void load_xr(const A& a, int col, const uint16_t* xs, uint32_t (&xr)[XR][16]) {
#pragma unroll
  for (int b = 0; b < XR; ++b) lds_chunk(xs + (size_t)min(b, a.B - 1) * a.H + col, xr[b]);
}

// ---------------------------------------------------------------------------
// routing (every workgroup, from the gathered logits)
// ---------------------------------------------------------------------------

// Routing weights and shared coefficients of the TPW tokens (wave + t NW),
// into shared memory, with the token masks of the selected experts.
template <int TPW, class A>
__device__ __forceinline__ void route_weights(const A& a, Smem& s, const float* lg, int lane,
                                              const int (&my_e)[TPW], const float (&my_l)[TPW],
                                              const float (&my_sg)[TPW], const float (&sg_sum)[TPW]) {
  const int wave = wave_id();
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int b = wave + t * NW;
    if (b >= a.B) continue;
    float wv, shc;
    token_weights(a, lg + (size_t)b * a.Er, lane, my_l[t], my_sg[t], sg_sum[t], wv, shc);
    if (lane < a.S) s.shc[b][lane] = shc;
    if (lane < a.k) {
      s.sel[b][lane] = my_e[t];
      s.selw[b][lane] = wv;
      atomicOr(&s.emask[my_e[t]], 1u << b);
    }
  }
}

// Wave 0: the distinct selected experts, numbered by first appearance in
// (token, rank) order, with their token masks, expert bases and W13 tensor
// scales; the rank of every (slot, token); the combine weight of every pair.
// eb/er: this lane's two (token, rank) entries (lane and lane + 64).
template <int WTR, int WTS, class A>
__device__ __forceinline__ void number_slots(const A& a, Smem& s, int lane, const int (&eb)[2],
                                             const int (&er)[2]) {
  const int nk = a.B * a.k;
  int nd = 0;
  int eh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    const bool valid = i < nk;
    const int b = eb[h], r = er[h];
    const int e = valid ? s.sel[b][r] : 0;
    const unsigned mk = valid ? s.emask[e] : 0u;
    const bool rep = valid && b == __builtin_ctz(mk | 0x80000000u);
    const unsigned long long bal = __ballot(rep);
    const int slot = nd + __popcll(bal & ((1ull << lane) - 1ull));
    if (rep) {
      s.ids[slot] = e;
      s.dmask[slot] = mk;
      s.slotmap[e] = slot;
      s.xg[slot] = (WTR == WT_NVFP4) ? s.tsr[e][0] : 1.0f;
      s.pr[slot][0] = 0u;
      s.pr[slot][1] = 0u;
    }
    nd += __popcll(bal);
    eh[h] = e;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    if (i < nk) {
      atomicOr(&s.pr[s.slotmap[eh[h]]][eb[h] >> 2], (uint32_t)er[h] << (8 * (eb[h] & 3)));
      const float g2 = (WTR == WT_NVFP4) ? s.tsr[eh[h]][1] : 1.0f;
      s.pw[i] = s.selw[eb[h]][er[h]] * g2;
    }
  }
  for (int i = lane; i < a.B * a.S; i += 64) {
    const int sh = i / a.B, b = i - sh * a.B;
    const float g2 = (WTS == WT_NVFP4) ? s.tss[sh][1] : 1.0f;
    s.pw[nk + i] = s.shc[b][sh] * g2;
  }
  if (lane == 0) s.nd = nd;
}

template <int MK, int TPW, int TB, int WTR, int WTS, class A>
__device__ __forceinline__ void route(const A& a, Smem& s, const float* lg, const int (&eb)[2],
                                      const int (&er)[2]) {
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  if constexpr (TB == 1) {
    // One token: its k selections are the distinct experts, slot r = rank r,
    // so wave 0 fills the tables from its registers.
    if (wave == 0) {
      int my_e[1];
      float my_l[1], my_sg[1], sg_sum[1];
      topk<MK, 1>(a, lg, lane, my_e, my_l, my_sg, sg_sum);
      float wv, shc;
      token_weights(a, lg, lane, my_l[0], my_sg[0], sg_sum[0], wv, shc);
      if (lane < a.k) {
        const int e = my_e[0];
        s.ids[lane] = e;
        s.dmask[lane] = 1u;
        s.xg[lane] = (WTR == WT_NVFP4) ? s.tsr[e][0] : 1.0f;
        s.pr[lane][0] = (uint32_t)lane;
        s.pr[lane][1] = 0u;
        s.pw[lane] = wv * ((WTR == WT_NVFP4) ? s.tsr[e][1] : 1.0f);
        if (blockIdx.x == 0) {
          a.topk_ids[lane] = e;
          a.topk_w[lane] = wv;
        }
      }
      if (lane < a.S) {
        s.pw[a.k + lane] = shc * ((WTS == WT_NVFP4) ? s.tss[lane][1] : 1.0f);
        if (blockIdx.x == 0) a.shared_c[lane] = shc;
      }
      if (lane == 0) s.nd = a.k;
    }
    __syncthreads();
    return;
  }
  if (wave < a.B) {
    int my_e[TPW];
    float my_l[TPW], my_sg[TPW], sg_sum[TPW];
    topk<MK, TPW>(a, lg, lane, my_e, my_l, my_sg, sg_sum);
    route_weights<TPW>(a, s, lg, lane, my_e, my_l, my_sg, sg_sum);
  }
  __syncthreads();
  if (wave == 0) number_slots<WTR, WTS>(a, s, lane, eb, er);
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.B * a.k; i += NT) {
      const int b = i / a.k, r = i - b * a.k;
      a.topk_ids[i] = s.sel[b][r];
      a.topk_w[i] = s.selw[b][r];
    }
    for (int i = tid; i < a.B * a.S; i += NT) a.shared_c[i] = s.shc[i / a.S][i % a.S];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// down GEMV + combine
// ---------------------------------------------------------------------------

// The workgroup owns output steps [t_lo, t_lo + spg) of W2.  Experts in
// order: shared 0..S-1, then routed slots 0..nd-1.  If spg >= NW, wave w
// takes steps w, w + NW, ... with every expert; otherwise nsub = NW / spg
// waves share a step, wave w taking experts w / spg, w / spg + nsub, ...
// (at batch 4-8: every shared expert for its own tokens, see set_experts)
// Per step the lane sums weight x partial dot over its experts in
// registers; one lane reduction per (step, token) follows.  P tiles are
// loading at a time.
template <int TB, int WTR, int WTS, int P>
struct Down {
  Tile<WTR> br[P];
  Tile<WTS> bs[(WTR == WTS) ? 1 : P];   // same types: shared tiles use br
  int t_lo, spg, nsub, lg_nsub, sub, nex, nj, ntiles;
  int nsh;                             // shared experts every sub takes (batch 4-8 with nsub > 1), else 0
  unsigned smask;                      // tokens of the shared tiles this wave computes
  int cj, cx, nloaded;                 // next tile to load: step index, expert index (mine)
  int qj[P], qx[P];
  LaneGeo L;

  // Everything that does not depend on the routing.
  template <class A>
  __device__ __forceinline__ void init(const A& a, const LaneGeo& l2) {
    const int wave = wave_id();
    const uint32_t w = blockIdx.x;
    L = l2;
    t_lo = (int)(((uint32_t)a.g2.nsteps * w) >> a.log2G);
    spg = (int)(((uint32_t)a.g2.nsteps * (w + 1)) >> a.log2G) - t_lo;
    if (spg >= NW || spg == 0) {
      nsub = 1;
      sub = 0;
      nj = (spg > wave) ? (spg - wave + NW - 1) / NW : 0;
      cj = wave;
    } else {
      nsub = (spg == 1) ? 4 : (spg == 2) ? 2 : 1;
      // at batch 1-2 the first waves own the most gate/up items and load
      // their down tiles last: sub-group 0, which takes the most experts,
      // goes to the last waves (partials still combine in sub order)
      const int wv = (TB <= 2) ? NW - 1 - wave : wave;
      sub = wv / spg;
      nj = (sub < nsub) ? 1 : 0;
      cj = wv % spg;
    }
    lg_nsub = (nsub == 4) ? 2 : (nsub == 2) ? 1 : 0;
  }
  // S shared experts, nd selected ones.  Experts in order: shared 0..S-1,
  // then routed slots.  At batch 4-8 a shared tile carries every token
  // (several routed tiles' work), so when waves share a step every sub takes
  // every shared expert, for its tokens b = sub (mod nsub) only, and the
  // routed slots alternate; otherwise the whole list alternates.
  __device__ __forceinline__ void set_experts(int S, int nd) {
    nsh = (TB >= 4 && nsub > 1) ? S : 0;
    if (nsh > 0) {
      nex = nsh + ((nd > sub) ? (nd - sub + nsub - 1) >> lg_nsub : 0);
      smask = ((nsub == 4) ? 0x11111111u : 0x55555555u) << sub;
    } else {
      const int nexp = S + nd;
      nex = (nexp > sub) ? (nexp - sub + nsub - 1) >> lg_nsub : 0;
      smask = ~0u;
    }
    ntiles = nj * nex;
    cx = 0;
    nloaded = 0;
  }
  __device__ __forceinline__ int ex_of(int xi) const {
    return (xi < nsh) ? xi : nsh + sub + ((xi - nsh) << lg_nsub);
  }
  // Loads the next tile of this wave, or a dummy once they are all loaded.
  template <class A>
  __device__ __forceinline__ void load_next(const A& a, const SlotTab& tb, int p) {
    const bool dm = nloaded >= ntiles;
    const int ex = dm ? 0 : ex_of(cx), t = dm ? t_lo : t_lo + cj;
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.x);
    if (ex < a.S) {
      const uint8_t* c = a.s_codes + expert_off<A>(ex, a.s_code_stride) + a.s_w13_code;
      const uint8_t* sc = (WTS == WT_NVFP4) ? a.s_scales + expert_off<A>(ex, a.s_scale_stride) + a.s_w13_scale : dummy;
      if constexpr (WTR == WTS) tile_load<WTR>(br[p], c, sc, L, 0, t, dm, dummy);
      else tile_load<WTS>(bs[p], c, sc, L, 0, t, dm, dummy);
    } else {
      const int e = tb.expert(min(ex - a.S, kMaxD - 1), a.E);
      const uint8_t* c = a.r_codes + expert_off<A>(e, a.r_code_stride) + a.r_w13_code;
      const uint8_t* sc = (WTR == WT_NVFP4) ? a.r_scales + expert_off<A>(e, a.r_scale_stride) + a.r_w13_scale : dummy;
      tile_load<WTR>(br[p], c, sc, L, 0, t, dm, dummy);
    }
    qj[p] = cj;
    qx[p] = cx;
    if (!dm) {
      ++nloaded;
      if (++cx == nex) {
        cx = 0;
        cj += (nsub == 1) ? NW : 0;
      }
    }
  }
  template <class A>
  __device__ __forceinline__ void prime(const A& a, const SlotTab& tb) {
#pragma unroll
    for (int p = 0; p < P; ++p) load_next(a, tb, p);
  }
  // hs: activations [pairs][I] bf16 (shared memory).  Results: nsub == 1 ->
  // out directly; else partial sums into red2 [nsub][TB][spg * rpw].
  // Tile in buffer p (live: a real tile of this wave); acc: this lane's row
  // sums of the current step, per token.  RELOAD: refill the buffer with the
  // wave's next tile (a dummy past the end) once it is read.
  template <bool RELOAD, class A>
  __device__ __forceinline__ void step(const A& a, const SlotTab& tb, const uint16_t* hs, float* red2,
                                       float (&acc)[TB], int p, bool live, bool lead) {
    const int rpw = a.g2.rpw, lpr = a.g2.lpr;
    const int j = qj[p], xi = qx[p], ex = ex_of(xi), t = t_lo + j;
    if (live) {
      const bool sh = ex < a.S;
      const int slot = min(ex - a.S, kMaxD - 1);
      const unsigned mask = sh ? ((1u << a.B) - 1u) & smask : tb.tokens(slot);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if ((mask >> b) & 1u) {
          const int pr = sh ? a.B * a.k + ex * a.B + b : b * a.k + tb.rank(slot, b);
          uint32_t hv[16];
          lds_chunk(hs + (size_t)pr * a.I + L.jc * 32, hv);
          float v;
          if constexpr (WTR == WTS) v = tile_dot<WTR>(br[p], t, hv);
          else v = sh ? tile_dot<WTS>(bs[p], t, hv) : tile_dot<WTR>(br[p], t, hv);
          acc[b] = fmaf(L.active ? v : 0.f, tb.weight(pr), acc[b]);
        }
      }
    }
    // The refill path keeps its reload below the reads (see GateUp::step) and
    // tiles apart.  Without refills every tile's data have landed by now (the
    // activation polls waited for them), so the compiler may overlap one
    // tile's activation reads from shared memory with another's arithmetic.
    if constexpr (RELOAD) {
      __asm__ volatile("" ::: "memory");
      load_next(a, tb, p);   // unconditional, see GateUp::step
    }
    if (live && xi == nex - 1) {
      // step complete: reduce each token's row sums over the row's lanes
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if (b < a.B) {
          const float v = group_sum(acc[b], lpr);
          if (lead) {
            const int rl = j * rpw + L.ri;
            if (nsub == 1) {
              const int row = t * rpw + L.ri;
              float o = v;
              if (a.residual) o += bf16lo(a.x[(size_t)b * a.H + row]);
              a.out[(size_t)b * a.H + row] = (uint16_t)f2bf(o);
            } else {
              red2[(sub * TB + b) * (spg * rpw) + rl] = v;
            }
          }
        }
        acc[b] = 0.f;
      }
    }
  }
  // hs: activations [pairs][I] bf16 (shared memory).  Results: nsub == 1 ->
  // out directly; else partial sums into red2 [nsub][TB][spg * rpw].
  template <class A>
  __device__ __forceinline__ void run(const A& a, const SlotTab& tb, const uint16_t* hs, float* red2) {
    if constexpr (TB == 1 && WTR == WTS && kSkipRefills<TB, WTR>) {
      if (nj <= 1 && ntiles <= P) {
        run1(a, tb, hs, red2);
        return;
      }
    }
    float acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = 0.f;
    const bool lead = L.jj == a.g2.lpr - 1;
    if (kSkipRefills<TB, WTR> && kSkipRefills<TB, WTS> && ntiles <= P) {   // see GateUp::run
#pragma unroll
      for (int p = 0; p < P; ++p) step<false>(a, tb, hs, red2, acc, p, p < ntiles, lead);
    } else {
      for (int base = 0; base < ntiles; base += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) step<true>(a, tb, hs, red2, acc, p, base + p < ntiles, lead);
      }
    }
  }
  // Batch 1, every tile of the wave loaded and of one step: the tiles run
  // without branches (a dead tile's term is dropped by a select, its
  // activation row clamped to a real pair), so one tile's shared-memory
  // reads overlap another's arithmetic; the same fused multiply-adds in the
  // same order as step(), and one reduction at the end.
  template <class A>
  __device__ __forceinline__ void run1(const A& a, const SlotTab& tb, const uint16_t* hs, float* red2) {
    const int rpw = a.g2.rpw, lpr = a.g2.lpr;
    const int npairs = a.k + a.S;
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bool live = p < ntiles;
      const int ex = ex_of(qx[p]);
      const bool sh = ex < a.S;
      const int slot = min(max(ex - a.S, 0), kMaxD - 1);
      const int pr = min(sh ? a.k + ex : tb.rank(slot, 0), npairs - 1);
      uint32_t hv[16];
      lds_chunk(hs + (size_t)pr * a.I + L.jc * 32, hv);
      const float v = tile_dot<WTR>(br[p], t_lo + qj[p], hv);
      const float w = tb.weight(pr);
      acc = live ? fmaf(L.active ? v : 0.f, w, acc) : acc;
    }
    if (ntiles > 0) {
      const float v = group_sum(acc, lpr);
      if (L.jj == lpr - 1) {
        const int j = qj[0], t = t_lo + j;
        if (nsub == 1) {
          const int row = t * rpw + L.ri;
          float o = v;
          if (a.residual) o += bf16lo(a.x[row]);
          a.out[row] = (uint16_t)f2bf(o);
        } else {
          red2[sub * (spg * rpw) + j * rpw + L.ri] = v;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Items (gate/up) and tiles (down) in flight per wave.
template <int TB, int WT> constexpr int gu_depth() { return WT == WT_NVFP4 ? (TB <= 2 ? 2 : 4) : 1; }
template <int TB, int WTR, int WTS> constexpr int down_depth() {
  return (WTR == WT_NVFP4 && WTS == WT_NVFP4) ? (TB == 1 ? 4 : (TB == 2 ? 6 : 8)) : 3;
}

// Logit words each thread gathers: exact for a fixed shape, else enough for
// up to 512 router rows.
template <class A, int TB, bool DYN = std::is_base_of<DynShape, A>::value>
struct LogitWords { static constexpr int value = 2 * TB; };
template <class A, int TB>
struct LogitWords<A, TB, false> { static constexpr int value = (A::Er * TB + NT - 1) / NT; };

// Routed tensor-scale words (W13, W2 per expert) each thread loads into the
// shared-memory table: exact for a fixed shape, else enough for the largest
// routed expert count.
template <class A, bool DYN = std::is_base_of<DynShape, A>::value>
struct TsWords { static constexpr int value = (2 * MOE_MAX_ROUTED + NT - 1) / NT; };
template <class A>
struct TsWords<A, false> { static constexpr int value = (2 * A::E + NT - 1) / NT; };

// QX: 16-byte units of a router row per thread (H <= QX * NT * 8); the host
// picks the smallest that fits, so every one of them is a real load.
template <int TB, int QX, int WTR, int WTS, class A>
__global__ __launch_bounds__(NT) void k_fused_layer(A a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ Smem s;
  __shared__ float lg[TB * MOE_MAX_ROUTED];

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int w = blockIdx.x, G = a.G;
  uint16_t* act = reinterpret_cast<uint16_t*>(dyn);                  // x (phases 1-2), h (phase 3)
  float* part = reinterpret_cast<float*>(dyn + (size_t)TB * a.H * 2); // gate/up partials (ns > 1)
  float* red2 = reinterpret_cast<float*>(dyn + a.lds_act);            // down partial sums (nsub > 1)

  // ---- loads that need nothing: call counter, router rows, x, gamma, bias, tensor scales
  const uint32_t epoch = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int U = a.H / 8;                       // 16-byte units per row
  const int nrr = (w + G < a.Er) ? 2 : 1;      // router rows of this workgroup
  uint4 rw[2][QX], xv[TB][QX], gv[QX];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int u = min(tid + q * NT, U - 1);
      const int row = (rr < nrr) ? w + rr * G : w;   // second row: a duplicate when absent
      rw[rr][q] = ld16nt(a.router_w + (size_t)row * a.H + u * 8);
    }
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < QX; ++q) xv[b][q] = ld16(a.x + (size_t)min(b, a.B - 1) * a.H + min(tid + q * NT, U - 1) * 8);
  {
    const uint16_t* gsrc = a.prenorm ? a.gamma : a.x;
#pragma unroll
    for (int q = 0; q < QX; ++q) gv[q] = ld16(gsrc + (size_t)min(tid + q * NT, U - 1) * 8);
  }
  float biasv[2];
  {
    const float* bsrc = a.bias != nullptr ? a.bias : reinterpret_cast<const float*>(a.x);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) biasv[rr] = bsrc[a.bias != nullptr ? min(w + rr * G, a.E - 1) : 0];
  }
  // tensor scales for the shared-memory tables (loaded unconditionally from
  // clamped addresses so that no load depends on a condition; a layer
  // without shared experts has no shared buffer: x stands in)
  const int nts = (WTR == WT_NVFP4 && a.r_tscale != nullptr) ? 2 * a.E : 0;
  const float* tsr_src = (WTR == WT_NVFP4 && a.r_tscale != nullptr) ? a.r_tscale : reinterpret_cast<const float*>(a.x);
  const float* tss_src = (WTS == WT_NVFP4 && a.S > 0 && a.s_tscale != nullptr)
                             ? a.s_tscale : reinterpret_cast<const float*>(a.x);
  constexpr int NTS = TsWords<A>::value;
  float tsv[NTS];
#pragma unroll
  for (int h = 0; h < NTS; ++h) tsv[h] = tsr_src[min(tid + h * NT, max(nts, 1) - 1)];
  const float tss = tss_src[min(tid, max(2 * a.S, 1) - 1)];

  // ---- set-up that needs no data (overlaps the loads above) -------------------
  const LaneGeo L13 = lane_geo(a.g13, lane), L2 = lane_geo(a.g2, lane);
  int eb[2], er[2];   // (token, rank) of this lane's routing entries lane, lane + 64
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    eb[h] = min(i / a.k, MOE_MAX_BATCH - 1);
    er[h] = i - (i / a.k) * a.k;
  }
  Down<TB, WTR, WTS, down_depth<TB, WTR, WTS>()> down;
  down.init(a, L2);
  const int gs2 = a.I / a.g13.rpw / 2;
  SlotTab tab = {};   // filled after routing
  // the shared experts' tiles need no routing: they load from the start
  GateUp<TB, WTS, 1> gus;   // one item in flight: its tiles stay in registers until after routing
  gus.init(a, L13, 1);
  gus.set_items(a, a.S * gs2);
  using SKP = SplitKPlan<A, TB, WTR, WTS>;
  const bool sk = SKP::on && a.log2G == 8;   // batch-1 split-K gate/up (uniform)
  SplitK<SKP::KS, SKP::KR> skg;
  if constexpr (SKP::on) skg.init(a, L13);

  // ---- pre-norm: xhat = bf16(x / rms(x) * gamma) -----------------------------
  if (a.prenorm) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < QX; ++q) {
        if (tid + q * NT < U) {
          const uint32_t d[4] = {xv[b][q].x, xv[b][q].y, xv[b][q].z, xv[b][q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = bf16lo(d[i]), hi = bf16hi(d[i]);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
          }
        }
      }
      ss = wave_sum(ss);
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
        uint4& v = xv[b][q];
        v.x = norm_pair(v.x, gv[q].x, rn);
        v.y = norm_pair(v.y, gv[q].y, rn);
        v.z = norm_pair(v.z, gv[q].z, rn);
        v.w = norm_pair(v.w, gv[q].w, rn);
      }
    }
  }
  // x (or xhat) into shared memory for the gate/up tiles
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < QX; ++q) {
      const int u = tid + q * NT;
      if (u < U && b < a.B) *reinterpret_cast<uint4*>(act + (size_t)b * a.H + u * 8) = xv[b][q];
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
            if (tid + q * NT < U) {
              v = dot2(rw[rr][q].x, xv[b][q].x, v);
              v = dot2(rw[rr][q].y, xv[b][q].y, v);
              v = dot2(rw[rr][q].z, xv[b][q].z, v);
              v = dot2(rw[rr][q].w, xv[b][q].w, v);
            }
          }
        }
        racc[rr][b] = (rr < nrr) ? group_sum(v, 64) : 0.f;
      }
    if (lane == 63)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int b = 0; b < TB; ++b) s.red[wave][rr][b] = racc[rr][b];
  }
#pragma unroll
  for (int h = 0; h < NTS; ++h) {
    const int i = tid + h * NT;
    if (i < nts) (&s.tsr[0][0])[i] = tsv[h];
  }
  if (WTS == WT_NVFP4 && tid < 2 * a.S) (&s.tss[0][0])[tid] = tss;
  for (int e = tid; e < a.E; e += NT) s.emask[e] = 0u;
  if (tid == 0) s.tag = (epoch + 1u == 0u) ? 1u : epoch + 1u;   // tag 0 marks never-written words
  __syncthreads();
  const uint32_t tag = s.tag;
  if (tid < nrr * a.B) {
    const int rr = tid / a.B, b = tid % a.B;
    const int row = w + rr * G;
    float v = 0.f;
    for (int q = 0; q < NW; ++q) v += s.red[q][rr][b];
    if (a.bias != nullptr && row < a.E) v += (rr == 0) ? biasv[0] : biasv[1];
    publish(a.xlog + (size_t)row * kLogitLine + b, __float_as_uint(v), tag);
  }

  // ---- activation chunks; every workgroup gathers all logits ---------------------
  constexpr int XR = (TB <= 2) ? TB : 1;   // activation chunks held in registers
  const int xcol = x_col(a, L13);
  uint32_t xr[XR][16];
  load_xr<XR>(a, xcol, act, xr);
  auto laddr = [&](int i) { return a.xlog + (size_t)(i / a.B) * kLogitLine + (i % a.B); };
  Gather<LogitWords<A, TB>::value> lgat;
  // The first poll waits ~0.2 us (s_sleep 8 = 512 cycles): every workgroup has
  // just published, and polls sent earlier find nothing new yet while they
  // crowd the memory side the other workgroups' logits are on their way to
  // (measured: 10.6 -> 9.7 us per step at batch 1; 0.1 or 0.3 us do less).
  __builtin_amdgcn_s_sleep(8);
  lgat.issue(0, a.Er * a.B, laddr);
  // every wait ends by this time (measured from here, not from the start:
  // the bound is not needed before the first wait)
  const u64 deadline = clock100() + a.wait_ticks;
  lgat.finish(tag, deadline, a.err, kErrLogitWait, laddr,
              [&](int i, uint32_t v) { lg[(i % a.B) * a.Er + i / a.B] = __uint_as_float(v); });
  __syncthreads();
  if (w == 0 && tid == 0) __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- routing ---------------------------------------------------------------------
  // At batch 1 routing runs in wave 0 alone; meanwhile the other waves issue
  // their tiles of the shared item (a wave without one issues nothing).  Wave
  // 0 issues its own after routing: loads in flight in wave 0 delay its
  // routing code (about 0.2 us per step).  Not before the logit gather: the
  // polls wait, in order, for every load of their wave.
  if constexpr (TB == 1) {
    if (SKP::on && sk) { if (wave != 0) skg.load_shared(a, L13); }
    else gus.prime(a, tab);
  }
  constexpr int TPW = (TB > NW) ? 2 : 1;
  if (a.E <= 64) route<1, TPW, TB, WTR, WTS>(a, s, lg, eb, er);
  else if (a.E <= 256) route<4, TPW, TB, WTR, WTS>(a, s, lg, eb, er);
  else route<8, TPW, TB, WTR, WTS>(a, s, lg, eb, er);

  // ---- phase 2: shared and selected experts' gate/up --------------------------------
  // The shared experts' tiles first (at batch 1 they are already loading).
  if constexpr (TB != 1) gus.prime(a, tab);
  tab.load(s, lane);
  const int nd = s.nd;
  down.set_experts(a.S, nd);
  if (SKP::on && sk) {
    if constexpr (SKP::on) {
      if (wave == 0) skg.load_shared(a, L13);
      skg.load_routed(a, tab, L13);
      skg.run(a, s, act, tag);
    }
  } else {
    GateUp<TB, WTR, gu_depth<TB, WTR>()> gur;
    gur.init(a, L13, 0);
    gur.set_items(a, nd * gs2);
    gur.prime(a, tab);
    // At batch 4-8 gate/up is long enough to hide the down weights' loads too.
    if constexpr (TB > 2) down.prime(a, tab);
    // the shared experts' tiles are on their way: their gate/up runs while the
    // selected experts' first tiles are in flight
    gus.run(a, s, tab, xr, act, xcol, part, tag);
    gur.run(a, s, tab, xr, act, xcol, part, tag);
  }
  // At batch 1-2 the down weights load after gate/up, while the activations
  // are exchanged: issued with the gate/up burst they arrived late, and the
  // exchange's polls wait, in order, for every load of their wave.
  if constexpr (TB <= 2) down.prime(a, tab);

  // ---- phase 3: gather activations, down GEMV + combine ---------------------------------
  // a wave with no expert of its subset writes no partial sums: start from zero
  if (down.nsub > 1)
    for (int i = tid; i < a.lds_acc / (int)sizeof(float); i += NT) red2[i] = 0.f;
  __syncthreads();   // every wave is done with x before h overwrites it
  const int I2 = a.I / 2;
  const int npairs = a.B * (a.k + a.S);
  {
    const int rpw = a.g13.rpw;
    gather_all<(TB >= 4 ? 32 : TB * 8)>(
        npairs * I2, tag, deadline, a.err, kErrActWait, [&](int i) { return a.xh + i; },
        [&](int i, uint32_t v) {
          const int pr = i / I2, q = i - pr * I2;
          if (rpw == 1) {
            *reinterpret_cast<uint32_t*>(act + (size_t)pr * a.I + 2 * q) = v;
          } else {
            const int t2 = q / rpw, ri = q - t2 * rpw;
            const int r0 = 2 * t2 * rpw + ri;
            act[(size_t)pr * a.I + r0] = (uint16_t)(v & 0xffffu);
            act[(size_t)pr * a.I + r0 + rpw] = (uint16_t)(v >> 16);
          }
        });
  }
  __syncthreads();
  down.run(a, tab, act, red2);
  if (down.nsub > 1) {
    __syncthreads();
    const int rows = down.spg * a.g2.rpw;
    const int nsub = down.nsub;
    for (int i = tid; i < a.B * rows; i += NT) {
      const int b = i / rows, r = i - b * rows;
      float v = 0.f;
      for (int u = 0; u < nsub; ++u) v += red2[(u * TB + b) * rows + r];
      const int row = down.t_lo * a.g2.rpw + r;
      if (a.residual) v += bf16lo(a.x[(size_t)b * a.H + row]);
      a.out[(size_t)b * a.H + row] = (uint16_t)f2bf(v);
    }
  }
}

// Test hook: the SiLU*up activations of the last call, from the tagged words.
// h_r [B][k][I] in selection order, h_s [B][S][I].
__global__ __launch_bounds__(NT) void k_fused_debug_h(FusedArgs a, uint16_t* h_r, uint16_t* h_s) {
  const int row = blockIdx.x;   // 0 .. B*k + B*S - 1
  int pr;
  uint16_t* dst;
  if (row < a.B * a.k) {
    pr = row;
    dst = h_r ? h_r + (size_t)row * a.I : nullptr;
  } else {
    const int p = row - a.B * a.k, b = p / a.S, sh = p % a.S;
    pr = a.B * a.k + sh * a.B + b;
    dst = h_s ? h_s + (size_t)p * a.I : nullptr;
  }
  if (dst == nullptr) return;
  const int I2 = a.I / 2, rpw = a.g13.rpw;
  for (int q = threadIdx.x; q < I2; q += NT) {
    const u64 v = peek(a.xh + (size_t)pr * I2 + q);
    const int t2 = q / rpw, ri = q % rpw, r0 = 2 * t2 * rpw + ri;
    dst[r0] = (uint16_t)(v & 0xffffu);
    dst[r0 + rpw] = (uint16_t)((v >> 16) & 0xffffu);
  }
}

// Workspace of moe_decode_layer_static: the exchange words, call counter,
// error word and routing readback of handle-less calls, one copy per device
// for the life of the process.  Zero at load (tag 0 marks never-written
// words).  Host code never uses this name as an address: it reads the
// per-device address once with hipGetSymbolAddress (static_scratch below).
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

}  // namespace

void* static_scratch(int device) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (addr[device] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[device] = ptr;
  }
  return addr[device];
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

// One compiled variant of the layer kernel: layer shape (fixed or read from
// the arguments), batch bucket, router units per thread, weight types.
template <class SH, int TB, int QX, int WTR, int WTS>
struct Variant {
  static constexpr int BF = (TB <= 2) ? TB : 0;   // buckets 1 and 2 hold exactly TB tokens
  using Args = KArgs<SH, BF>;
  static const void* fn() { return reinterpret_cast<const void*>(&k_fused_layer<TB, QX, WTR, WTS, Args>); }
  static int launch(const FusedArgs& f, hipStream_t st) {
    Args k = kargs_of<SH, BF>(f);
    void* args[] = {&k};
    return (int)hipLaunchKernel(fn(), dim3(f.G), dim3(NT), args, (size_t)fused_lds_bytes(f), st);
  }
};
template <class T> struct Tag { using type = T; };
constexpr int kNoVariant = (int)hipErrorInvalidValue;

template <class SH, int TB, int QX, class F>
static int by_wtype(int rwt, int swt, F&& f) {
  if (rwt == WT_NVFP4 && swt == WT_NVFP4) return f(Tag<Variant<SH, TB, QX, WT_NVFP4, WT_NVFP4>>{});
  if (rwt == WT_BF16 && swt == WT_BF16) return f(Tag<Variant<SH, TB, QX, WT_BF16, WT_BF16>>{});
  if constexpr (std::is_same<SH, DynShape>::value)
    if (rwt == WT_NVFP4 && swt == WT_BF16) return f(Tag<Variant<SH, TB, QX, WT_NVFP4, WT_BF16>>{});
  return kNoVariant;
}

// Calls f(Tag<Variant>) for the variant of (shape, bucket, qx, weight types).
// qx 1 covers H <= 2048, qx 4 H <= 8192 (batch buckets 1, 2, 4 only); the
// Flint shape has its own variants.
template <class F>
static int with_variant(int shape, int tb, int qx, int rwt, int swt, F&& f) {
  if (shape == 1) {
    if (qx != 1) return kNoVariant;
    switch (tb) {
      case 1: return by_wtype<FlintShape, 1, 1>(rwt, swt, f);
      case 2: return by_wtype<FlintShape, 2, 1>(rwt, swt, f);
      case 4: return by_wtype<FlintShape, 4, 1>(rwt, swt, f);
      case 8: return by_wtype<FlintShape, 8, 1>(rwt, swt, f);
      default: return kNoVariant;
    }
  }
  if (qx == 1) {
    switch (tb) {
      case 1: return by_wtype<DynShape, 1, 1>(rwt, swt, f);
      case 2: return by_wtype<DynShape, 2, 1>(rwt, swt, f);
      case 4: return by_wtype<DynShape, 4, 1>(rwt, swt, f);
      case 8: return by_wtype<DynShape, 8, 1>(rwt, swt, f);
      default: return kNoVariant;
    }
  }
  if (qx == 4) {
    switch (tb) {
      case 1: return by_wtype<DynShape, 1, 4>(rwt, swt, f);
      case 2: return by_wtype<DynShape, 2, 4>(rwt, swt, f);
      case 4: return by_wtype<DynShape, 4, 4>(rwt, swt, f);
      default: return kNoVariant;
    }
  }
  return kNoVariant;
}

bool fused_variant_exists(int shape, int tb, int qx, int rwt, int swt) {
  return with_variant(shape, tb, qx, rwt, swt, [](auto) -> int { return 0; }) == 0;
}

int fused_qx(int hidden) { return hidden / 8 <= NT ? 1 : (hidden / 8 <= 4 * NT ? 4 : 0); }

int fused_occupancy(int shape, int tb, int qx, int rwt, int swt, int lds_bytes, int* blocks_per_cu) {
  return with_variant(shape, tb, qx, rwt, swt, [&](auto t) -> int {
    const void* f = decltype(t)::type::fn();
    if (lds_bytes > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
      if (e != hipSuccess) return (int)e;
    }
    return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, NT, lds_bytes);
  });
}

int launch_fused(const FusedArgs& a, int tb, int rwt, int swt, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so it is not reported as ours
  const int shape = fixed_shape_of(a.H, a.I, a.E, a.k, a.S, a.Er, rwt, swt);
  // a fixed shape addresses experts with 32-bit offsets
  if (shape != 0 && ((size_t)a.E * a.r_code_stride >= (1ull << 32) || (size_t)a.E * a.r_scale_stride >= (1ull << 32)))
    return kNoVariant;
  return with_variant(shape, tb, fused_qx(a.H), rwt, swt,
                      [&](auto t) -> int { return decltype(t)::type::launch(a, st); });
}

int launch_fused_debug_h(const FusedArgs& a, uint16_t* h_r, uint16_t* h_s, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int n = a.B * a.k + a.B * a.S;
  hipLaunchKernelGGL(k_fused_debug_h, dim3(n), dim3(NT), 0, st, a, h_r, h_s);
  return (int)hipGetLastError();
}

}  // namespace moe
