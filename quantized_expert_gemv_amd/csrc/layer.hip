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

// The wavefront's index in its workgroup, as a uniform (scalar) value: the
// compiler cannot tell that threadIdx.x / 64 is the same for a whole wave,
// and per-wave loop bounds derived from it would otherwise become divergent
// loops whose register copies wait for every load in flight.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

__device__ __forceinline__ void publish(u64* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 peek(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls a set of tagged words until their tags equal `tag`.  Each thread
// owns words i = tid + NT*q, q < NB.  issue() sends the first loads (they can
// fly while the thread does other work); finish() waits for the stragglers,
// then hands (i, value) to sink.  Past the deadline the error bit is set and
// the words are taken as they are.
template <int NB>
struct Gather {
  u64 v[NB];
  unsigned pend;
  int base, n;

  template <typename Addr>
  __device__ __forceinline__ void issue(int base_, int n_, Addr&& addr) {
    base = base_;
    n = n_;
    pend = 0u;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = base + q * NT + (int)threadIdx.x;
      v[q] = peek(addr(i < n ? i : 0));
      if (i < n) pend |= 1u << q;
    }
  }
  template <typename Addr, typename Sink>
  __device__ __forceinline__ void finish(uint32_t tag, u64 deadline, unsigned* err, unsigned bit, Addr&& addr,
                                         Sink&& sink) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (((pend >> q) & 1u) && (uint32_t)(v[q] >> 32) == tag) pend &= ~(1u << q);
    while (pend != 0u) {
      if (clock100() > deadline) {
        __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((pend >> q) & 1u) v[q] = peek(addr(base + q * NT + (int)threadIdx.x));
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (((pend >> q) & 1u) && (uint32_t)(v[q] >> 32) == tag) pend &= ~(1u << q);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = base + q * NT + (int)threadIdx.x;
      if (i < n) sink(i, (uint32_t)v[q]);
    }
  }
};

// All n words, NB per thread per round.
template <int NB, typename Addr, typename Sink>
__device__ __forceinline__ void gather_all(int n, uint32_t tag, u64 deadline, unsigned* err, unsigned bit, Addr&& addr,
                                           Sink&& sink) {
  for (int base = 0; base < n; base += NB * NT) {
    Gather<NB> g;
    g.issue(base, n, addr);
    g.finish(tag, deadline, err, bit, addr, sink);
  }
}

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
  int ids[kMaxD];                             // distinct selected experts (slot order)
  unsigned dmask[kMaxD];                      // their token masks
  unsigned char pr[kMaxD][MOE_MAX_BATCH];     // selection rank r of token b for slot d
  float pw[kMaxPairs];                        // combine weight x W2 tensor scale, per pair
  float red[NW][2][MOE_MAX_BATCH];            // router / norm partial sums
  float rn[MOE_MAX_BATCH];                    // 1/rms per token
  int nd;
  uint32_t tag;
};

// Activation pairs: routed pair of token b's r-th selection = b k + r;
// shared expert s of token b = B k + s B + b.

// ---------------------------------------------------------------------------
// weight tiles
// ---------------------------------------------------------------------------

// One lane's share of one wave step of a packed matrix.
template <int WT> struct Tile;
template <> struct Tile<WT_NVFP4> { uint4 c; uint32_t sw; };
template <> struct Tile<WT_BF16> { uint4 c[4]; };

// `dummy` when dm, else `real`, computed without a branch (a branch would
// duplicate the load that uses it and make the loads in flight depend on
// data, which costs a full wait for every load before the copy).
__device__ __forceinline__ const uint8_t* pick(bool dm, const uint8_t* real, const uint8_t* dummy) {
  const uintptr_t m = (uintptr_t)0 - (uintptr_t)dm;
  return reinterpret_cast<const uint8_t*>((uintptr_t)real ^ (((uintptr_t)real ^ (uintptr_t)dummy) & m));
}

// Loads the lane's chunk of (slice s, step t) of a packed matrix.  A dummy
// load reads the first bytes of `dummy` instead (same instructions, so the
// number of loads in flight never depends on data; the value is unused).
template <int WT>
__device__ __forceinline__ void tile_load(Tile<WT>& tl, const uint8_t* codes, const uint8_t* scales,
                                          const MatGeom& g, int s, int t, int ri, int j, bool dm,
                                          const uint8_t* dummy) {
  if constexpr (WT == WT_NVFP4) {
    tl.c = ld16(pick(dm, codes + code_unit(g, s, t, ri, j) * 16, dummy));
    tl.sw = *reinterpret_cast<const uint32_t*>(pick(dm, scales + scale_word(g, s, t, ri, j), dummy));
  } else {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) tl.c[sub] = ld16(pick(dm, codes + bf16_unit(g, s, t, sub, ri, j) * 16, dummy));
  }
}

// sum of the lane's 32 weights times act (16 bf16 pairs).  NVFP4: the two
// block scales are bytes 0, 1 of sp.
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4& c, uint32_t sp, const uint32_t (&act)[16]) {
  uint32_t w[16];
  decode_chunk(c, w);
  return fmaf(dot8<8>(w, act), e4m3f<1>(sp), dot8<0>(w, act) * e4m3f<0>(sp));
}
__device__ __forceinline__ float chunk_dot_bf16(const uint4 (&c)[4], const uint32_t (&act)[16]) {
  uint32_t w[16];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) unpack4(c[sub], &w[4 * sub]);
  return dot8<0>(w, act) + dot8<8>(w, act);
}
template <int WT>
__device__ __forceinline__ float tile_dot(const Tile<WT>& tl, int t, const uint32_t (&act)[16]) {
  if constexpr (WT == WT_NVFP4) return chunk_dot<WT>(tl.c, (t & 1) ? (tl.sw >> 16) : tl.sw, act);
  else return chunk_dot_bf16(tl.c, act);
}

// The four tiles of one gate/up item (gate steps 2t2, 2t2+1, up steps
// gate_steps + 2t2, +1) for one slice; NVFP4 scale words pair the two steps.
template <int WT> struct Quad;
template <> struct Quad<WT_NVFP4> { uint4 c[4]; uint32_t sw[2]; };
template <> struct Quad<WT_BF16> { uint4 c[4][4]; };

template <int WT>
__device__ __forceinline__ void quad_load(Quad<WT>& q, const uint8_t* codes, const uint8_t* scales, const MatGeom& g,
                                          int sl, int gate_steps, int t2, int ri, int j, bool dm,
                                          const uint8_t* dummy) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = u * gate_steps + 2 * t2;
    if constexpr (WT == WT_NVFP4) {
      q.c[2 * u] = ld16(pick(dm, codes + code_unit(g, sl, t, ri, j) * 16, dummy));
      q.c[2 * u + 1] = ld16(pick(dm, codes + code_unit(g, sl, t + 1, ri, j) * 16, dummy));
      q.sw[u] = *reinterpret_cast<const uint32_t*>(pick(dm, scales + scale_word(g, sl, t, ri, j), dummy));
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
          q.c[2 * u + st][sub] = ld16(pick(dm, codes + bf16_unit(g, sl, t + st, sub, ri, j) * 16, dummy));
    }
  }
}

// v = (gate st0, gate st1, up st0, up st1) lane partial dots.
template <int WT>
__device__ __forceinline__ void quad_dot(const Quad<WT>& q, const uint32_t (&x)[16], float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (WT == WT_NVFP4) v[i] = chunk_dot<WT>(q.c[i], (i & 1) ? (q.sw[i >> 1] >> 16) : q.sw[i >> 1], x);
    else v[i] = chunk_dot_bf16(q.c[i], x);
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
// gate/up phases
// ---------------------------------------------------------------------------

// Expert of a gate/up slot: shared expert `slot`, or the slot-th distinct
// selected routed expert.
struct Expert {
  const uint8_t* codes;
  const uint8_t* scales;
  float g13;
  unsigned mask;
};

template <int WT>
__device__ __forceinline__ Expert expert_of(const FusedArgs& a, const Smem& s, int shared, int slot) {
  Expert x;
  if (shared) {
    // a layer without shared experts has no shared buffer: x stands in (its
    // items are all dummies, whose loads read x anyway)
    const uint8_t* sc = a.s_codes ? a.s_codes : reinterpret_cast<const uint8_t*>(a.x);
    const uint8_t* ss = a.s_scales ? a.s_scales : reinterpret_cast<const uint8_t*>(a.x);
    slot = min(slot, MOE_MAX_SHARED - 1);
    x.codes = sc + (size_t)slot * a.s_code_stride;
    x.scales = (WT == WT_NVFP4) ? ss + (size_t)slot * a.s_scale_stride : nullptr;
    x.g13 = (WT == WT_NVFP4) ? s.tss[slot][0] : 1.0f;
    x.mask = (1u << a.B) - 1u;
  } else {
    slot = min(slot, kMaxD - 1);
    const int e = min(max(s.ids[slot], 0), a.E - 1);
    x.codes = a.r_codes + (size_t)e * a.r_code_stride;
    x.scales = (WT == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride : nullptr;
    x.g13 = (WT == WT_NVFP4) ? s.tsr[e][0] : 1.0f;
    x.mask = s.dmask[slot];
  }
  return x;
}

__device__ __forceinline__ int gu_pair(const FusedArgs& a, const Smem& s, int shared, int slot, int b) {
  return shared ? a.B * a.k + slot * a.B + b : b * a.k + s.pr[slot][b];
}

// Gate/up items of one workgroup: item j = (slot j / gs2, step pair j % gs2),
// block [lo, hi).  With one wave step per row (ns = 1) each wave takes items
// lo + wave, lo + wave + NW, ... on its own and publishes their SiLU*up
// words; with ns > 1 the ns waves of a group share items, wave w % ns taking
// slice w % ns, and after one barrier the workgroup combines the slices in
// order.  PI items are loading at a time.
template <int TB, int WT, int PI>
struct GateUp {
  Quad<WT> q[PI];
  int qslot[PI], qt2[PI];
  int shared, lo, hi, gs2, gate_steps;
  int ns, grp, ngr, sl;
  int nmine, nloaded, cslot, ct2;   // this wave's item count, items loaded, next item
  int ri, jj, jc;
  bool active;

  __device__ __forceinline__ void setup(const FusedArgs& a, int shared_, int n, int w, int G) {
    const MatGeom& g = a.g13;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    shared = shared_;
    gate_steps = a.I / g.rpw;
    gs2 = gate_steps / 2;
    lo = (int)((long long)n * w / G);
    hi = (int)((long long)n * (w + 1) / G);
    ns = g.ns;
    ngr = NW / ns;
    grp = wave / ns;
    sl = wave % ns;
    if (ns == 1) {
      ri = lane / g.lpr;
      jj = lane % g.lpr;
      active = jj < g.cw;
    } else {
      ri = 0;
      jj = lane;
      active = lane < g.cw;
    }
    jc = active ? jj : 0;
    const int first = lo + grp;
    nmine = (hi > first) ? (hi - first + ngr - 1) / ngr : 0;
    nloaded = 0;
    cslot = first / gs2;
    ct2 = first % gs2;
  }
  // Loads the next item of this wave, or a dummy once they are all loaded.
  __device__ __forceinline__ void load_next(const FusedArgs& a, const Smem& s, int p) {
    const bool dm = nloaded >= nmine;
    const Expert x = expert_of<WT>(a, s, shared, cslot);
    quad_load<WT>(q[p], x.codes, x.scales, a.g13, sl, gate_steps, ct2, ri, jc, dm,
                  reinterpret_cast<const uint8_t*>(a.x));
    qslot[p] = cslot;
    qt2[p] = ct2;
    if (!dm) {
      ++nloaded;
      ct2 += ngr;
      while (ct2 >= gs2) {
        ct2 -= gs2;
        ++cslot;
      }
    }
  }
  __device__ __forceinline__ void prime(const FusedArgs& a, const Smem& s) {
#pragma unroll
    for (int p = 0; p < PI; ++p) load_next(a, s, p);
  }
  // part: TB * 4 * ns floats per item of the block (ns > 1 only).
  __device__ __forceinline__ void run(const FusedArgs& a, const Smem& s, const uint32_t (&xr)[TB][16], float* part,
                                      uint32_t tag) {
    const int I2 = a.I / 2;
    const int lpr = a.g13.lpr;
    for (int base = 0; base < nmine; base += PI) {
#pragma unroll
      for (int p = 0; p < PI; ++p) {
        const int i = base + p;
        const bool live = i < nmine;   // uniform
        const int slot = qslot[p], t2 = qt2[p];
        const Expert x = expert_of<WT>(a, s, shared, slot);
        float v[TB][4];
        if (live) {
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if ((x.mask >> b) & 1u) {
              quad_dot<WT>(q[p], xr[b], v[b]);
              if (!active) v[b][0] = v[b][1] = v[b][2] = v[b][3] = 0.f;
            }
          }
        }
        // The buffer is free only now.  Its reload is unconditional (a dummy
        // past the end) and kept below the reads: a conditional or hoisted
        // reload would make the compiler copy registers and wait for every
        // load in flight.
        __asm__ volatile("" ::: "memory");
        load_next(a, s, p);
        if (live) {
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if (!((x.mask >> b) & 1u)) continue;
            if (ns == 1) {
#pragma unroll
              for (int c = 0; c < 4; ++c) v[b][c] = lane_reduce(v[b][c], lpr);
              if (jj == 0) {
                const float h0 = silu_mul(v[b][0] * x.g13, v[b][2] * x.g13);
                const float h1 = silu_mul(v[b][1] * x.g13, v[b][3] * x.g13);
                publish(a.xh + (size_t)gu_pair(a, s, shared, slot, b) * I2 + t2 * a.g13.rpw + ri,
                        f2bf(h0) | (f2bf(h1) << 16), tag);
              }
            } else {
              const int il = slot * gs2 + t2 - lo;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float sum = lane_reduce(v[b][c], 64);
                if (jj == 0) part[((il * TB + b) * 4 + c) * ns + sl] = sum;
              }
            }
          }
        }
      }
    }
    if (ns > 1) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < (hi - lo) * TB; idx += NT) {
        const int il = idx / TB, b = idx % TB;
        const int j = lo + il, slot = j / gs2, t2 = j % gs2;
        const Expert x = expert_of<WT>(a, s, shared, slot);
        if (!((x.mask >> b) & 1u)) continue;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float acc = 0.f;
          for (int u = 0; u < ns; ++u) acc += part[((il * TB + b) * 4 + c) * ns + u];
          v[c] = acc;
        }
        const float h0 = silu_mul(v[0] * x.g13, v[2] * x.g13);
        const float h1 = silu_mul(v[1] * x.g13, v[3] * x.g13);
        publish(a.xh + (size_t)gu_pair(a, s, shared, slot, b) * I2 + t2, f2bf(h0) | (f2bf(h1) << 16), tag);
      }
    }
  }
};

// This lane's activation chunk(s) from the x region of shared memory.
template <int TB>
__device__ __forceinline__ void load_xr(const FusedArgs& a, const uint16_t* xs, uint32_t (&xr)[TB][16]) {
  const MatGeom& g = a.g13;
  const int wave = wave_id(), lane = threadIdx.x & 63;
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
// [l m, l m + m) and keeps its best untaken one; each round the wave's best
// key wins, ties to the lowest lane, i.e. the lowest expert index), routing
// weights and shared coefficients.  Then wave 0 numbers the distinct
// selected experts by first appearance in (token, rank) order and fills the
// combine weight of every pair.  Ends with a barrier.
template <int WTR, int WTS>
__device__ __forceinline__ void route(const FusedArgs& a, Smem& s, const float* lg /* [B][Er] */) {
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
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
    unsigned bk = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if (key[i] > bk) { bk = key[i]; bi = i; }
    int my_e = 0;
    float my_l = 0.f;
    for (int r = 0; r < a.k; ++r) {
      const unsigned M = wave_umax(bk);
      const int win = __builtin_ctzll(__ballot(bk == M));
      const int wi = __builtin_amdgcn_readlane(bi, win);
      if (lane == r) {
        my_e = min(win * m + wi, a.E - 1);
        my_l = unkey(M);
      }
      if (lane == win) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i == wi) key[i] = 0u;
        bk = key[0];
        bi = 0;
#pragma unroll
        for (int i = 1; i < 8; ++i)
          if (key[i] > bk) { bk = key[i]; bi = i; }
      }
    }
    float wv;
    if (a.route == MOE_ROUTE_SOFTMAX_SINK) {
      float mx = -INFINITY;
      for (int e = lane; e < a.Er; e += 64) mx = fmaxf(mx, l[e]);
      mx = unkey(wave_umax(fkey(mx)));
      float z = 0.f;
      for (int e = lane; e < a.Er; e += 64) z += __expf(l[e] - mx);
      z = wave_fsum(z);
      wv = __expf(my_l - mx) / z;
      if (lane < a.S) s.shc[b][lane] = __expf(l[a.E + lane] - mx) / z;
    } else {
      const float sg = (lane < a.k) ? 1.0f / (1.0f + __expf(-my_l)) : 0.f;
      wv = sg / wave_fsum(sg);
      if (lane < a.S) s.shc[b][lane] = 1.0f;
    }
    if (lane < a.k) {
      s.sel[b][lane] = my_e;
      s.selw[b][lane] = wv;
      atomicOr(&s.emask[my_e], 1u << b);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int nk = a.B * a.k;
    int nd = 0;
    int eh[2], bh[2], rh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      const bool valid = i < nk;
      const int b = valid ? i / a.k : 0, r = valid ? i - b * a.k : 0;
      const int e = valid ? s.sel[b][r] : 0;
      const unsigned mk = valid ? s.emask[e] : 0u;
      const bool rep = valid && b == __builtin_ctz(mk | 0x80000000u);
      const unsigned long long bal = __ballot(rep);
      const int slot = nd + __popcll(bal & ((1ull << lane) - 1ull));
      if (rep) {
        s.ids[slot] = e;
        s.dmask[slot] = mk;
        s.slotmap[e] = slot;
      }
      nd += __popcll(bal);
      eh[h] = e;
      bh[h] = b;
      rh[h] = r;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      if (i < nk) {
        s.pr[s.slotmap[eh[h]]][bh[h]] = (unsigned char)rh[h];
        const float g2 = (WTR == WT_NVFP4) ? s.tsr[eh[h]][1] : 1.0f;
        s.pw[i] = s.selw[bh[h]][rh[h]] * g2;
      }
    }
    for (int i = lane; i < a.B * a.S; i += 64) {
      const int sh = i / a.B, b = i - sh * a.B;
      const float g2 = (WTS == WT_NVFP4) ? s.tss[sh][1] : 1.0f;
      s.pw[nk + i] = s.shc[b][sh] * g2;
    }
    if (lane == 0) s.nd = nd;
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

// The workgroup owns output steps [t_lo, t_lo + spg) of W2.  Experts in
// order: shared 0..S-1, then routed slots 0..nd-1.  If spg >= NW, wave w
// takes steps w, w + NW, ... with every expert; otherwise nsub = NW / spg
// waves share a step, wave w taking experts w / spg, w / spg + nsub, ...
// Per step the lane sums weight x partial dot over its experts in
// registers; one lane reduction per (step, token) follows.  P tiles are
// loading at a time.
template <int TB, int WTR, int WTS, int P>
struct Down {
  Tile<WTR> br[P];
  Tile<WTS> bs[(WTR == WTS) ? 1 : P];   // same types: shared tiles use br
  int t_lo, spg, nsub, sub, nex, nj, ntiles;
  int cj, cx, nloaded;                 // next tile to load: step index, expert index (mine)
  int qj[P], qx[P];
  int ri, jj, jc;
  bool active;

  __device__ __forceinline__ void setup(const FusedArgs& a, const Smem& s, int t_lo_, int spg_) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    t_lo = t_lo_;
    spg = spg_;
    ri = lane / a.g2.lpr;
    jj = lane % a.g2.lpr;
    active = jj < a.g2.cw;
    jc = active ? jj : 0;
    const int nexp = a.S + s.nd;
    if (spg >= NW || spg == 0) {
      nsub = 1;
      sub = 0;
      nj = (spg > wave) ? (spg - wave + NW - 1) / NW : 0;
      cj = wave;
    } else {
      nsub = NW / spg;
      sub = wave / spg;
      nj = (sub < nsub) ? 1 : 0;
      cj = wave % spg;
    }
    nex = (nexp > sub) ? (nexp - sub + nsub - 1) / nsub : 0;
    ntiles = nj * nex;
    cx = 0;
    nloaded = 0;
  }
  __device__ __forceinline__ int ex_of(int xi) const { return sub + xi * nsub; }
  // Loads the next tile of this wave, or a dummy once they are all loaded.
  __device__ __forceinline__ void load_next(const FusedArgs& a, const Smem& s, int p) {
    const bool dm = nloaded >= ntiles;
    const int ex = dm ? 0 : ex_of(cx), t = dm ? t_lo : t_lo + cj;
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.x);
    if (ex < a.S) {
      const uint8_t* c = a.s_codes + (size_t)ex * a.s_code_stride + a.s_w13_code;
      const uint8_t* sc = (WTS == WT_NVFP4) ? a.s_scales + (size_t)ex * a.s_scale_stride + a.s_w13_scale : nullptr;
      if constexpr (WTR == WTS) tile_load<WTR>(br[p], c, sc, a.g2, 0, t, ri, jc, dm, dummy);
      else tile_load<WTS>(bs[p], c, sc, a.g2, 0, t, ri, jc, dm, dummy);
    } else {
      const int e = min(max(s.ids[min(ex - a.S, kMaxD - 1)], 0), a.E - 1);
      const uint8_t* c = a.r_codes + (size_t)e * a.r_code_stride + a.r_w13_code;
      const uint8_t* sc = (WTR == WT_NVFP4) ? a.r_scales + (size_t)e * a.r_scale_stride + a.r_w13_scale : nullptr;
      tile_load<WTR>(br[p], c, sc, a.g2, 0, t, ri, jc, dm, dummy);
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
  __device__ __forceinline__ void prime(const FusedArgs& a, const Smem& s) {
#pragma unroll
    for (int p = 0; p < P; ++p) load_next(a, s, p);
  }
  // hs: activations [pairs][I] bf16 (shared memory).  Results: nsub == 1 ->
  // out directly; else partial sums into red2 [nsub][TB][spg * rpw].
  __device__ __forceinline__ void run(const FusedArgs& a, const Smem& s, const uint16_t* hs, float* red2) {
    float acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = 0.f;
    const int rpw = a.g2.rpw, lpr = a.g2.lpr;
    for (int base = 0; base < ntiles; base += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int tau = base + p;
        const bool live = tau < ntiles;   // uniform
        const int j = qj[p], xi = qx[p], ex = ex_of(xi), t = t_lo + j;
        if (live) {
          const bool sh = ex < a.S;
          const int slot = ex - a.S;
          const unsigned mask = sh ? (1u << a.B) - 1u : s.dmask[slot];
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if ((mask >> b) & 1u) {
              const int pr = sh ? a.B * a.k + ex * a.B + b : b * a.k + s.pr[slot][b];
              uint32_t hv[16];
              lds_chunk(hs + (size_t)pr * a.I + jc * 32, hv);
              float v;
              if constexpr (WTR == WTS) v = tile_dot<WTR>(br[p], t, hv);
              else v = sh ? tile_dot<WTS>(bs[p], t, hv) : tile_dot<WTR>(br[p], t, hv);
              acc[b] = fmaf(active ? v : 0.f, s.pw[pr], acc[b]);
            }
          }
        }
        __asm__ volatile("" ::: "memory");
        load_next(a, s, p);   // unconditional, see GateUp::run
        if (live && xi == nex - 1) {
          // step complete: reduce each token's row sums over the row's lanes
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if (b < a.B) {
              const float v = lane_reduce(acc[b], lpr);
              if (jj == 0) {
                const int rl = j * rpw + ri;
                if (nsub == 1) {
                  const int row = t * rpw + ri;
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
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Items (gate/up) and tiles (down) in flight per wave.
template <int WT> constexpr int gu_depth() { return WT == WT_NVFP4 ? 2 : 1; }
template <int TB, int WTR, int WTS> constexpr int down_depth() {
  return (WTR == WT_NVFP4 && WTS == WT_NVFP4) ? (TB >= 8 ? 4 : 6) : 3;
}

// QX: 16-byte units of a router row per thread (H <= QX * NT * 8); the host
// picks the smallest that fits, so every one of them is a real load.
template <int TB, int QX, int WTR, int WTS>
__global__ __launch_bounds__(NT) void k_fused_layer(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ Smem s;
  __shared__ float lg[TB * MOE_MAX_ROUTED];

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int w = blockIdx.x, G = a.G;
  const u64 deadline = clock100() + a.wait_ticks;
  uint16_t* act = reinterpret_cast<uint16_t*>(dyn);                  // x (phases 1-2), h (phase 3)
  float* part = reinterpret_cast<float*>(dyn + (size_t)TB * a.H * 2); // gate/up partials (ns > 1)
  float* red2 = reinterpret_cast<float*>(dyn + a.lds_act);            // down partial sums (nsub > 1)

  // ---- loads that need nothing: call counter, router rows, x, gamma, tensor scales, shared tiles
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
      rw[rr][q] = ld16(a.router_w + (size_t)row * a.H + u * 8);
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
  // router bias of this workgroup's rows (unconditional: clamped row, x as a stand-in)
  float biasv[2];
  {
    const float* bsrc = a.bias != nullptr ? a.bias : reinterpret_cast<const float*>(a.x);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) biasv[rr] = bsrc[a.bias != nullptr ? min(w + rr * G, a.E - 1) : 0];
  }
  // tensor scales for the shared-memory tables (loaded unconditionally from
  // clamped addresses so that no load depends on a condition)
  const int nts = (WTR == WT_NVFP4 && a.r_tscale != nullptr) ? 2 * a.E : 0;
  const float* tsr_src = (WTR == WT_NVFP4 && a.r_tscale != nullptr) ? a.r_tscale : reinterpret_cast<const float*>(a.x);
  // (a layer without shared experts has no shared buffer: x stands in)
  const float* tss_src = (WTS == WT_NVFP4 && a.S > 0 && a.s_tscale != nullptr)
                             ? a.s_tscale : reinterpret_cast<const float*>(a.x);
  float tsv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) tsv[h] = tsr_src[min(tid + h * NT, max(nts, 1) - 1)];
  const float tss = tss_src[min(tid, max(2 * a.S, 1) - 1)];
  const int gs2 = a.I / a.g13.rpw / 2;
  GateUp<TB, WTS, gu_depth<WTS>()> gus;
  gus.setup(a, 1, a.S * gs2, w, G);
  gus.prime(a, s);     // shared experts' tiles (their addresses need no shared-memory table)

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
        {
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
        racc[rr][b] = (rr < nrr) ? lane_reduce(v, 64) : 0.f;
      }
    if (lane == 0)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int b = 0; b < TB; ++b) s.red[wave][rr][b] = racc[rr][b];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = tid + h * NT;
    if (i < nts) (&s.tsr[0][0])[i] = tsv[h];
  }
  if (WTS == WT_NVFP4 && tid < 2 * a.S) (&s.tss[0][0])[tid] = tss;
  if (tid == 0) s.tag = epoch + 1u;
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

  // ---- first poll of the logits, shared experts' gate/up, rest of the logits ----
  uint32_t xr[TB][16];
  load_xr<TB>(a, act, xr);
  auto laddr = [&](int i) { return a.xlog + (size_t)(i / a.B) * kLogitLine + (i % a.B); };
  Gather<2 * TB> lgat;
  lgat.issue(0, a.Er * a.B, laddr);
  gus.run(a, s, xr, part, tag);
  lgat.finish(tag, deadline, a.err, kErrLogitWait, laddr,
              [&](int i, uint32_t v) { lg[(i % a.B) * a.Er + i / a.B] = __uint_as_float(v); });
  __syncthreads();
  if (w == 0 && tid == 0) __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- routing ---------------------------------------------------------------------
  route<WTR, WTS>(a, s, lg);

  // ---- phase 2: selected experts' gate/up; the down weights start loading ------------
  const int nsteps2 = a.g2.nsteps;
  const int t_lo = (int)((long long)nsteps2 * w / G);
  const int t_hi = (int)((long long)nsteps2 * (w + 1) / G);
  Down<TB, WTR, WTS, down_depth<TB, WTR, WTS>()> down;
  down.setup(a, s, t_lo, t_hi - t_lo);
  {
    GateUp<TB, WTR, gu_depth<WTR>()> gur;
    gur.setup(a, 0, s.nd * gs2, w, G);
    gur.prime(a, s);
    down.prime(a, s);
    gur.run(a, s, xr, part, tag);
  }

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
  down.run(a, s, act, red2);
  if (down.nsub > 1) {
    __syncthreads();
    const int rows = (t_hi - t_lo) * a.g2.rpw;
    const int nsub = down.nsub;
    for (int i = tid; i < a.B * rows; i += NT) {
      const int b = i / rows, r = i - b * rows;
      float v = 0.f;
      for (int u = 0; u < nsub; ++u) v += red2[(u * TB + b) * rows + r];
      const int row = t_lo * a.g2.rpw + r;
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

}  // namespace

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <int TB, int QX, int WTR, int WTS>
static const void* fused_fn() {
  return reinterpret_cast<const void*>(&k_fused_layer<TB, QX, WTR, WTS>);
}

template <int TB, int QX>
static const void* fused_fn_wt(int rwt, int swt) {
  if (rwt == WT_NVFP4 && swt == WT_NVFP4) return fused_fn<TB, QX, WT_NVFP4, WT_NVFP4>();
  if (rwt == WT_BF16 && swt == WT_BF16) return fused_fn<TB, QX, WT_BF16, WT_BF16>();
  if (rwt == WT_NVFP4 && swt == WT_BF16) return fused_fn<TB, QX, WT_NVFP4, WT_BF16>();
  return nullptr;
}

// qx 1 covers H <= 2048, qx 4 H <= 8192 (batch buckets 1, 2, 4 only).
static const void* fused_kernel(int tb, int qx, int rwt, int swt) {
  if (qx == 1) {
    switch (tb) {
      case 1: return fused_fn_wt<1, 1>(rwt, swt);
      case 2: return fused_fn_wt<2, 1>(rwt, swt);
      case 4: return fused_fn_wt<4, 1>(rwt, swt);
      case 8: return fused_fn_wt<8, 1>(rwt, swt);
      default: return nullptr;
    }
  }
  if (qx == 4) {
    switch (tb) {
      case 1: return fused_fn_wt<1, 4>(rwt, swt);
      case 2: return fused_fn_wt<2, 4>(rwt, swt);
      case 4: return fused_fn_wt<4, 4>(rwt, swt);
      default: return nullptr;
    }
  }
  return nullptr;
}

int fused_qx(int hidden) { return hidden / 8 <= NT ? 1 : (hidden / 8 <= 4 * NT ? 4 : 0); }

int fused_occupancy(int tb, int qx, int rwt, int swt, int lds_bytes, int* blocks_per_cu) {
  const void* f = fused_kernel(tb, qx, rwt, swt);
  if (f == nullptr) return (int)hipErrorInvalidValue;
  if (lds_bytes > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, NT, lds_bytes);
}

int launch_fused(const FusedArgs& a, int tb, int rwt, int swt, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const void* f = fused_kernel(tb, fused_qx(a.H), rwt, swt);
  if (f == nullptr) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();  // clear a stale error so it is not reported as ours
  void* args[] = {const_cast<FusedArgs*>(&a)};
  return (int)hipLaunchKernel(f, dim3(a.G), dim3(NT), args, (size_t)fused_lds_bytes(a), st);
}

int launch_fused_debug_h(const FusedArgs& a, uint16_t* h_r, uint16_t* h_s, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int n = a.B * a.k + a.B * a.S;
  hipLaunchKernelGGL(k_fused_debug_h, dim3(n), dim3(NT), 0, st, a, h_r, h_s);
  return (int)hipGetLastError();
}

}  // namespace moe
