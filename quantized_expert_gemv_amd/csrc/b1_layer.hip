// Batch-1 Flint-shaped NVFP4 MoE decode layer for MI355X (gfx950): one
// launch of 256 workgroups of eight wavefronts with fixed roles, for one
// layer or a chain of up to 16 layers (layer l + 1 takes layer l's output).
//
// The layer (Flint page, "A 40B MoE that activates 2.5B parameters": hidden
// 2048, 256 routed experts of intermediate 512, sigmoid top-6 plus one shared
// expert; NVFP4 weights, bf16 activations) at batch 1 is a chain of memory
// latencies: router rows -> logits of all 256 workgroups -> routing -> the
// selected experts' gate/up rows -> SiLU*up of all workgroups -> down rows.
// The Flint page ("From 1,096 kernels to 346") shortens such a chain by letting
// each kernel load its weights while the previous one still runs.  Here the
// chain is one launch, and each workgroup gives each expert a wavefront of its
// own, so that an expert's weights start loading the moment it is selected:
//
//   wave 0      control: the workgroup's router row (row w), its logit for
//               every workgroup, the gather of all 256 logits and the top-6.
//               Each round of the top-6 publishes its winner in shared memory
//               at once.  At the end it adds the experts' output rows with the
//               routing weights in a fixed order (+ residual) into bf16.
//   wave 1 + m  item m (0: the shared expert, 1 + r: the expert of round r):
//               gate/up rows 2w, 2w + 1 and the down rows [8w, 8w + 8) of its
//               expert, loaded as soon as the expert is known; SiLU(gate) * up
//               for intermediates 2w, 2w + 1 (one h word, published for every
//               workgroup); the gather of the item's 256 h words; its share of
//               the down GEMV.
//
// In a chain the next layer's router row and shared expert load while the
// current layer finishes (the Flint page's programmatic dependent launch lets
// each kernel load its weights while the previous one runs), and the layer's
// output rows travel to every workgroup as tagged words, the next layer's x.
//
// Waves of one workgroup hand data to each other through shared memory with
// flags and counters (counted over the chain: round r of layer l is 6l + r + 1);
// workgroups through tagged words in device memory (the same words and tags as
// the general kernel; layer l of a call uses the call's l-th tag).  Every wait
// is bounded.  No floating-point atomics: the result is the same on every run.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

using F = FlintShape;
constexpr int kB1Waves = 8;
constexpr int kB1Threads = 64 * kB1Waves;
constexpr int B1H = F::H, B1I = F::I, B1E = F::E, B1K = F::k;
constexpr int kItems = 1 + B1K;          // the shared expert, then the selected ones
constexpr uint32_t kRowBytes13 = 1024;   // codes of one W13 row (NVFP4, 2048 columns)
constexpr uint32_t kStepBytes2 = 1024;   // codes of one W2 step (4 rows of 512 columns)
static_assert(kB1Waves == 1 + kItems, "one wave per item plus the control wave");
static_assert(F::g13.rpw == 1 && F::g13.lpr == 64 && F::g2.rpw == 4 && F::g2.lpr == 16, "Flint geometry");
static_assert(F::g2.nsteps == 2 * 256 && F::g13.nsteps / 2 == 2 * 256,
              "two down steps and one gate/up step pair per workgroup");

struct __align__(16) B1Smem {
  uint4 xs[B1H / 8];             // xhat, 16-byte units in swizzled order
  uint32_t hs[kItems][B1I / 2];  // h pairs of each item, gathered by the item's wave
  int sel_e[B1K];                // expert of round r
  float wv[kItems];              // routing weight of item m (1 for the shared expert)
  float ts2[kItems];             // W2 tensor scale of item m's expert
  float part[kItems][2][4];      // item m's down rows [8w + 4 st + ri]
  float orows[8];                // the layer's output rows (chain: the next layer's words)
  uint32_t tag0;                 // the call's first tag (control -> items, before the first round)
  int nsel;                      // rounds published over the chain (control -> items)
  int x_ready;                   // layers whose xhat is in xs (control -> items)
  int dn_done;                   // items done over the chain (items -> control)
};

// Shared-memory flags and counters between the waves of a workgroup.
__device__ __forceinline__ void lds_release(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_arrive(int* p) {
  __hip_atomic_fetch_add(p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Waits (bounded) until *p >= v; past the deadline sets the error bit and returns.
__device__ __forceinline__ void lds_wait(int* p, int v, u64 deadline, unsigned* err) {
  while (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < v) {
    if (clock100() > deadline) {
      __hip_atomic_fetch_or(err, kErrLocalWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ uint32_t tag_of(uint32_t epoch) { return (epoch + 1u == 0u) ? 1u : epoch + 1u; }
// Tag of layer l of a call whose first tag is t0.
__device__ __forceinline__ uint32_t tag_at(uint32_t t0, int l) {
  uint32_t t = t0;
  for (int i = 0; i < l; ++i) t = tag_of(t);
  return t;
}


// Shared-memory position of 16-byte unit q of 64-byte chunk c: the units a
// wave reads in one instruction (one per chunk, same q) fall in distinct banks.
__device__ __forceinline__ int unit_pos(int c, int q) { return (c << 2) | (q ^ ((c >> 2) & 3)); }

// The kernel's arguments for chains of at most NMAX layers (a single layer
// gets a kernel of its own, NMAX = 1, with no layer loop).
template <int NMAX>
struct B1ArgsT {
  KCommon a;
  u64* xx;
  int n;
  ChainLayer L[NMAX];
};

// ------------------------------------------------------------------ control
template <int NMAX>
__device__ __forceinline__ void control(const B1ArgsT<NMAX>& args, B1Smem& s, int w, int lane, u64 deadline) {
  const KCommon& a = args.a;
  const int n = NMAX == 1 ? 1 : args.n;
  // lanes 0 .. 7 write rows (2w + lane / 4) 4 + lane % 4 of each layer
  const int orow = (2 * w + ((lane >> 2) & 1)) * 4 + (lane & 3);
  uint4 xv[4], rw[4], gv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rw[q] = ld16nt(args.L[0].router_w + (size_t)w * B1H + lane * 32 + q * 8);
#pragma unroll
  for (int q = 0; q < 4; ++q) xv[q] = ld16(a.x + lane * 32 + q * 8);
  uint16_t xres = a.x[orow];   // layer 0's residual, loaded long before it is added
  float bias = args.L[0].bias ? args.L[0].bias[w] : 0.0f;
  if (args.L[0].prenorm) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gv[q] = ld16(args.L[0].gamma + lane * 32 + q * 8);
  }
  // issued after the weights, so no wait for it delays them
  const uint32_t tag0 = tag_of(__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (lane == 0) s.tag0 = tag0;
  uint32_t tag = tag0;
  for (int l = 0; l < n; ++l) {
    const ChainLayer& Ly = args.L[l];
    if (NMAX > 1 && l > 0) {
      // the previous layer's output, as 1024 words of two bf16 each: lane l
      // takes words 16 l .. 16 l + 15 (its 32 elements).  Polls start ~0.85 us
      // after this workgroup's own words went out and repeat every ~0.4 us:
      // 8 KB per workgroup and round, sent earlier or more often they slow
      // the workgroups that are still finishing the layer
      const uint32_t tprev = tag;
      tag = tag_of(tag);
      __builtin_amdgcn_s_sleep(32);
      u64 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = peek(args.xx + 16 * lane + i);
      unsigned pend = 0xffffu;
      while (true) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((uint32_t)(v[i] >> 32) == tprev) pend &= ~(1u << i);
        if (__ballot(pend != 0u) == 0ull) break;
        if (clock100() > deadline) {
          __hip_atomic_fetch_or(a.err, kErrActWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(16);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((pend >> i) & 1u) v[i] = peek(args.xx + 16 * lane + i);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[q] = make_uint4((uint32_t)v[4 * q], (uint32_t)v[4 * q + 1], (uint32_t)v[4 * q + 2], (uint32_t)v[4 * q + 3]);
    }
    if (Ly.prenorm) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t d[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss = fmaf(bf16lo(d[i]), bf16lo(d[i]), ss);
          ss = fmaf(bf16hi(d[i]), bf16hi(d[i]), ss);
        }
      }
      const float rn = 1.0f / sqrtf(wave_sum(ss) / (float)B1H + Ly.eps);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[q] = make_uint4(norm_pair(xv[q].x, gv[q].x, rn), norm_pair(xv[q].y, gv[q].y, rn),
                           norm_pair(xv[q].z, gv[q].z, rn), norm_pair(xv[q].w, gv[q].w, rn));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) s.xs[unit_pos(lane, q)] = xv[q];
    if (lane == 0) lds_release(&s.x_ready, l + 1);
    // router row w -> this workgroup's logit, for every workgroup
    uint32_t xr[16], wr[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unpack4(xv[q], &xr[4 * q]);
      unpack4(rw[q], &wr[4 * q]);
    }
    const float logit = wave_sum(dot8<0>(wr, xr) + dot8<8>(wr, xr)) + bias;
    if (lane == 0) publish(a.xlog + (size_t)w * kLogitLine, __float_as_uint(logit), tag);
    // all logits (one 128-byte line each): lane l polls experts 4l .. 4l + 3,
    // the layout of the top-k below.  The first poll waits ~0.6 us (s_sleep
    // 24 = 1536 cycles): the others' logits are on their way, and polls sent
    // earlier slow the exchange.
    __builtin_amdgcn_s_sleep(24);
    u64 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = peek(a.xlog + (size_t)(4 * lane + i) * kLogitLine);
    unsigned pend = 0xfu;
    while (true) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((uint32_t)(v[i] >> 32) == tag) pend &= ~(1u << i);
      if (__ballot(pend != 0u) == 0ull) break;
      if (clock100() > deadline) {
        __hip_atomic_fetch_or(a.err, kErrLogitWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((pend >> i) & 1u) v[i] = peek(a.xlog + (size_t)(4 * lane + i) * kLogitLine);
    }
    // top-6 over lists of 4 per lane, sorted first; each round's winner (the
    // largest head key, ties to the lowest expert) goes to shared memory at once
    unsigned key[4];
    int idx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      key[i] = sel_key(__uint_as_float((uint32_t)v[i]));
      idx[i] = 4 * lane + i;
    }
    cas(key[0], idx[0], key[1], idx[1]);
    cas(key[2], idx[2], key[3], idx[3]);
    cas(key[0], idx[0], key[2], idx[2]);
    cas(key[1], idx[1], key[3], idx[3]);
    cas(key[1], idx[1], key[2], idx[2]);
    int my_e = 0;
    unsigned my_key = 0u;
#pragma unroll
    for (int r = 0; r < B1K; ++r) {
      const unsigned M = wave_max_u32(key[0]);
      const int win = __builtin_ctzll(__ballot(key[0] == M));
      const int e_sel = __builtin_amdgcn_readlane(idx[0], win);
      if (lane == 0) {
        s.sel_e[r] = e_sel;
        lds_release(&s.nsel, B1K * l + r + 1);
      }
      const bool me = lane == win;
      my_e = (lane == r) ? e_sel : my_e;
      my_key = (lane == r) ? M : my_key;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        key[i] = me ? key[i + 1] : key[i];
        idx[i] = me ? idx[i + 1] : idx[i];
      }
      key[3] = me ? 0u : key[3];
    }
    // routing weights: each selection's logistic value over their sum
    const float sg = (lane < B1K) ? __builtin_amdgcn_rcpf(1.0f + __expf(-unkey(my_key))) : 0.0f;
    const float sum = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(group_sum(sg, 16))));
    const float wgt = sg * __builtin_amdgcn_rcpf(sum);
    if (lane < B1K) s.wv[1 + lane] = wgt;
    if (lane == 0) s.wv[0] = 1.0f;   // the shared expert's coefficient
    if (w == 0) {
      if (lane < B1K) {
        Ly.topk_ids[lane] = my_e;
        Ly.topk_w[lane] = wgt;
      }
      if (lane == 0) {
        Ly.shared_c[0] = 1.0f;
        // every workgroup read the call counter before it published its
        // first logit; the counter moves past all of the call's tags
        if (l == 0) __hip_atomic_store(a.epoch, tag_at(tag0, n - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    const bool last = l + 1 == n;
    if (!last) {
      // the next layer's router row, bias and norm weights load while this
      // layer's experts run (issued here, they have arrived before the combine
      // below, whose shared-memory reads would otherwise wait for them)
      const ChainLayer& Ln = args.L[NMAX > 1 ? l + 1 : 0];
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[q] = ld16nt(Ln.router_w + (size_t)w * B1H + lane * 32 + q * 8);
      bias = Ln.bias ? Ln.bias[w] : 0.0f;
      if (Ln.prenorm) {
#pragma unroll
        for (int q = 0; q < 4; ++q) gv[q] = ld16(Ln.gamma + lane * 32 + q * 8);
      }
    }
    // the items' output rows, weighted and added in item order (+ residual)
    lds_wait(&s.dn_done, kItems * (l + 1), deadline, a.err);
    if (lane < 8) {
      const int st = lane >> 2, ri = lane & 3;
      float o = 0.f;
#pragma unroll
      for (int m = 0; m < kItems; ++m) o = fmaf(s.wv[m] * s.ts2[m], s.part[m][st][ri], o);
      if (Ly.residual) o += bf16lo(xres);
      const uint16_t ob = (uint16_t)f2bf(o);
      xres = ob;                               // the next layer's residual: this output
      if (last) a.out[orow] = ob;
      else s.orows[lane] = __uint_as_float((uint32_t)ob);
    }
    if (!last) {
      // rows 8w .. 8w + 7 -> words 4w .. 4w + 3 of the next layer's x
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < 4) {
        const uint32_t lo = __float_as_uint(s.orows[2 * lane]) & 0xffffu;
        const uint32_t hi = __float_as_uint(s.orows[2 * lane + 1]) & 0xffffu;
        publish(args.xx + 4 * w + lane, lo | (hi << 16), tag);
      }
    }
  }
}

// ------------------------------------------------------------------ items
// Item m's wave.  Gate/up: lanes 16 g .. 16 g + 15 take row g of (gate 2w,
// gate 2w + 1, up 2w, up 2w + 1), chunks (lane % 16) + 16 i, i < 4, of 32
// columns.  Down: lane = (row ri of the step's 4, 32-column chunk jj), steps
// 2w and 2w + 1, whose block scales share one word per lane.
template <int NMAX, bool R2>
__device__ __forceinline__ void item(const B1ArgsT<NMAX>& args, B1Smem& s, int w, int m, int lane, u64 deadline) {
  const KCommon& a = args.a;
  const int n = NMAX == 1 ? 1 : args.n;
  const int gq = lane >> 4, jj = lane & 15;
  const int grow = ((gq >> 1) ? B1I : 0) + 2 * w + (gq & 1);
  const uint32_t off_c = (uint32_t)grow * kRowBytes13 + (uint32_t)jj * 16u;
  const uint32_t off_s = (uint32_t)((grow >> 1) * 64 + jj) * 4u;
  const uint32_t dn_c = (uint32_t)(2 * w) * kStepBytes2 + (uint32_t)lane * 16u;
  const uint32_t dn_s = (uint32_t)(w * 64 + lane) * 4u;
  const int pr = (m == 0) ? B1K : m - 1;   // pair index: routed rank, then the shared expert
  for (int l = 0; l < n; ++l) {
    const ChainLayer& Ly = args.L[l];
    const uint8_t *cb, *sb;
    const float* tsp;
    uint32_t w2c, w2s;
    if (m == 0) {
      // the shared expert's loads wait for layer 0's x (issued at the start
      // they slowed the router rows, which every later step waits for), and
      // for a later layer, for this workgroup's items of the layer before:
      // they then load while the rows travel
      if (l == 0) lds_wait(&s.x_ready, 1, deadline, a.err);
      else lds_wait(&s.dn_done, kItems * l, deadline, a.err);
      cb = Ly.s_codes;
      sb = Ly.s_scales;
      tsp = Ly.s_tscale;
      w2c = (uint32_t)a.s_w13_code;
      w2s = (uint32_t)a.s_w13_scale;
    } else {
      lds_wait(&s.nsel, B1K * l + m, deadline, a.err);
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(s.sel_e[m - 1]);
      cb = Ly.r_codes + (size_t)(e * (uint32_t)a.r_code_stride);
      sb = Ly.r_scales + (size_t)(e * (uint32_t)a.r_scale_stride);
      tsp = Ly.r_tscale + 2 * e;
      w2c = (uint32_t)a.r_w13_code;
      w2s = (uint32_t)a.r_w13_scale;
    }
    // the tensor scales first, then the gate/up rows, then the down rows:
    // each wait below is for the oldest loads only.  A routed expert in the
    // 2-bit planes has 8-byte chunks at half the offsets (the same scales);
    // they are widened to e2m1 once they are in.
    const bool two = R2 && m > 0;
    const float ts13 = tsp[0], ts2 = tsp[1];
    uint4 c[4], d[2];
    uint2 c8[4], d8[2];
    uint32_t sw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (two) c8[i] = ld8o(cb, (off_c >> 1) + 128u * i);
      else c[i] = ld16o(cb, off_c + 256u * i);
      sw[i] = ld32o(sb, off_s + 64u * i);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (two) d8[st] = ld8o(cb + w2c, (dn_c >> 1) + (kStepBytes2 / 2) * st);
      else d[st] = ld16o(cb + w2c, dn_c + kStepBytes2 * st);
    }
    const uint32_t dsw = ld32o(sb + w2s, dn_s);
    // gate/up: four chunks per lane, then the row sums of 16 lanes
    lds_wait(&s.x_ready, l + 1, deadline, a.err);
    if (two) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = widen_2bit(c8[i]);
#pragma unroll
      for (int st = 0; st < 2; ++st) d[st] = widen_2bit(d8[st]);
    }
    uint32_t xk[4][16], sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) unpack4(s.xs[unit_pos(jj + 16 * i, q)], &xk[i][4 * q]);
      sp[i] = (gq & 1) ? (sw[i] >> 16) : sw[i];
    }
    float v[4];
    dots_fp4(c, sp, [&](int i) -> const uint32_t(&)[16] { return xk[i]; }, v);
    const float row = group_sum(((v[0] + v[1]) + v[2]) + v[3], 16);
    // SiLU(gate) * up of intermediates 2w, 2w + 1 -> the item's h word w
    const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row), 15));
    const float g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row), 31));
    const float u0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row), 47));
    const float u1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row), 63));
    const uint32_t tag = tag_at(s.tag0, l);
    if (lane == 0)
      publish(a.xh + (size_t)pr * (B1I / 2) + w, pack_bf16x2(silu_mul(g0 * ts13, u0 * ts13), silu_mul(g1 * ts13, u1 * ts13)),
              tag);
    // the item's 256 h words, from every workgroup.  Polling starts ~0.8 us
    // (s_sleep 32) after this workgroup's word is out, when the others' have
    // about arrived, and repeats every ~0.2 us: polls sent earlier or more
    // often slow the exchange they wait for.
    __builtin_amdgcn_s_sleep(32);
    // In a chain the workgroups drift apart over the layers and the polls of
    // the early ones slow the late ones: there the routed items wait ~0.4 us
    // more, and the shared expert, whose word is out well before the others'
    // (its weights loaded during the layer before), ~1 us more.
    if (NMAX > 1 && l > 0) {
      __builtin_amdgcn_s_sleep(16);
      if (m == 0) __builtin_amdgcn_s_sleep(24);
    }
    constexpr int NB = (B1I / 2) / 64;
    const u64* hp = a.xh + (size_t)pr * (B1I / 2) + lane;
    u64 hv[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) hv[q] = peek(hp + 64 * q);
    unsigned pend = (1u << NB) - 1u;
    while (true) {
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((uint32_t)(hv[q] >> 32) == tag) pend &= ~(1u << q);
      if (__ballot(pend != 0u) == 0ull) break;
      if (clock100() > deadline) {
        __hip_atomic_fetch_or(a.err, kErrActWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((pend >> q) & 1u) hv[q] = peek(hp + 64 * q);
    }
    // to the lanes that use them: lane (ri, jj) takes pairs 16 jj .. 16 jj + 15
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = lane + 64 * q, u = i >> 2;
      s.hs[m][(unit_pos(u >> 2, u & 3) << 2) | (i & 3)] = (uint32_t)hv[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint32_t hk[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(reinterpret_cast<const uint4*>(&s.hs[m][0])[unit_pos(jj, q)], &hk[4 * q]);
    // down rows [8w, 8w + 8): two steps of 4 rows
    const uint32_t dsp[2] = {dsw, dsw >> 16};
    float dv[2];
    dots_fp4(d, dsp, [&](int) -> const uint32_t(&)[16] { return hk; }, dv);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float r = group_sum(dv[st], 16);
      if (jj == 15) s.part[m][st][lane >> 4] = r;
    }
    if (lane == 0) s.ts2[m] = ts2;
    if (lane == 0) lds_arrive(&s.dn_done);
  }
}

template <int NMAX, bool R2>
__global__ __launch_bounds__(kB1Threads) void k_b1_layer(B1ArgsT<NMAX> args) {
  __shared__ B1Smem s;
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int w = blockIdx.x;
  // the flags start at zero before any wave waits on them; the barrier comes
  // before the first global load, so it waits for no memory
  if (threadIdx.x == 0) {
    s.nsel = 0;
    s.x_ready = s.dn_done = 0;
  }
  __syncthreads();
  const u64 deadline = clock100() + args.a.wait_ticks;
  if (wave == 0) control(args, s, w, lane, deadline);
  else item<NMAX, R2>(args, s, w, wave - 1, lane, deadline);
}

}  // namespace

int launch_b1(const B1Args& a, void* stream) {
  if (a.n < 1 || a.n > kMaxChain || (a.r2bit && a.n != 1)) return (int)hipErrorInvalidValue;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.n == 1) {
    B1ArgsT<1> one;
    one.a = a.a;
    one.xx = a.xx;
    one.n = 1;
    one.L[0] = a.L[0];
    if (a.r2bit) hipLaunchKernelGGL((k_b1_layer<1, true>), dim3(256), dim3(kB1Threads), 0, st, one);
    else hipLaunchKernelGGL((k_b1_layer<1, false>), dim3(256), dim3(kB1Threads), 0, st, one);
  } else {
    B1ArgsT<kMaxChain> all;
    all.a = a.a;
    all.xx = a.xx;
    all.n = a.n;
    for (int l = 0; l < kMaxChain; ++l) all.L[l] = a.L[l];
    hipLaunchKernelGGL((k_b1_layer<kMaxChain, false>), dim3(256), dim3(kB1Threads), 0, st, all);
  }
  return (int)hipGetLastError();
}

int b1_occupancy(int* blocks_per_cu) {
  int one = 0, two = 0, all = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &one, reinterpret_cast<const void*>(&k_b1_layer<1, false>), kB1Threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&two, reinterpret_cast<const void*>(&k_b1_layer<1, true>),
                                                     kB1Threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &all, reinterpret_cast<const void*>(&k_b1_layer<kMaxChain, false>), kB1Threads, 0);
  *blocks_per_cu = one < all ? (one < two ? one : two) : (all < two ? all : two);
  return (int)e;
}

}  // namespace moe
