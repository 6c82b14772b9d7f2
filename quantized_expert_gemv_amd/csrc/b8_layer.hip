// Small-batch (2 to 8 tokens) Flint-shaped NVFP4 MoE decode layer for MI355X
// (gfx950): one launch of 256 workgroups of eight wavefronts.
//
// The layer (Flint page, "A 40B MoE that activates 2.5B parameters": hidden
// 2048, 256 routed experts of intermediate 512, sigmoid top-6 plus one shared
// expert; NVFP4 weights, bf16 activations) at batch B reads the union of the
// tokens' selected experts once (Flint page, "From 1,096 kernels to 346": the
// weight bytes of experts nobody chose are never fetched).  Workgroup w owns
// gate/up rows 2w, 2w + 1 (and the matching up rows) and down rows
// [8w, 8w + 8) of every expert in the union.
//
//   1. Wave b < B loads token b's x (and the pre-norm), the workgroup's router
//      row, and publishes token b's logit for expert w; wave 7 starts loading
//      the shared expert's rows.
//   2. Every workgroup gathers the 256 x B logits; wave b takes token b's
//      top-6 and routing weights; the union of the selections becomes a list
//      of slots (in expert order) with the tokens of each.
//   3. Items (the shared expert, then the slots) go round-robin to the waves.
//      A wave streams its items' gate/up rows two at a time, computes
//      SiLU(gate) * up of intermediates 2w, 2w + 1 for each token of the item
//      and publishes it (one h word per token and item), then loads its
//      items' down rows.
//   4. All h words are gathered; each wave multiplies its items' down rows
//      with the items' tokens' h and routing weights, and the waves' partial
//      rows are added in wave order (+ residual) into the bf16 output.
//
// Workgroups exchange data through tagged words in device memory (the same
// words, layout and tags as the general kernel).  Every wait is bounded.
// No floating-point atomics: the result is the same on every run.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

using F = FlintShape;
constexpr int kSbWaves = 8;
constexpr int kSbThreads = 64 * kSbWaves;
constexpr int SH = F::H, SI = F::I, SE = F::E, SK = F::k;
constexpr int kSbMaxB = MOE_MAX_BATCH;
constexpr int kSbSlots = kSbMaxB * SK;                 // distinct routed experts at most
constexpr int kSbPairs = kSbMaxB * (SK + 1);           // h pairs at most
constexpr uint32_t kSbRow13 = 1024;                    // codes of one W13 row
constexpr uint32_t kSbStep2 = 1024;                    // codes of one W2 step (4 rows)
static_assert(kSbWaves == kSbMaxB, "one routing wave per token");
static_assert(F::g13.rpw == 1 && F::g13.lpr == 64 && F::g2.rpw == 4 && F::g2.lpr == 16, "Flint geometry");

struct __align__(16) SbSmem {
  // x-hat and the logits until the routing is done, then the h words
  union {
    struct {
      uint4 xs[kSbMaxB][SH / 8];   // token b's x-hat, 16-byte units in swizzled order
      float lg[kSbMaxB][SE];
      uint4 rws[SH / 8];           // the workgroup's router row
    } a;
    uint32_t hs[kSbPairs][SI / 2];
  } u;
  unsigned emask[SE];             // tokens that selected expert e
  int slot_of[SE];                // slot of expert e (if selected)
  int sel[kSbMaxB][SK];           // token b's r-th selection
  float wv[kSbMaxB][SK];          // its routing weight
  int slot_e[kSbSlots];           // expert of slot d
  unsigned slot_m[kSbSlots];      // tokens of slot d
  int rk[kSbSlots][kSbMaxB];      // rank of slot d in token b's selections
  int cnt[4];
  int nd;
  uint32_t tag;
  int x_ready, rw_ready;
  int next_item;                  // routed items handed out so far
};
static_assert(sizeof(SbSmem) <= 64 * 1024, "shared memory of one workgroup");

__device__ __forceinline__ uint32_t tag_of_epoch(uint32_t epoch) { return (epoch + 1u == 0u) ? 1u : epoch + 1u; }

__device__ __forceinline__ void sb_wait(int* p, int v, u64 deadline, unsigned* err) {
  while (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < v) {
    if (clock100() > deadline) {
      __hip_atomic_fetch_or(err, kErrLocalWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Shared-memory position of 16-byte unit q (0..3) of 64-byte chunk l in a
// row of chunks: the units a wave reads in one instruction (one per chunk,
// same q) then fall in distinct banks.
__device__ __forceinline__ int unit_pos(int l, int q) { return (l << 2) | (q ^ ((l >> 2) & 3)); }

// One item's gate/up share in one lane: 32-column chunk `lane` of rows gate
// 2w, gate 2w + 1, up 2w, up 2w + 1; the block scales of a row pair share a
// word (bytes 0-1 the even row's, 2-3 the odd row's).
struct GuTile {
  uint4 c[4];
  uint32_t sg, su;
  float2 ts;   // tensor scales (W13, W2)
};
// One item's down share in one lane: steps 2w, 2w + 1, row lane / 16 of the
// step, chunk lane % 16; the two steps' block scales share one word.
struct DnTile {
  uint4 c[2];
  uint32_t sw;
};

// Item j of the layer: 0 the shared expert, 1 + d slot d.
struct ItemRef {
  const uint8_t *cb, *sb;
  const float* ts;
  uint32_t w2c, w2s;
};
__device__ __forceinline__ ItemRef item_ref(const KCommon& a, const SbSmem& s, int j) {
  ItemRef r;
  if (j == 0) {
    r.cb = a.s_codes;
    r.sb = a.s_scales;
    r.ts = a.s_tscale;
    r.w2c = (uint32_t)a.s_w13_code;
    r.w2s = (uint32_t)a.s_w13_scale;
  } else {
    const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(s.slot_e[j - 1]);
    r.cb = a.r_codes + (size_t)(e * (uint32_t)a.r_code_stride);
    r.sb = a.r_scales + (size_t)(e * (uint32_t)a.r_scale_stride);
    r.ts = a.r_tscale + 2 * e;
    r.w2c = (uint32_t)a.r_w13_code;
    r.w2s = (uint32_t)a.r_w13_scale;
  }
  return r;
}

// A dummy load (dm: past the last item) reads the first bytes of the item's
// regions (every lane the same 16 bytes) with the same instructions: the
// number of loads in flight then never depends on the item count, so each
// wait is for the oldest loads only.
struct GuOffsets {
  uint32_t gate, up, sg, su;   // byte offsets of this lane's gate / up codes and scale words
};
// two: the item's codes are 2-bit planes (same chunk order, 8 bytes a
// chunk: every code offset halves); they stay narrow in t.c[].x, .y until
// gu_item widens them, so that no instruction touches them before then.
__device__ __forceinline__ void gu_load(GuTile& t, const ItemRef& r, const GuOffsets& o, bool dm, bool two) {
  const uint32_t m = dm ? 0u : ~0u;
  t.ts = *reinterpret_cast<const float2*>(r.ts);
  const uint32_t off[4] = {o.gate & m, (o.gate + kSbRow13) & m, o.up & m, (o.up + kSbRow13) & m};
  if (two) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 v = ld8o(r.cb, off[i] >> 1);
      t.c[i] = make_uint4(v.x, v.y, 0u, 0u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) t.c[i] = ld16o(r.cb, off[i]);
  }
  t.sg = ld32o(r.sb, o.sg & m);
  t.su = ld32o(r.sb, o.su & m);
}

// Sums over the wave of four values at once (their DPP steps interleaved).
__device__ __forceinline__ void wave_sum4(float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = add_dpp<MOE_DPP_XOR1>(v[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = add_dpp<MOE_DPP_XOR2>(v[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = add_dpp<MOE_DPP_HALF_MIRROR>(v[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = add_dpp<MOE_DPP_MIRROR>(v[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[i]), MOE_DPP_ROW_BCAST15, 0xA, 0xF, false));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[i]), MOE_DPP_ROW_BCAST31, 0xC, 0xF, false));
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// SiLU(gate) * up of intermediates 2w, 2w + 1 for each token of item j, from
// the item's gate/up share; published as the token's h word w of its pair.
__device__ __forceinline__ void gu_item(const KCommon& a, SbSmem& s, const GuTile& t, int j, int B, int w, int lane,
                                        uint32_t tag, bool two) {
  uint32_t wd[4][16];
#pragma unroll
  for (int r = 0; r < 4; ++r) decode_chunk(two ? widen_2bit(make_uint2(t.c[r].x, t.c[r].y)) : t.c[r], wd[r]);
  float sc0[4], sc1[4];
  sc0[0] = e4m3f<0>(t.sg);
  sc1[0] = e4m3f<1>(t.sg);
  sc0[1] = e4m3f<2>(t.sg);
  sc1[1] = e4m3f<3>(t.sg);
  sc0[2] = e4m3f<0>(t.su);
  sc1[2] = e4m3f<1>(t.su);
  sc0[3] = e4m3f<2>(t.su);
  sc1[3] = e4m3f<3>(t.su);
  const unsigned mask = (j == 0) ? ((1u << B) - 1u) : (unsigned)__builtin_amdgcn_readfirstlane(s.slot_m[j - 1]);
  for (int b = 0; b < B; ++b) {
    if (!((mask >> b) & 1u)) continue;
    uint32_t xk[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(s.u.a.xs[b][unit_pos(lane, q)], &xk[4 * q]);
    float lo[4], hi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lo[r] = dot2(wd[r][0], xk[0], 0.f);
      hi[r] = dot2(wd[r][8], xk[8], 0.f);
    }
#pragma unroll
    for (int p = 1; p < 8; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lo[r] = dot2(wd[r][p], xk[p], lo[r]);
        hi[r] = dot2(wd[r][8 + p], xk[8 + p], hi[r]);
      }
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = fmaf(hi[r], sc1[r], lo[r] * sc0[r]);
    wave_sum4(v);   // gate 2w, gate 2w + 1, up 2w, up 2w + 1
    const float g = t.ts.x;
    const int pr = (j == 0) ? B * SK + b : b * SK + s.rk[j - 1][b];
    if (lane == 0)
      publish(a.xh + (size_t)pr * (SI / 2) + w, pack_bf16x2(silu_mul(v[0] * g, v[2] * g), silu_mul(v[1] * g, v[3] * g)), tag);
  }
}

// R2: the routed experts are 2-bit planes (the shared expert stays NVFP4).
template <bool R2>
__global__ __launch_bounds__(kSbThreads) void k_b8_layer(KCommon a, int B) {
  __shared__ SbSmem s;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int w = blockIdx.x;
  if (tid < SE) s.emask[tid] = 0u;
  if (tid == 0) s.x_ready = s.rw_ready = s.next_item = 0;
  __syncthreads();
  const u64 deadline = clock100() + a.wait_ticks;

  // ---- 1. token b's x-hat and logit for expert w (wave b) ------------------------------
  // wave 7 first issues the shared expert's gate/up share (item 0 is its)
  const int gq = lane >> 4, jj = lane & 15;
  const GuOffsets go = {(uint32_t)(2 * w) * kSbRow13 + (uint32_t)lane * 16u,
                        (uint32_t)(SI + 2 * w) * kSbRow13 + (uint32_t)lane * 16u,
                        (uint32_t)(w * 64 + lane) * 4u, (uint32_t)((SI / 2 + w) * 64 + lane) * 4u};
  uint32_t tag = 0;
  if (wave < B) {
    const int b = wave;
    uint4 xv[4], rw[4], gv[4];
    // wave 0 loads the router row for every token's wave
    if (b == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[q] = ld16nt(a.router_w + (size_t)w * SH + lane * 32 + q * 8);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = ld16(a.x + (size_t)b * SH + lane * 32 + q * 8);
    if (a.prenorm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) gv[q] = ld16(a.gamma + lane * 32 + q * 8);
    }
    const float bias = a.bias ? a.bias[w] : 0.0f;
    tag = tag_of_epoch(__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (b == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) s.u.a.rws[4 * lane + q] = rw[q];
      if (lane == 0) __hip_atomic_store(&s.rw_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (a.prenorm) {
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
      const float rn = 1.0f / sqrtf(wave_sum(ss) / (float)SH + a.eps);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[q] = make_uint4(norm_pair(xv[q].x, gv[q].x, rn), norm_pair(xv[q].y, gv[q].y, rn),
                           norm_pair(xv[q].z, gv[q].z, rn), norm_pair(xv[q].w, gv[q].w, rn));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) s.u.a.xs[b][unit_pos(lane, q)] = xv[q];
    if (b != 0) {
      sb_wait(&s.rw_ready, 1, deadline, a.err);
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[q] = s.u.a.rws[4 * lane + q];
    }
    uint32_t xr[16], wr[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unpack4(xv[q], &xr[4 * q]);
      unpack4(rw[q], &wr[4 * q]);
    }
    const float logit = wave_sum(dot8<0>(wr, xr) + dot8<8>(wr, xr)) + bias;
    if (lane == 0) {
      publish(a.xlog + (size_t)w * kLogitLine + b, __float_as_uint(logit), tag);
      if (b == 0) s.tag = tag;
      __hip_atomic_fetch_add(&s.x_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  GuTile g0, g1;
  const bool shared_wave = wave == kSbWaves - 1;
  if (shared_wave) {
    // after x: issued at the start, these loads slowed the router rows
    sb_wait(&s.x_ready, B, deadline, a.err);
    gu_load(g0, item_ref(a, s, 0), go, false, false);
  }

  // ---- 2. logits of every expert and token; routing; the union of the selections ---------
  // thread t polls expert t / 2, tokens 4 (t % 2) .. + 3; the first poll waits
  // ~0.6 us (s_sleep 24), while the others' logits are on their way
  __builtin_amdgcn_s_sleep(24);
  {
    const int e = tid >> 1, b0 = 4 * (tid & 1);
    const u64* lp = a.xlog + (size_t)e * kLogitLine + b0;
    u64 v[4];
    unsigned pend = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = peek(lp + min(i, max(B - b0 - 1, 0)));
      if (b0 + i < B) pend |= 1u << i;
    }
    __syncthreads();   // s.tag is written
    tag = s.tag;
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
        if ((pend >> i) & 1u) v[i] = peek(lp + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (b0 + i < B) s.u.a.lg[b0 + i][e] = __uint_as_float((uint32_t)v[i]);
  }
  __syncthreads();
  // every workgroup read the call counter before it published its logits
  if (w == 0 && tid == 0) __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wave < B) {
    // token b's top-6: lane l holds experts 4l .. 4l + 3, sorted; each round
    // the largest head key wins (ties to the lowest expert)
    const int b = wave;
    const float4 l4 = *reinterpret_cast<const float4*>(&s.u.a.lg[b][4 * lane]);
    unsigned key[4] = {sel_key(l4.x), sel_key(l4.y), sel_key(l4.z), sel_key(l4.w)};
    int idx[4] = {4 * lane, 4 * lane + 1, 4 * lane + 2, 4 * lane + 3};
    cas(key[0], idx[0], key[1], idx[1]);
    cas(key[2], idx[2], key[3], idx[3]);
    cas(key[0], idx[0], key[2], idx[2]);
    cas(key[1], idx[1], key[3], idx[3]);
    cas(key[1], idx[1], key[2], idx[2]);
    int my_e = 0;
    unsigned my_key = 0u;
#pragma unroll
    for (int r = 0; r < SK; ++r) {
      const unsigned M = wave_max_u32(key[0]);
      const int win = __builtin_ctzll(__ballot(key[0] == M));
      const int e_sel = __builtin_amdgcn_readlane(idx[0], win);
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
    const float sg = (lane < SK) ? __builtin_amdgcn_rcpf(1.0f + __expf(-unkey(my_key))) : 0.0f;
    const float sum = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(group_sum(sg, 16))));
    const float wgt = sg * __builtin_amdgcn_rcpf(sum);
    if (lane < SK) {
      s.sel[b][lane] = my_e;
      s.wv[b][lane] = wgt;
      __hip_atomic_fetch_or(&s.emask[my_e], 1u << b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (w == 0) {
        a.topk_ids[b * SK + lane] = my_e;
        a.topk_w[b * SK + lane] = wgt;
      }
    }
    if (w == 0 && lane == 0) a.shared_c[b] = 1.0f;
  }
  __syncthreads();
  // slots: the selected experts in expert order
  bool nz = false;
  unsigned long long bal = 0ull;
  if (tid < SE) {
    nz = s.emask[tid] != 0u;
    bal = __ballot(nz);
    if (lane == 0) s.cnt[wave] = __popcll(bal);
  }
  __syncthreads();
  if (tid < SE) {
    int off = 0;
    for (int q = 0; q < wave; ++q) off += s.cnt[q];
    const int d = off + __popcll(bal & ((1ull << lane) - 1ull));
    s.slot_of[tid] = d;
    if (nz) {
      s.slot_e[d] = tid;
      s.slot_m[d] = s.emask[tid];
    }
    if (tid == SE - 1) s.nd = off + __popcll(bal);
  }
  __syncthreads();
  if (tid < B * SK) {
    const int b = tid / SK, r = tid - b * SK;
    s.rk[s.slot_of[s.sel[b][r]]][b] = r;
  }
  __syncthreads();
  const int nd = s.nd;

  // ---- 3. gate/up of this wave's items, two in flight ---------------------------------
  // Down rows (step 4) are taken by token: wave b takes token b's seven pairs
  // (its selections in rank order, then the shared expert).  Their down
  // shares (rows [8w, 8w + 8) of each pair's expert; lane: row lane / 16 of a
  // 4-row step, 32-column chunk lane % 16) load now, with the gate/up rows.
  const int b = wave;
  const bool dn_wave = b < B;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.x);
  DnTile dn[SK + 1];
  {
    const uint32_t dn_c = (uint32_t)(2 * w) * kSbStep2 + (uint32_t)lane * 16u;
    const uint32_t dn_s = (uint32_t)(w * 64 + lane) * 4u;
#pragma unroll
    for (int p = 0; p <= SK; ++p) {
      // pair p < 6: the token's p-th selection; p = 6: the shared expert
      const int j = (p == SK) ? 0 : 1 + s.slot_of[s.sel[min(b, B - 1)][p]];
      const ItemRef r = item_ref(a, s, j);
      const uint8_t* cb = dn_wave ? r.cb + r.w2c : dummy;
      const uint8_t* sb = dn_wave ? r.sb + r.w2s : dummy;
      if (R2 && p < SK) {   // a routed pair's 2-bit rows: narrow until the down products
        const uint2 v0 = ld8o(cb, dn_wave ? dn_c >> 1 : 0u), v1 = ld8o(cb, dn_wave ? (dn_c + kSbStep2) >> 1 : 0u);
        dn[p].c[0] = make_uint4(v0.x, v0.y, 0u, 0u);
        dn[p].c[1] = make_uint4(v1.x, v1.y, 0u, 0u);
      } else {
        dn[p].c[0] = ld16o(cb, dn_wave ? dn_c : 0u);
        dn[p].c[1] = ld16o(cb, dn_wave ? dn_c + kSbStep2 : 0u);
      }
      dn[p].sw = ld32o(sb, dn_wave ? dn_s : 0u);
    }
  }
  // lanes 16 ri + 15 write rows 8w + ri and 8w + 4 + ri of token b at the end;
  // their residuals
  const int bb = min(b, B - 1);
  const uint16_t xr0 = a.x[(size_t)bb * SH + (2 * w) * 4 + gq];
  const uint16_t xr1 = a.x[(size_t)bb * SH + (2 * w + 1) * 4 + gq];
  // Items are handed out in order from a counter, two per wave at a time:
  // a wave takes the next one when it starts the load that replaces a
  // finished item, so the waves finish together.  The shared expert (item 0,
  // every token) is wave 7's first item.
  auto grab = [&]() {
    int j = 0;
    if (lane == 0) j = __hip_atomic_fetch_add(&s.next_item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return 1 + __builtin_amdgcn_readfirstlane(j);
  };
  // a grab past the last slot loads a dummy; later grabs are past it too
  int ja = shared_wave ? 0 : grab();
  int jb = grab();
  // item j's codes are 2-bit planes when R2 and j is a routed slot; a dummy
  // load past the last slot reads the last slot's region
  if (!shared_wave) gu_load(g0, item_ref(a, s, min(ja, nd)), go, ja > nd, R2 && ja > 0);
  gu_load(g1, item_ref(a, s, min(jb, nd)), go, jb > nd, R2);
  while (true) {
    if (ja > nd) break;
    gu_item(a, s, g0, ja, B, w, lane, tag, R2 && ja > 0);
    ja = grab();
    gu_load(g0, item_ref(a, s, min(ja, nd)), go, ja > nd, R2);
    if (jb > nd) break;
    gu_item(a, s, g1, jb, B, w, lane, tag, R2 && jb > 0);
    jb = grab();
    gu_load(g1, item_ref(a, s, min(jb, nd)), go, jb > nd, R2);
  }
  // ---- 4. down rows of token b: its pairs' 256 h words each, then the rows,
  // written straight to the output ---------------------------------------------------
  __syncthreads();   // every wave is done with x-hat and the logits
  if (!dn_wave) return;
  // combine weights: lane p < 6 the routing weight x W2 tensor scale of
  // selection p, lane 6 the shared expert's (coefficient 1)
  float cwl = 0.f;
  if (lane <= SK) {
    const float* ts = (lane == SK) ? a.s_tscale : a.r_tscale + 2 * s.sel[b][min(lane, SK - 1)];
    cwl = ((lane == SK) ? 1.0f : s.wv[b][min(lane, SK - 1)]) * ts[1];
  }
  // the token's 7 x 256 h words: lane l polls words l + 64 q of each pair.
  // The first poll waits ~0.4 us (s_sleep 16), when the other workgroups'
  // words have about arrived, and repeats every ~0.2 us.
  __builtin_amdgcn_s_sleep(16);
  {
    constexpr int NB = (SK + 1) * 4;
    auto word = [&](int q) {   // pair q / 4, word lane + 64 (q % 4)
      const int p = q >> 2;
      const int pr = (p == SK) ? B * SK + b : b * SK + p;
      return a.xh + (size_t)pr * (SI / 2) + lane + 64 * (q & 3);
    };
    u64 v[NB];
    unsigned pend = (1u << NB) - 1u;
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = peek(word(q));
    while (true) {
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((uint32_t)(v[q] >> 32) == tag) pend &= ~(1u << q);
      if (__ballot(pend != 0u) == 0ull) break;
      if (clock100() > deadline) {
        __hip_atomic_fetch_or(a.err, kErrActWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((pend >> q) & 1u) v[q] = peek(word(q));
    }
    // this wave's region: pair p's words, 16-byte units in swizzled order
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = lane + 64 * (q & 3), u = i >> 2;
      s.u.hs[b * (SK + 1) + (q >> 2)][(unit_pos(u >> 2, u & 3) << 2) | (i & 3)] = (uint32_t)v[q];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int p = 0; p <= SK; ++p) {
    uint32_t wd[2][16], hk[16];
    const bool two = R2 && p < SK;
    decode_chunk(two ? widen_2bit(make_uint2(dn[p].c[0].x, dn[p].c[0].y)) : dn[p].c[0], wd[0]);
    decode_chunk(two ? widen_2bit(make_uint2(dn[p].c[1].x, dn[p].c[1].y)) : dn[p].c[1], wd[1]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      unpack4(reinterpret_cast<const uint4*>(&s.u.hs[b * (SK + 1) + p][0])[unit_pos(jj, q)], &hk[4 * q]);
    float lo0 = dot2(wd[0][0], hk[0], 0.f), hi0 = dot2(wd[0][8], hk[8], 0.f);
    float lo1 = dot2(wd[1][0], hk[0], 0.f), hi1 = dot2(wd[1][8], hk[8], 0.f);
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      lo0 = dot2(wd[0][k], hk[k], lo0);
      hi0 = dot2(wd[0][8 + k], hk[8 + k], hi0);
      lo1 = dot2(wd[1][k], hk[k], lo1);
      hi1 = dot2(wd[1][8 + k], hk[8 + k], hi1);
    }
    const float cw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cwl), p));
    acc0 = fmaf(fmaf(hi0, e4m3f<1>(dn[p].sw), lo0 * e4m3f<0>(dn[p].sw)), cw, acc0);
    acc1 = fmaf(fmaf(hi1, e4m3f<3>(dn[p].sw), lo1 * e4m3f<2>(dn[p].sw)), cw, acc1);
  }
  const float r0 = group_sum(acc0, 16), r1 = group_sum(acc1, 16);
  // rows 8w + ri (step 2w) and 8w + 4 + ri (step 2w + 1) in lanes 16 ri + 15
  if (jj == 15) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = (2 * w + st) * 4 + gq;
      float o = st ? r1 : r0;
      if (a.residual) o += bf16lo(st ? xr1 : xr0);
      a.out[(size_t)b * SH + row] = (uint16_t)f2bf(o);
    }
  }
}

}  // namespace

int launch_b8(const KCommon& a, int batch, bool r2bit, void* stream) {
  if (batch < 2 || batch > kSbMaxB) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (r2bit) hipLaunchKernelGGL(k_b8_layer<true>, dim3(256), dim3(kSbThreads), 0, st, a, batch);
  else hipLaunchKernelGGL(k_b8_layer<false>, dim3(256), dim3(kSbThreads), 0, st, a, batch);
  return (int)hipGetLastError();
}

int b8_occupancy(int* blocks_per_cu) {
  int o0 = 0, o1 = 0;
  int rc = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &o0, reinterpret_cast<const void*>(&k_b8_layer<false>), kSbThreads, 0);
  if (rc == 0)
    rc = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&o1, reinterpret_cast<const void*>(&k_b8_layer<true>),
                                                           kSbThreads, 0);
  *blocks_per_cu = o0 < o1 ? o0 : o1;
  return rc;
}

}  // namespace moe
