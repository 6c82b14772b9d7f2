// Device building blocks shared by the MoE decode kernels (gfx950): tagged
// cross-workgroup words with bounded polls, DPP lane reductions, weight
// loads, the NVFP4 chunk dot product, SiLU*up, and the per-token top-k.
// Included inside namespace moe's anonymous namespace by each kernel file.
#pragma once

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
// owns words i = base + tid + NT*q, q < NB.  issue() sends the first poll (it
// can fly while the thread does other work); finish() re-reads the words
// that have not matched yet until all have, then hands (i, value) to sink.
// (A second poll in flight did not shorten the hand-off: its time is the
// stores' way to the memory side, not the polling rate.)  Past the deadline
// the error bit is set and the words are taken as they are.
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
// cross-lane reductions
// ---------------------------------------------------------------------------

// Reductions inside rows of 16 lanes use DPP butterflies (every lane of a
// group gets the group's result); across rows, DPP row broadcasts carry lane
// 15 of each row into the next row and lane 31 into rows 2 and 3, so lane 63
// ends with the result of all 64 lanes (lanes 31 and 63 with those of their
// 32-lane halves).  No permlane or LDS traffic; the order of the operations
// is fixed, so sums are deterministic.
#define MOE_DPP_ROW_BCAST15 0x142
#define MOE_DPP_ROW_BCAST31 0x143

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of `width` consecutive lanes (a power of two <= 64); the
// result is valid in lane width - 1 of each group (in every lane when width <= 16).
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v = add_dpp<MOE_DPP_XOR1>(v);
  if (width >= 4) v = add_dpp<MOE_DPP_XOR2>(v);
  if (width >= 8) v = add_dpp<MOE_DPP_HALF_MIRROR>(v);
  if (width >= 16) v = add_dpp<MOE_DPP_MIRROR>(v);
  if (width >= 32)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_ROW_BCAST15, 0xA, 0xF, false));
  if (width >= 64)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), MOE_DPP_ROW_BCAST31, 0xC, 0xF, false));
  return v;
}

// Wave-wide max of an unsigned key and sum of a float, uniform results.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_XOR1, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_XOR2, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_HALF_MIRROR, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_MIRROR, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_ROW_BCAST15, 0xA, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_ROW_BCAST31, 0xC, 0xF, false));
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum(v, 64)), 63));
}

// Loads at a wave-uniform base plus the lane's 32-bit offset (the
// scalar-base addressing form: no per-lane 64-bit address arithmetic).
// Weights are read once per call: non-temporal loads, so that they do not
// push the kernel's code, arguments and small shared data out of the L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16o(const uint8_t* base, uint32_t off) { return ld16nt(base + off); }
__device__ __forceinline__ uint32_t ld32o(const uint8_t* base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(base + off));
}

// One 8-byte chunk of the 2-bit planes (32 codes, element k in bits 2k,
// 2k+1) as the 16-byte e2m1 chunk of the same values: code q -> nibble
// {-4, -1, 1, 4} = {0xE, 0xA, 0x2, 0x6}, i.e. 0b0010 with bit 3 = NOT q1 and
// bit 2 = (q0 == q1).  The 2-bit fields are first spread to nibbles.
__device__ __forceinline__ uint32_t widen_2bit_half(uint32_t h) {
  uint32_t x = h & 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  const uint32_t b0 = x & 0x11111111u, b1 = (x >> 1) & 0x11111111u;
  return 0x22222222u | ((b1 ^ 0x11111111u) << 3) | ((~(b0 ^ b1) & 0x11111111u) << 2);
}
__device__ __forceinline__ uint4 widen_2bit(const uint2& v) {
  return make_uint4(widen_2bit_half(v.x), widen_2bit_half(v.x >> 16), widen_2bit_half(v.y), widen_2bit_half(v.y >> 16));
}
__device__ __forceinline__ uint2 ld8o(const uint8_t* base, uint32_t off) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(base + off));
  return make_uint2(v.x, v.y);
}

// sum of the lane's 32 weights times act (16 bf16 pairs).  NVFP4: the two
// block scales are bytes 0, 1 of sp.
__device__ __forceinline__ float chunk_dot_fp4(const uint4& c, uint32_t sp, const uint32_t (&act)[16]) {
  uint32_t w[16];
  decode_chunk(c, w);
  return fmaf(dot8c<8>(w, act), e4m3f<1>(sp), dot8c<0>(w, act) * e4m3f<0>(sp));
}
// N chunk dot products at once, each equal bit for bit to chunk_dot_fp4(c[j],
// sp[j], act(j)), with their dependent dot2 chains interleaved: a wave with
// few chains waits on each step's latency, N chains hide it N-fold.
template <int N, typename Act>
__device__ __forceinline__ void dots_fp4(const uint4 (&c)[N], const uint32_t (&sp)[N], Act&& act, float (&out)[N]) {
  uint32_t w[N][16];
#pragma unroll
  for (int j = 0; j < N; ++j) decode_chunk(c[j], w[j]);
  float lo[N], hi[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    lo[j] = dot2(w[j][0], act(j)[0], 0.f);
    hi[j] = dot2(w[j][8], act(j)[8], 0.f);
  }
#pragma unroll
  for (int i = 1; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) {
      lo[j] = dot2(w[j][i], act(j)[i], lo[j]);
      hi[j] = dot2(w[j][8 + i], act(j)[8 + i], hi[j]);
    }
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = fmaf(hi[j], e4m3f<1>(sp[j]), lo[j] * e4m3f<0>(sp[j]));
}

// 32 bf16 activations (16 pairs) at p (16-byte aligned, shared memory).
__device__ __forceinline__ void lds_chunk(const uint16_t* p, uint32_t (&a)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack4(q[i], &a[4 * i]);
}

// SiLU(g) * u; the logistic's reciprocal is the hardware's (1 ulp), far
// below the bf16 rounding of h that follows.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Key for selection: order-preserving integer of the logit; NaN ranks below
// every number (key 1) and a taken or absent expert has key 0.
__device__ __forceinline__ unsigned sel_key(float f) {
  const unsigned k = fkey(f);
  return k == 0u ? 1u : k;
}

// Compare-exchange for a descending order by key, ties to the lower expert.
__device__ __forceinline__ void cas(unsigned& ka, int& ia, unsigned& kb, int& ib) {
  const bool sw = kb > ka || (kb == ka && ib < ia);
  const unsigned k0 = sw ? kb : ka, k1 = sw ? ka : kb;
  const int i0 = sw ? ib : ia, i1 = sw ? ia : ib;
  ka = k0; kb = k1; ia = i0; ib = i1;
}

// Top-k of TPW tokens at once (token wave + t NW): lane l holds experts
// [l MK, l MK + MK), sorted by key.  Each round the wave's largest head key
// wins (ties to the lowest lane, i.e. the lowest expert), the winning lane
// shifts its list; the lanes' chains for the TPW tokens are independent.
// Lane r ends with the r-th selection: expert my_e, logit my_l, and its
// sigmoid my_sg; sg_sum (uniform) is the sum of the k sigmoids.  The rounds
// carry only the keys: the logistic values are computed afterwards, each in
// its own lane, which keeps them off the rounds' dependency chain.
template <int MK, int TPW, class A>
__device__ __forceinline__ void topk(const A& a, const float* lg, int lane, int (&my_e)[TPW], float (&my_l)[TPW],
                                     float (&my_sg)[TPW], float (&sg_sum)[TPW]) {
  const int wave = wave_id();
  unsigned key[TPW][MK];
  int idx[TPW][MK];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int b = min(wave + t * NW, a.B - 1);
    const float* l = lg + (size_t)b * a.Er;
#pragma unroll
    for (int i = 0; i < MK; ++i) {
      const int e = lane * MK + i;
      idx[t][i] = e;
      key[t][i] = (e < a.E) ? sel_key(l[e]) : 0u;
    }
    if constexpr (MK == 2) {
      cas(key[t][0], idx[t][0], key[t][1], idx[t][1]);
    } else if constexpr (MK == 4) {
      cas(key[t][0], idx[t][0], key[t][1], idx[t][1]);
      cas(key[t][2], idx[t][2], key[t][3], idx[t][3]);
      cas(key[t][0], idx[t][0], key[t][2], idx[t][2]);
      cas(key[t][1], idx[t][1], key[t][3], idx[t][3]);
      cas(key[t][1], idx[t][1], key[t][2], idx[t][2]);
    } else if constexpr (MK == 8) {
      constexpr int net[19][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6}, {5, 7}, {1, 2}, {5, 6},
                                  {0, 4}, {1, 5}, {2, 6}, {3, 7}, {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
      for (int c = 0; c < 19; ++c) cas(key[t][net[c][0]], idx[t][net[c][0]], key[t][net[c][1]], idx[t][net[c][1]]);
    }
    my_e[t] = 0;
    my_l[t] = 0.f;
    my_sg[t] = 0.f;
    sg_sum[t] = 0.f;
  }
  for (int r = 0; r < a.k; ++r) {
    unsigned M[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) M[t] = wave_max_u32(key[t][0]);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int win = __builtin_ctzll(__ballot(key[t][0] == M[t]));
      const int e_sel = __builtin_amdgcn_readlane(idx[t][0], win);
      const bool mine = lane == r, me = lane == win;
      my_e[t] = mine ? e_sel : my_e[t];
      my_l[t] = mine ? __uint_as_float(M[t]) : my_l[t];   // the key; decoded below
#pragma unroll
      for (int i = 0; i + 1 < MK; ++i) {
        key[t][i] = me ? key[t][i + 1] : key[t][i];
        idx[t][i] = me ? idx[t][i + 1] : idx[t][i];
      }
      key[t][MK - 1] = me ? 0u : key[t][MK - 1];
    }
  }
  // the k selections' logistic values, in parallel lanes, and their sum
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const float l_sel = unkey(__float_as_uint(my_l[t]));
    const float sg = (lane < a.k) ? __builtin_amdgcn_rcpf(1.0f + __expf(-l_sel)) : 0.0f;
    my_l[t] = l_sel;
    my_sg[t] = sg;
    float sum = sg;
    if (a.k <= 16) {
      sum = group_sum(sum, 16);
      sg_sum[t] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sum)));
    } else {
      sg_sum[t] = wave_sum(sum);
    }
  }
}

// One token's routing weight in lane r < k (its r-th selection, logit
// my_l, sigmoid my_sg; sg_sum the sum of the k sigmoids) and shared
// coefficient in lane s < S, from its logits l.
template <class A>
__device__ __forceinline__ void token_weights(const A& a, const float* l, int lane, float my_l, float my_sg,
                                              float sg_sum, float& wv, float& shc) {
  if (a.route == MOE_ROUTE_SOFTMAX_SINK) {
    unsigned mk = 0u;
    for (int e = lane; e < a.Er; e += 64) mk = max(mk, fkey(l[e]));
    const float mx = unkey(wave_max_u32(mk));
    float z = 0.f;
    for (int e = lane; e < a.Er; e += 64) z += __expf(l[e] - mx);
    z = wave_sum(z);
    wv = __expf(my_l - mx) / z;
    shc = (lane < a.S) ? __expf(l[a.E + min(lane, a.S - 1)] - mx) / z : 0.f;
  } else {
    wv = my_sg * __builtin_amdgcn_rcpf(sg_sum);
    shc = 1.0f;
  }
}

