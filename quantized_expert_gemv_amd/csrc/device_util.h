// Device helpers of the MoE decode kernel (gfx950): bf16 and e2m1/e4m3
// conversions, dot products, DPP lane-permute encodings, sortable keys.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

enum { WT_NVFP4 = 0, WT_BF16 = 1 };

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32); a NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values as one packed bf16 pair (lo in the low half): one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// The same sum as one 8-long chain: half the accumulator set-up of dot8.
// The NVFP4 chunks use it; four chunks per item keep eight chains in flight.
template <int OFF>
__device__ __forceinline__ float dot8c(const uint32_t* w, const uint32_t* x) {
  float p = dot2(w[OFF], x[OFF], 0.f);
#pragma unroll
  for (int i = 1; i < 8; ++i) p = dot2(w[OFF + i], x[OFF + i], p);
  return p;
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

// xhat pair = bf16(x * rn * gamma) elementwise on a packed bf16 pair.
__device__ __forceinline__ uint32_t norm_pair(uint32_t xv, uint32_t gv, float rn) {
  const float lo = (bf16lo(xv) * rn) * bf16lo(gv);
  const float hi = (bf16hi(xv) * rn) * bf16hi(gv);
  return pack_bf16x2(lo, hi);
}

}  // namespace moe
