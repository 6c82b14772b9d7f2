// Small-batch dense NVFP4 GEMV for MI355X (gfx950): y[b][n] = sum_k W[n][k] x[b][k]
// for 1-8 bf16 tokens, W packed exactly as the experts' matrices are (Flint page,
// "From 1,096 kernels to 346": a small-batch dense GEMV on the same packed NVFP4
// weights; the attention projections and the dense MLP of layers 0 and 1).
//
// The GEMV reads each weight byte once.  A wave takes one scale-word step
// pair (two wave steps of rpw rows each) and issues its loads at once, so the
// whole matrix is in flight from the start; the workgroup's eight waves share
// x, staged once in shared memory.  Lane (row ri of a step, 32-column chunk
// jj) decodes its chunk once per step and reuses it for every token.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

constexpr int kDnsWaves = 8;
constexpr int kDnsThreads = 64 * kDnsWaves;
constexpr int kDnsPairs = 1;                 // step pairs per wave
constexpr int kDnsMaxChunks = 64;            // cols <= 2048: one wave step covers a row

// Shared-memory position of 16-byte unit q of 64-byte chunk c (the units a
// wave reads in one instruction fall in distinct banks).
__device__ __forceinline__ int dense_unit(int c, int q) { return (c << 2) | (q ^ ((c >> 2) & 3)); }

template <int TB>
__global__ __launch_bounds__(kDnsThreads) void k_dense_gemv(DenseArgs a) {
  __shared__ uint4 xs[TB][kDnsMaxChunks * 4];
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const MatGeom g = a.g;
  const int ri = lane / g.lpr, jj = lane % g.lpr;
  const bool active = jj < g.cw;
  const int jc = active ? jj : 0;
  const uint32_t u = (uint32_t)(ri * g.cw + jc);
  const int pair0 = (blockIdx.x * kDnsWaves + wave) * kDnsPairs;
  const int npairs = g.nsteps >> 1;
  // this wave's weights first (a wave past the end loads its last pair again:
  // the same instructions, valid addresses; its results are not written)
  uint4 c[kDnsPairs][2];
  uint32_t sw[kDnsPairs];
#pragma unroll
  for (int p = 0; p < kDnsPairs; ++p) {
    const int pr = min(pair0 + p, npairs - 1);
#pragma unroll
    for (int st = 0; st < 2; ++st) c[p][st] = ld16o(a.codes, ((uint32_t)(2 * pr + st) * g.su + u) * 16u);
    sw[p] = ld32o(a.scales, ((uint32_t)pr * g.su + u) * 4u);
  }
  const float ts = *a.tscale;
  // then x of every token, staged once for the workgroup: all loads first,
  // then the stores (a load-store loop would wait for each load in turn)
  const int units = g.C * 4;   // 16-byte units per token, <= 256
  uint4 xv[TB];
#pragma unroll
  for (int k = 0; k < TB; ++k) {
    const int i = (int)threadIdx.x + kDnsThreads * k, b = i / units, r = i - b * units;
    xv[k] = ld16(a.x + (size_t)min(b, a.B - 1) * g.cols + (size_t)r * 8);
  }
#pragma unroll
  for (int k = 0; k < TB; ++k) {
    const int i = (int)threadIdx.x + kDnsThreads * k, b = i / units, r = i - b * units;
    if (b < a.B) xs[b][dense_unit(r >> 2, r & 3)] = xv[k];
  }
  __syncthreads();
  uint32_t xk[TB][16];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack4(xs[b][dense_unit(jc, q)], &xk[b][4 * q]);
#pragma unroll
  for (int p = 0; p < kDnsPairs; ++p) {
    if (pair0 + p >= npairs) break;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t wd[16];
      decode_chunk(c[p][st], wd);
      const uint32_t sp = st ? (sw[p] >> 16) : sw[p];
      const float s0 = e4m3f<0>(sp) * ts, s1 = e4m3f<1>(sp) * ts;
      const int row = (2 * (pair0 + p) + st) * g.rpw + ri;
      float v[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        float lo = dot2(wd[0], xk[b][0], 0.f), hi = dot2(wd[8], xk[b][8], 0.f);
#pragma unroll
        for (int k = 1; k < 8; ++k) {
          lo = dot2(wd[k], xk[b][k], lo);
          hi = dot2(wd[8 + k], xk[b][8 + k], hi);
        }
        v[b] = active ? fmaf(hi, s1, lo * s0) : 0.f;
      }
#pragma unroll
      for (int b = 0; b < TB; ++b) v[b] = group_sum(v[b], g.lpr);
      // the row's sum is in its group's last lane
      if (jj == g.lpr - 1 && row < a.rows) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
          if (b < a.B) a.y[(size_t)b * a.rows + row] = (uint16_t)f2bf(v[b]);
      }
    }
  }
}

}  // namespace

int dense_grid(const MatGeom& g) {
  const int npairs = g.nsteps >> 1;
  const int per = kDnsWaves * kDnsPairs;
  return (npairs + per - 1) / per;
}

int launch_dense(const DenseArgs& a, void* stream) {
  if (a.g.ns != 1 || a.g.C > kDnsMaxChunks || a.B < 1 || a.B > MOE_MAX_BATCH) return (int)hipErrorInvalidValue;
  const int tb = a.B <= 1 ? 1 : a.B <= 2 ? 2 : a.B <= 4 ? 4 : 8;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(dense_grid(a.g)), block(kDnsThreads);
  (void)hipGetLastError();
  switch (tb) {
    case 1: hipLaunchKernelGGL(k_dense_gemv<1>, grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_dense_gemv<2>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(k_dense_gemv<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(k_dense_gemv<8>, grid, block, 0, st, a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace moe
