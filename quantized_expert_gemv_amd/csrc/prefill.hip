// Prefill / large-batch MoE layer for MI355X (gfx950): T tokens through the
// same layer as the decode kernels (router GEMV, sigmoid top-k, NVFP4 gate/up
// with SiLU*up, down, weighted combine), as grouped GEMMs on the matrix cores.
//
// The Flint page ("From 1,096 kernels to 346") counts the MoE kernel work as
// the largest prefill gain; the SM120 page ("How it fits") replaces a
// [tokens * top_k, hidden] fp32 scatter buffer and its weighted temporary by a
// direct gather/reduce.  Here, in six launches on one stream:
//
//   k_pf_route    16 tokens per workgroup: the rows (pre-norm), the router
//                 logits on MFMA (bf16 x bf16 -> fp32), the top-k and weights.
//   k_pf_count    one workgroup per expert: its number of (token, slot) pairs.
//   k_pf_place    one workgroup per expert: its pairs in token order, as the
//                 expert's rows of the sorted list (perm) and the inverse map
//                 (inv); workgroup 0 also writes the group and tile offsets.
//   k_pf_gateup   one workgroup per (32-row tile of a group, 64 intermediates):
//                 the group's tokens' xhat rows staged in shared memory, the
//                 expert's gate and up rows decoded in registers; h = SiLU(g)*u
//                 in bf16 at the tile's sorted rows.  A group is an expert's
//                 sorted rows, or all T tokens for a shared expert.
//   k_pf_down     one workgroup per (32-row tile, 128 outputs): y = W2 h in
//                 fp32 at the same sorted rows.
//   k_pf_combine  one workgroup per token: out = sum over its shared then its
//                 routed slots (selection order) of coef * tensor scale * y,
//                 gathered through inv (+ residual), one bf16 rounding.
//
// The NVFP4 products e2m1 * bf16 are exact in the matrix core's fp32 sums;
// each 16-column block gets its own MFMA (16x16x16) so that its e4m3 scale
// multiplies the block's partial sum, as the decode kernels do.  Every sum
// has a fixed order: the result does not depend on scheduling.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfThreads = 256;   // four waves
constexpr int kRouteTok = 16;     // tokens per routing workgroup (one MFMA row block)
constexpr int kTileTok = 32;      // rows per gate/up and down tile (two MFMA row blocks)
constexpr int kSlice = 512;       // K columns staged in shared memory at a time
constexpr int kSlicePad = kSlice + 8;   // row stride in bf16: 16 B of padding spreads the rows over the banks
constexpr int kGuCols = 64;       // intermediates per gate/up workgroup (16 per wave)
constexpr int kDnCols = 128;      // outputs per down workgroup (32 per wave)

__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ s16x4_t as_s16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
}

// The 4 + 4 weights lane group kb (= lane / 16) feeds to the MFMA from one
// 32-column NVFP4 chunk: columns 4 kb .. 4 kb + 3 of each 16-column block
// (b[0]: block 0, b[1]: block 1), as bf16 (codes unscaled, exact).
__device__ __forceinline__ void chunk_frags(const uint4& c, int kb, s16x4_t (&b)[2]) {
  const int sh = (kb & 1) << 4;
  const uint32_t d0 = ((kb & 2) ? c.y : c.x) >> sh;
  const uint32_t d1 = ((kb & 2) ? c.w : c.z) >> sh;
  b[0] = as_s16x4(fp4pair<0>(d0), fp4pair<1>(d0));
  b[1] = as_s16x4(fp4pair<0>(d1), fp4pair<1>(d1));
}

// Block scales (e4m3) of chunk cc of row `row` of a matrix with geometry g.
__device__ __forceinline__ uint32_t scale_word_off(const MatGeom& g, int row, int cc) {
  const int t = row / g.rpw, ri = row - t * g.rpw;
  return (uint32_t)((t >> 1) * g.su + ri * g.cw + cc) * 4u;
}
__device__ __forceinline__ uint32_t scale_half(const MatGeom& g, int row) { return ((row / g.rpw) & 1) << 4; }

// ---------------------------------------------------------------- routing
__global__ __launch_bounds__(kPfThreads) void k_pf_route(PrefillArgs a) {
  // xhat rows [16][H] (+ one 16-byte unit of padding per row) and the logits
  __shared__ uint4 xs[kRouteTok * (kPfMaxH / 8 + 1)];
  __shared__ float lg[kRouteTok][kPfMaxE];
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTok;
  const int H = a.H, upr = H / 8, ups = upr + 1;   // 16-byte units per row, row stride in units
  for (int u = (int)threadIdx.x; u < kRouteTok * upr; u += kPfThreads) {
    const int m = u / upr, q = u - m * upr, t = t0 + m;
    xs[m * ups + q] = t < a.T ? ld16(a.x + (size_t)t * H + q * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  if (a.prenorm) {
    // wave w normalises rows 4w .. 4w + 3 and writes them to xhat for the gate/up GEMM
    for (int i = 0; i < kRouteTok / 4; ++i) {
      const int m = 4 * wave + i, t = t0 + m;
      float ss = 0.f;
      for (int q = lane; q < upr; q += 64) {
        const uint4 v = xs[m * ups + q];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ss = fmaf(bf16lo(d[j]), bf16lo(d[j]), ss);
          ss = fmaf(bf16hi(d[j]), bf16hi(d[j]), ss);
        }
      }
      const float rn = 1.0f / sqrtf(wave_sum(ss) / (float)H + a.eps);
      for (int q = lane; q < upr; q += 64) {
        const uint4 v = xs[m * ups + q];
        const uint4 gm = ld16(a.gamma + q * 8);
        const uint4 o = make_uint4(norm_pair(v.x, gm.x, rn), norm_pair(v.y, gm.y, rn), norm_pair(v.z, gm.z, rn),
                                   norm_pair(v.w, gm.w, rn));
        xs[m * ups + q] = o;
        if (t < a.T) *reinterpret_cast<uint4*>(a.xhat + (size_t)t * H + q * 8) = o;
      }
    }
    __syncthreads();
  }
  // logits: wave w takes experts [64 w, 64 w + 64) as four 16-expert tiles;
  // lane (m = lane % 16, kb = lane / 16) feeds row m and columns 8 kb .. 8 kb + 7
  // of each 32-column step
  const int mi = lane & 15, kb = lane >> 4;
  f32x4_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int e_base = 64 * wave;
  if (e_base < a.E) {
    const int ntiles = min(4, (a.E - e_base) / 16);
    for (int c = 0; c < H / 32; ++c) {
      const uint4 av = xs[mi * ups + 4 * c + kb];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt < ntiles) {
          const uint4 bv = ld16(a.router_w + (size_t)(e_base + 16 * nt + mi) * H + 32 * c + 8 * kb);
          acc[nt] = mfma32(av, bv, acc[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt < ntiles) {
        const int e = e_base + 16 * nt + mi;
        const float bias = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[4 * kb + r][e] = acc[nt][r] + bias;
      }
    }
  }
  __syncthreads();
  // top-k of rows 4w .. 4w + 3: lane l holds experts 4 l .. 4 l + 3, sorted;
  // each round the largest head key wins (ties to the lowest expert)
  for (int i = 0; i < kRouteTok / 4; ++i) {
    const int m = 4 * wave + i, t = t0 + m;
    if (t >= a.T) break;
    unsigned key[4];
    int idx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      idx[j] = 4 * lane + j;
      key[j] = idx[j] < a.E ? sel_key(lg[m][idx[j]]) : 0u;
    }
    cas(key[0], idx[0], key[1], idx[1]);
    cas(key[2], idx[2], key[3], idx[3]);
    cas(key[0], idx[0], key[2], idx[2]);
    cas(key[1], idx[1], key[3], idx[3]);
    cas(key[1], idx[1], key[2], idx[2]);
    int my_e = 0;
    unsigned my_key = 0u;
    for (int r = 0; r < a.k; ++r) {
      const unsigned M = wave_max_u32(key[0]);
      const int win = __builtin_ctzll(__ballot(key[0] == M));
      const int e_sel = __builtin_amdgcn_readlane(idx[0], win);
      my_e = (lane == r) ? e_sel : my_e;
      my_key = (lane == r) ? M : my_key;
      const bool me = lane == win;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        key[j] = me ? key[j + 1] : key[j];
        idx[j] = me ? idx[j + 1] : idx[j];
      }
      key[3] = me ? 0u : key[3];
    }
    // weights: each selection's logistic value over their sum
    const float sg = (lane < a.k) ? __builtin_amdgcn_rcpf(1.0f + __expf(-unkey(my_key))) : 0.0f;
    const float sum = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(group_sum(sg, 16))));
    const float wgt = sg * __builtin_amdgcn_rcpf(sum);
    if (lane < a.k) {
      a.ids[(size_t)t * a.k + lane] = my_e;
      a.wts[(size_t)t * a.k + lane] = wgt;
      if (a.out_ids) a.out_ids[(size_t)t * a.k + lane] = my_e;
      if (a.out_w) a.out_w[(size_t)t * a.k + lane] = wgt;
    }
  }
}

// ---------------------------------------------------------------- grouping
__device__ __forceinline__ int block_sum_int(int v, int* red) {
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const int s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(kPfThreads) void k_pf_count(PrefillArgs a) {
  __shared__ int red[4];
  const int e = blockIdx.x, n = a.T * a.k;
  int c = 0;
  for (int i = (int)threadIdx.x; i < n; i += kPfThreads) c += a.ids[i] == e;
  c = block_sum_int(c, red);
  if (threadIdx.x == 0) a.counts[e] = c;
}

__global__ __launch_bounds__(kPfThreads) void k_pf_place(PrefillArgs a) {
  __shared__ int red[4];
  __shared__ int wsum[4];
  __shared__ int tiles[kPfMaxE + MOE_MAX_SHARED + 1];
  const int e = blockIdx.x, wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int n = a.T * a.k;
  // the expert's first row: the pairs of every lower expert
  int below = 0;
  for (int i = (int)threadIdx.x; i < e; i += kPfThreads) below += a.counts[i];
  const int off = block_sum_int(below, red);
  if (e == 0) {
    // group offsets (rows) and tile offsets; the shared groups' rows follow
    // the routed pairs, one group of T rows per shared expert
    for (int i = (int)threadIdx.x; i < a.E; i += kPfThreads) tiles[i] = a.counts[i];
    __syncthreads();
    if (threadIdx.x == 0) {
      int rows = 0, tl = 0;
      for (int g = 0; g < a.E; ++g) {
        a.offs[g] = rows;
        a.tile_off[g] = tl;
        rows += tiles[g];
        tl += (tiles[g] + kTileTok - 1) / kTileTok;
      }
      for (int s = 0; s < a.S; ++s) {
        a.offs[a.E + s] = rows;
        a.tile_off[a.E + s] = tl;
        rows += a.T;
        tl += (a.T + kTileTok - 1) / kTileTok;
      }
      a.offs[a.E + a.S] = rows;
      a.tile_off[a.E + a.S] = tl;
    }
  }
  // the expert's pairs in token order: a block-wide stable compaction
  int run = 0;
  for (int base = 0; base < n; base += kPfThreads) {
    const int i = base + (int)threadIdx.x;
    const bool hit = i < n && a.ids[i] == e;
    const unsigned long long b = __ballot(hit);
    const int before_lane = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(b);
    __syncthreads();
    int before_wave = 0;
    for (int w = 0; w < wave; ++w) before_wave += wsum[w];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (hit) {
      const int p = off + run + before_wave + before_lane;
      a.perm[p] = i;
      a.inv[i] = p;
    }
    run += total;
    __syncthreads();
  }
}

// The group of tile `tile`: binary search of the tile offsets (in shared memory).
__device__ __forceinline__ int group_of(const int* toff, int ng, int tile) {
  int lo = 0, hi = ng - 1;   // toff[lo] <= tile < toff[ng]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct TileRows {
  int g;       // group: routed expert g < E, else shared expert g - E
  int r0;      // first row of the tile within the group
  int nrows;   // valid rows of the tile (<= kTileTok)
  int row0;    // sorted row of the tile's first row (rows are consecutive)
};

// The tile this workgroup takes, or g = -1 past the last tile.
__device__ __forceinline__ TileRows tile_rows(const PrefillArgs& a, int* toff_s) {
  const int ng = a.E + a.S;
  for (int i = (int)threadIdx.x; i <= ng; i += kPfThreads) toff_s[i] = a.tile_off[i];
  __syncthreads();
  TileRows tr;
  const int tile = blockIdx.x;
  if (tile >= toff_s[ng]) {
    tr.g = -1;
    return tr;
  }
  tr.g = group_of(toff_s, ng, tile);
  tr.r0 = (tile - toff_s[tr.g]) * kTileTok;
  const int size = tr.g < a.E ? a.counts[tr.g] : a.T;
  tr.nrows = min(kTileTok, size - tr.r0);
  tr.row0 = a.offs[tr.g] + tr.r0;
  return tr;
}

// ---------------------------------------------------------------- gate/up
__global__ __launch_bounds__(kPfThreads) void k_pf_gateup(PrefillArgs a) {
  __shared__ uint16_t xs[kTileTok * kSlicePad];
  __shared__ int toff_s[kPfMaxE + MOE_MAX_SHARED + 1];
  __shared__ int tok_s[kTileTok];
  const TileRows tr = tile_rows(a, toff_s);
  if (tr.g < 0) return;
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int mi = lane & 15, kb = lane >> 4;
  const bool routed = tr.g < a.E;
  if (threadIdx.x < kTileTok) {
    const int r = (int)threadIdx.x;
    tok_s[r] = r >= tr.nrows ? -1 : routed ? a.perm[tr.row0 + r] / a.k : tr.r0 + r;
  }
  const uint8_t* codes = routed ? a.r_codes + (size_t)tr.g * a.r_code_stride
                                : a.s_codes + (size_t)(tr.g - a.E) * a.s_code_stride;
  const uint8_t* scales = routed ? a.r_scales + (size_t)tr.g * a.r_scale_stride
                                 : a.s_scales + (size_t)(tr.g - a.E) * a.s_scale_stride;
  const float ts13 = routed ? a.r_tscale[2 * tr.g] : a.s_tscale[2 * (tr.g - a.E)];
  const MatGeom& g = a.g13;
  const int j = blockIdx.y * kGuCols + 16 * wave + mi;   // this lane's intermediate (weight rows j and I + j)
  const uint32_t crow_g = (uint32_t)j * g.cw, crow_u = (uint32_t)(a.I + j) * g.cw;
  const uint32_t sh_g = scale_half(g, j), sh_u = scale_half(g, a.I + j);
  const uint16_t* xsrc = a.prenorm ? a.xhat : a.x;
  f32x4_t accg[2], accu[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int slice = min(kSlice, a.H);
  for (int k0 = 0; k0 < a.H; k0 += slice) {
    __syncthreads();   // tok_s written; the previous slice consumed
    // the tile's rows, columns k0 .. k0 + slice, 16 bytes per thread and step
    const int ups = slice / 8;
    for (int u = (int)threadIdx.x; u < kTileTok * ups; u += kPfThreads) {
      const int m = u / ups, q = u - m * ups, t = tok_s[m];
      const uint4 v = t >= 0 ? ld16(xsrc + (size_t)t * a.H + k0 + q * 8) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&xs[m * kSlicePad + q * 8]) = v;
    }
    __syncthreads();
    const int c0 = k0 / 32;
    for (int cs = 0; cs < slice / 32; cs += 4) {
      uint4 cg[4], cu[4];
      uint32_t sg[4], su[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = c0 + cs + q;
        cg[q] = ld16o(codes, (crow_g + cc) * 16u);
        cu[q] = ld16o(codes, (crow_u + cc) * 16u);
        sg[q] = ld32o(scales, scale_word_off(g, j, cc)) >> sh_g;
        su[q] = ld32o(scales, scale_word_off(g, a.I + j, cc)) >> sh_u;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s16x4_t bg[2], bu[2];
        chunk_frags(cg[q], kb, bg);
        chunk_frags(cu[q], kb, bu);
        const float g0 = e4m3f<0>(sg[q]), g1 = e4m3f<1>(sg[q]);
        const float u0 = e4m3f<0>(su[q]), u1 = e4m3f<1>(su[q]);
        const int col = 32 * (cs + q);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint16_t* xr = &xs[(16 * mt + mi) * kSlicePad + col + 4 * kb];
          const uint2 a0 = *reinterpret_cast<const uint2*>(xr);
          const uint2 a1 = *reinterpret_cast<const uint2*>(xr + 16);
          const s16x4_t x0 = __builtin_bit_cast(s16x4_t, a0), x1 = __builtin_bit_cast(s16x4_t, a1);
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          const f32x4_t pg0 = mfma16(x0, bg[0], z), pg1 = mfma16(x1, bg[1], z);
          const f32x4_t pu0 = mfma16(x0, bu[0], z), pu1 = mfma16(x1, bu[1], z);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            accg[mt][r] = fmaf(pg1[r], g1, fmaf(pg0[r], g0, accg[mt][r]));
            accu[mt][r] = fmaf(pu1[r], u1, fmaf(pu0[r], u0, accu[mt][r]));
          }
        }
      }
    }
  }
  // h = SiLU(g) * u at the tile's sorted rows; lane holds rows 16 mt + 4 kb + r, intermediate j
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * kb + r;
      if (m < tr.nrows) {
        const float hv = silu_mul(accg[mt][r] * ts13, accu[mt][r] * ts13);
        a.h[(size_t)(tr.row0 + m) * a.I + j] = (uint16_t)f2bf(hv);
      }
    }
  }
}

// ---------------------------------------------------------------- down
__global__ __launch_bounds__(kPfThreads) void k_pf_down(PrefillArgs a) {
  __shared__ uint16_t hs[kTileTok * kSlicePad];
  __shared__ int toff_s[kPfMaxE + MOE_MAX_SHARED + 1];
  const TileRows tr = tile_rows(a, toff_s);
  if (tr.g < 0) return;
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int mi = lane & 15, kb = lane >> 4;
  const bool routed = tr.g < a.E;
  const uint8_t* codes = routed ? a.r_codes + (size_t)tr.g * a.r_code_stride + a.r_w13_code
                                : a.s_codes + (size_t)(tr.g - a.E) * a.s_code_stride + a.s_w13_code;
  const uint8_t* scales = routed ? a.r_scales + (size_t)tr.g * a.r_scale_stride + a.r_w13_scale
                                 : a.s_scales + (size_t)(tr.g - a.E) * a.s_scale_stride + a.s_w13_scale;
  const MatGeom& g = a.g2;
  int n[2];
  uint32_t crow[2], sh[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    n[nt] = blockIdx.y * kDnCols + 32 * wave + 16 * nt + mi;   // output (W2 row) of this lane
    crow[nt] = (uint32_t)n[nt] * g.cw;
    sh[nt] = scale_half(g, n[nt]);
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int slice = min(kSlice, a.I);
  for (int k0 = 0; k0 < a.I; k0 += slice) {
    __syncthreads();
    const int ups = slice / 8;
    for (int u = (int)threadIdx.x; u < kTileTok * ups; u += kPfThreads) {
      const int m = u / ups, q = u - m * ups;
      const uint4 v = m < tr.nrows ? ld16(a.h + (size_t)(tr.row0 + m) * a.I + k0 + q * 8) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&hs[m * kSlicePad + q * 8]) = v;
    }
    __syncthreads();
    const int c0 = k0 / 32;
    for (int cs = 0; cs < slice / 32; cs += 2) {
      uint4 cw[2][2];
      uint32_t sw[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int cc = c0 + cs + q;
          cw[q][nt] = ld16o(codes, (crow[nt] + cc) * 16u);
          sw[q][nt] = ld32o(scales, scale_word_off(g, n[nt], cc)) >> sh[nt];
        }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = 32 * (cs + q);
        s16x4_t xa[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint16_t* hr = &hs[(16 * mt + mi) * kSlicePad + col + 4 * kb];
          xa[mt][0] = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const uint2*>(hr));
          xa[mt][1] = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const uint2*>(hr + 16));
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          s16x4_t b[2];
          chunk_frags(cw[q][nt], kb, b);
          const float s0 = e4m3f<0>(sw[q][nt]), s1 = e4m3f<1>(sw[q][nt]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t p0 = mfma16(xa[mt][0], b[0], z), p1 = mfma16(xa[mt][1], b[1], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nt][mt][r] = fmaf(p1[r], s1, fmaf(p0[r], s0, acc[nt][mt][r]));
          }
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * kb + r;
        if (m < tr.nrows) a.y[(size_t)(tr.row0 + m) * a.H + n[nt]] = acc[nt][mt][r];
      }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(kPfThreads) void k_pf_combine(PrefillArgs a) {
  // coefficient * W2 tensor scale and sorted row of each term: shared experts
  // first, then the routed slots in selection order
  __shared__ float coef[MOE_MAX_SHARED + MOE_MAX_TOPK];
  __shared__ int row[MOE_MAX_SHARED + MOE_MAX_TOPK];
  const int t = blockIdx.x;
  const int kk = a.k, S = a.S;
  const int m = (int)threadIdx.x;
  if (m < S) {
    coef[m] = 1.0f * a.s_tscale[2 * m + 1];
    row[m] = a.offs[a.E + m] + t;
  } else if (m < S + kk) {
    const int j = m - S, e = a.ids[(size_t)t * kk + j];
    coef[m] = a.wts[(size_t)t * kk + j] * a.r_tscale[2 * e + 1];
    row[m] = a.inv[(size_t)t * kk + j];
  }
  __syncthreads();
  for (int c = 8 * (int)threadIdx.x; c < a.H; c += 8 * kPfThreads) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
    for (int m = 0; m < S + kk; ++m) {
      const float4* yp = reinterpret_cast<const float4*>(a.y + (size_t)row[m] * a.H + c);
      const float4 v0 = yp[0], v1 = yp[1];
      const float y8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(coef[m], y8[i], o[i]);
    }
    if (a.residual) {
      const uint4 xv = ld16(a.x + (size_t)t * a.H + c);
      const uint32_t d[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16lo(d[i]);
        o[2 * i + 1] += bf16hi(d[i]);
      }
    }
    uint4 ov;
    ov.x = pack_bf16x2(o[0], o[1]);
    ov.y = pack_bf16x2(o[2], o[3]);
    ov.z = pack_bf16x2(o[4], o[5]);
    ov.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(a.out + (size_t)t * a.H + c) = ov;
  }
}

}  // namespace

int prefill_max_tiles(int T, int k, int E, int S) {
  return (T * k + kTileTok - 1) / kTileTok + E + S * ((T + kTileTok - 1) / kTileTok);
}

int launch_prefill(const PrefillArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int tiles = prefill_max_tiles(a.T, a.k, a.E, a.S);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_pf_route, dim3((a.T + kRouteTok - 1) / kRouteTok), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_count, dim3(a.E), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_place, dim3(a.E), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_gateup, dim3(tiles, a.I / kGuCols), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_down, dim3(tiles, a.H / kDnCols), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_combine, dim3(a.T), dim3(kPfThreads), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace moe
