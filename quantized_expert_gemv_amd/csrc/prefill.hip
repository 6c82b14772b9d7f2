// Prefill / large-batch MoE layer for MI355X (gfx950): T tokens through the
// same layer as the decode kernels (router GEMV, sigmoid top-k, NVFP4 or
// 2-bit gate/up with SiLU*up, down, weighted combine), as grouped GEMMs on the
// matrix cores.
//
// The Flint page ("From 1,096 kernels to 346") counts the MoE kernel work as
// the largest prefill gain; the SM120 page ("How it fits") replaces a
// [tokens * top_k, hidden] fp32 scatter buffer and its weighted temporary by a
// direct gather/reduce.  Here, in seven launches on one stream:
//
//   k_pf_logits   16 tokens x one or more blocks of 64 experts per workgroup:
//                 the rows (pre-norm), the router logits on MFMA (bf16 x bf16
//                 -> fp32).
//   k_pf_topk     one wave per token: the top-k and weights.
//   k_pf_count    one workgroup per expert: its number of (token, slot) pairs
//                 (and each scanning wave's share).
//   k_pf_place    one workgroup per expert: its pairs in token order, as the
//                 expert's rows of the sorted list (perm) and the inverse map
//                 (inv); workgroup 0 also writes the group and tile offsets.
//   k_pf_gateup   one workgroup per (tile of a group's rows, 64 intermediates):
//                 the tile's xhat rows and the expert's gate and up rows staged
//                 slice by slice in shared memory (2-bit codes widened to e2m1
//                 there); h = SiLU(g)*u in bf16 at the tile's sorted rows.  A
//                 group is an expert's sorted rows, or all T tokens for a shared
//                 expert; a tile is 64 rows, or 128 when the call's routed
//                 groups average 128 rows or more.
//   k_pf_down     one workgroup per (tile, 128 outputs): y = W2 h in fp32 at
//                 the same sorted rows.
//   k_pf_combine  one workgroup per token: out = sum over its shared then its
//                 routed slots (selection order) of coef * tensor scale * y,
//                 gathered through inv (+ residual), one bf16 rounding.
//
// The weights reach the matrix cores (MFMA 16x16x32 bf16, fp32 sums) as
// e2m1 code times e4m3 block scale, which bf16 holds exactly; the fp32
// tensor scale multiplies the finished sums.  Every sum
// has a fixed order: the result does not depend on scheduling.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

#include "device_util.h"

namespace moe {
namespace {

#include "kernel_common.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfThreads = 256;   // four waves
constexpr int kRouteTok = 16;     // tokens per routing workgroup (one MFMA row block)
constexpr int kTileTok = 128;     // rows per gate/up and down tile at most
// A call's tiles hold a.tile_rows rows (64, or 128 when the routed groups
// average 128 rows or more); a tile of more than 64 rows runs as 8 MFMA row
// blocks, a shorter one as 4.

// Tiles of a group of c rows.
__device__ __forceinline__ int group_tiles(int c, int rows) { return (c + rows - 1) / rows; }
constexpr int kSliceShort = 256;  // K columns staged in shared memory at a time, tiles of <= 64 rows
constexpr int kSliceLong = 128;   // and of more (at most: K = I may be shorter in the down GEMM)
constexpr int kGuCols = 64;       // intermediates per gate/up workgroup (16 per wave)
constexpr int kDnCols = 128;      // outputs per down workgroup (32 per wave)

__device__ __forceinline__ f32x4_t mfma32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ---------------------------------------------------------------- routing
// Logits: workgroup (token block, y) takes 16 tokens and the blocks of 64
// experts y, y + Y, ... (Y = gridDim.y: the fewer, the fewer times a token's
// row is read; the host keeps >= ~1024 workgroups); wave w the 16 experts at
// 16 w of each block.  The 16 rows (pre-normed if the layer has a pre-norm;
// workgroups of y = 0 write them to xhat) sit in shared memory;
// lane (m = lane % 16, kb = lane / 16) feeds row m and columns 8 kb .. + 8 of
// each 32-column step, router rows stream from memory 8 steps at a time
// (the next 8 in flight while these 8 multiply).
constexpr int kLogitSteps = 8;

__global__ __launch_bounds__(kPfThreads) void k_pf_logits(PrefillArgs a) {
  __shared__ uint4 xs[kRouteTok * (kPfMaxH / 8 + 1)];
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTok;
  const int H = a.H, upr = H / 8, ups = upr + 1;   // 16-byte units per row; row stride (+1: banks)
  {
    // all of this thread's loads first, then the stores: one round trip
    constexpr int kXU = kRouteTok * kPfMaxH / 8 / kPfThreads;
    uint4 xv[kXU];
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, m = u / upr, q = u - m * upr, t = t0 + m;
      xv[i] = (u < kRouteTok * upr && t < a.T) ? ld16(a.x + (size_t)t * H + q * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, m = u / upr, q = u - m * upr;
      if (u < kRouteTok * upr) xs[m * ups + q] = xv[i];
    }
  }
  __syncthreads();
  if (a.prenorm) {
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
        if (blockIdx.y == 0 && t < a.T) *reinterpret_cast<uint4*>(a.xhat + (size_t)t * H + q * 8) = o;
      }
    }
    __syncthreads();
  }
  const int mi = lane & 15, kb = lane >> 4;
  for (int e0 = 64 * blockIdx.y + 16 * wave; e0 < a.E; e0 += 64 * gridDim.y) {   // the wave's 16-expert blocks
  const uint16_t* rrow = a.router_w + (size_t)(e0 + mi) * H + 8 * kb;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // two sets of router steps: one set's loads fly while the other's products run
  const int nc = H / 32;
  uint4 b0[kLogitSteps], b1[kLogitSteps];
  const auto load = [&](uint4(&bv)[kLogitSteps], int c) {
#pragma unroll
    for (int i = 0; i < kLogitSteps; ++i) bv[i] = ld16(rrow + 32 * (c + i));
  };
  const auto mma = [&](const uint4(&bv)[kLogitSteps], int c) {
#pragma unroll
    for (int i = 0; i < kLogitSteps; ++i) acc = mfma32(xs[mi * ups + 4 * (c + i) + kb], bv[i], acc);
  };
  load(b0, 0);
  for (int c = 0; c < nc; c += 2 * kLogitSteps) {
    if (c + kLogitSteps < nc) load(b1, c + kLogitSteps);
    mma(b0, c);
    if (c + kLogitSteps >= nc) break;
    if (c + 2 * kLogitSteps < nc) load(b0, c + 2 * kLogitSteps);
    mma(b1, c + kLogitSteps);
  }
  const int e = e0 + mi;
  const float bias = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * kb + r;
    if (t < a.T) a.logits[(size_t)t * a.E + e] = acc[r] + bias;
  }
  }
}

// Top-k and weights: one wave per token.  Lane l holds experts 4 l .. 4 l + 3,
// sorted; each round the largest head key wins (ties to the lowest expert),
// the decode kernels' rule; weights are the selections' logistic values over
// their sum.
__global__ __launch_bounds__(kPfThreads) void k_pf_topk(PrefillArgs a) {
  const int lane = (int)threadIdx.x & 63;
  const int t = blockIdx.x * (kPfThreads / 64) + wave_id();
  if (t >= a.T) return;
  unsigned key[4];
  int idx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    idx[j] = 4 * lane + j;
    key[j] = idx[j] < a.E ? sel_key(a.logits[(size_t)t * a.E + idx[j]]) : 0u;
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

// ---------------------------------------------------------------- grouping
// The selection list ids[T * k] (pair i = token i / k, slot i % k) is read in
// groups of four pairs (16 bytes); wave w of a workgroup takes a contiguous
// quarter of the groups, so the waves' pairs follow each other in list
// order.  A partial last group reads -1 past the end.
__device__ __forceinline__ int4 ids4(const int* ids, int g, int n) {
  if (4 * g + 3 < n) return *reinterpret_cast<const int4*>(ids + 4 * g);
  int4 v = make_int4(-1, -1, -1, -1);
  if (4 * g < n) v.x = ids[4 * g];
  if (4 * g + 1 < n) v.y = ids[4 * g + 1];
  if (4 * g + 2 < n) v.z = ids[4 * g + 2];
  return v;
}
__device__ __forceinline__ int matches4(const int4& v, int e) {
  return (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
}
// Groups [g0, g1) of wave `wave` (4 waves per workgroup).
__device__ __forceinline__ void wave_groups(int n, int wave, int& g0, int& g1) {
  const int ng = (n + 3) >> 2, per = (ng + 3) >> 2;
  g0 = min(ng, wave * per);
  g1 = min(ng, g0 + per);
}
// The wave's number of pairs that selected expert e.
__device__ __forceinline__ int wave_count(const int* ids, int n, int e, int g0, int g1) {
  const int lane = (int)threadIdx.x & 63;
  int c = 0;
  for (int g = g0 + lane; g < g1; g += 4 * 64) {
    int4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ids4(ids, min(g + 64 * u, g1 - 1), n);
#pragma unroll
    for (int u = 0; u < 4; ++u) c += g + 64 * u < g1 ? matches4(v[u], e) : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  return c;
}

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

// counts[e]: the pairs that selected expert e; counts[E + 4 e + w]: those
// among wave w's quarter of the list.
__global__ __launch_bounds__(kPfThreads) void k_pf_count(PrefillArgs a) {
  __shared__ int red[4];
  const int e = blockIdx.x, n = a.T * a.k, wave = wave_id();
  int g0, g1;
  wave_groups(n, wave, g0, g1);
  const int c = wave_count(a.ids, n, e, g0, g1);
  if (((int)threadIdx.x & 63) == 0) {
    red[wave] = c;
    a.counts[a.E + 4 * e + wave] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) a.counts[e] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kPfThreads) void k_pf_place(PrefillArgs a) {
  __shared__ int red[4];
  __shared__ int wsum[8];   // each wave's row and tile totals
  const int e = blockIdx.x, wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int n = a.T * a.k;
  // the expert's first row: the pairs of every lower expert
  int below = 0;
  for (int i = (int)threadIdx.x; i < e; i += kPfThreads) below += a.counts[i];
  const int off = block_sum_int(below, red);
  if (e == 0) {
    // group offsets (rows) and tile offsets: exclusive sums over the routed
    // experts (thread t holds expert t), then the shared groups, T rows each
    const int t = (int)threadIdx.x;
    const int c = t < a.E ? a.counts[t] : 0, nt = group_tiles(c, a.tile_rows);
    int rc = c, rt = nt;   // inclusive sums within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int uc = __shfl_up(rc, o), ut = __shfl_up(rt, o);
      if (lane >= o) {
        rc += uc;
        rt += ut;
      }
    }
    if (lane == 63) {
      wsum[2 * wave] = rc;
      wsum[2 * wave + 1] = rt;
    }
    __syncthreads();
    int bc = 0, bt = 0;   // the waves before this one
    for (int w = 0; w < wave; ++w) {
      bc += wsum[2 * w];
      bt += wsum[2 * w + 1];
    }
    if (t < a.E) {
      a.offs[t] = bc + rc - c;
      a.tile_off[t] = bt + rt - nt;
    }
    if (t == kPfThreads - 1) {   // the last thread's inclusive sums are the totals
      int rows = bc + rc, tl = bt + rt;
      for (int s = 0; s < a.S; ++s) {
        a.offs[a.E + s] = rows;
        a.tile_off[a.E + s] = tl;
        rows += a.T;
        tl += group_tiles(a.T, a.tile_rows);
      }
      a.offs[a.E + a.S] = rows;
      a.tile_off[a.E + a.S] = tl;
    }
  }
  // the expert's pairs in list order: each wave writes the pairs of its
  // quarter after those of the waves before it (the quarters' counts are
  // the counting kernel's)
  int g0, g1;
  wave_groups(n, wave, g0, g1);
  int run = off;
  for (int w = 0; w < wave; ++w) run += a.counts[a.E + 4 * e + w];
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int gb = g0; gb < g1; gb += 4 * 64) {
    int4 v[4];   // four steps' loads in flight at once
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ids4(a.ids, min(gb + 64 * u + lane, g1 - 1), n);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = gb + 64 * u + lane;
      const bool in = g < g1;
      const int m0 = in && v[u].x == e, m1 = in && v[u].y == e, m2 = in && v[u].z == e, m3 = in && v[u].w == e;
      const int cl = m0 + m1 + m2 + m3;   // 0 .. 4
      // matches in the lanes before this one: the three bits of cl, counted
      const unsigned long long b0 = __ballot(cl & 1), b1 = __ballot(cl & 2), b2 = __ballot(cl & 4);
      int p = run + __popcll(b0 & lt) + 2 * __popcll(b1 & lt) + 4 * __popcll(b2 & lt);
      const int i0 = 4 * g;
      if (m0) { a.perm[p] = i0; a.inv[i0] = p; ++p; }
      if (m1) { a.perm[p] = i0 + 1; a.inv[i0 + 1] = p; ++p; }
      if (m2) { a.perm[p] = i0 + 2; a.inv[i0 + 2] = p; ++p; }
      if (m3) { a.perm[p] = i0 + 3; a.inv[i0 + 3] = p; }
      run += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    }
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

// The tile and column block this workgroup takes, or g = -1 past the last
// tile.  Workgroup b runs on XCD b % 8 (workgroups are dealt to the 8 XCDs in
// turn); XCD x takes the tiles [x M, x M + M) of the N tiles of this call
// (M = ceil(N / 8)), in order, each with its ny column blocks back to back.
// A tile's column blocks then share its activation rows in that XCD's L2,
// and the consecutive tiles of one expert share its weight rows there.  The
// grid holds 8 ny workgroups per 8 tiles of the host's bound on N; the rest
// find no tile.
__device__ __forceinline__ TileRows tile_rows(const PrefillArgs& a, int* toff_s, int ny, int& yb) {
  const int ng = a.E + a.S;
  for (int i = (int)threadIdx.x; i <= ng; i += kPfThreads) toff_s[i] = a.tile_off[i];
  __syncthreads();
  const int n = toff_s[ng], per = (n + 7) >> 3;
  const int x = (int)blockIdx.x & 7, i = (int)blockIdx.x >> 3, t = i / ny;
  yb = i - t * ny;
  const int tile = x * per + t;
  TileRows tr;
  if (t >= per || tile >= n) {
    tr.g = -1;
    return tr;
  }
  tr.g = group_of(toff_s, ng, tile);
  const int size = tr.g < a.E ? a.counts[tr.g] : a.T;
  tr.r0 = (tile - toff_s[tr.g]) * a.tile_rows;
  tr.nrows = min(a.tile_rows, size - tr.r0);
  tr.row0 = a.offs[tr.g] + tr.r0;
  return tr;
}

// ---------------------------------------------------------------- gate/up and down
// Both GEMMs run slice by slice over K (SLICE columns, a power of two that
// divides K): the workgroup stages the slice of its 64 activation rows and of
// its 128 weight rows (codes and block scales) in shared memory, every thread
// issuing all of its loads before its first store, so that one memory round
// trip brings the whole slice; each wave then multiplies its rows out of
// shared memory.  The workgroup loads slice i + 1 while it multiplies slice
// i.  Which rows and columns a thread moves does not change from slice to
// slice: the offsets are worked out once, before the first slice.
constexpr int kWRows = 128;                        // weight rows per workgroup
template <int SLICE, int ROWS>
struct __align__(16) GemmSmem {
  static constexpr int kSlice = SLICE, kRows = ROWS;
  static constexpr int kPad = SLICE + 8;           // activation row stride in bf16 (+16 B: banks)
  static constexpr int kWStride = SLICE / 2 + 16;  // bytes per staged weight row (+16 B: banks)
  uint16_t act[ROWS * kPad];                       // activation rows, bf16
  uint8_t wc[kWRows * kWStride];                   // weight codes
  uint16_t wsc[kWRows][SLICE / 32];                // block scale pair (2 x e4m3) per row and chunk
};
using SmemShort = GemmSmem<kSliceShort, 64>;
template <int SLICE>
using SmemLong = GemmSmem<SLICE, 128>;
constexpr int kSmemBytes = sizeof(SmemShort) > sizeof(SmemLong<kSliceLong>) ? sizeof(SmemShort)
                                                                            : sizeof(SmemLong<kSliceLong>);
// The tile's bookkeeping, beside the staging buffers.
struct TileSmem {
  int toff[kPfMaxE + MOE_MAX_SHARED + 1];
  int tok[kTileTok];
};

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// This thread's share of a slice: activation units (16 bytes of one row) and
// weight chunks (16 bytes of codes, 32 columns of one row, with their scale
// pair).  Unit u = tid + 256 i of the slice is row u / (SLICE / 8), 16-byte
// column u % (SLICE / 8); chunk u is local weight row u / (SLICE / 32),
// chunk u % (SLICE / 32).  The counts divide exactly for SLICE = 64, 128, 256.
template <class SM>
struct Stage {
  static constexpr int SLICE = SM::kSlice, ROWS = SM::kRows;
  static constexpr int kAsh = ilog2(SLICE / 8), kNsh = ilog2(SLICE / 32);
  static constexpr int kA = ROWS * SLICE / 8 / kPfThreads;
  static constexpr int kW = kWRows * SLICE / 32 / kPfThreads;
  static_assert(kA * kPfThreads == ROWS * SLICE / 8 && kW * kPfThreads == kWRows * SLICE / 32, "whole units");
  // fixed per workgroup
  uint32_t aoff[kA];     // element offset of the unit's row start + column, from the activation base
  uint32_t avalid;       // bit i: unit i's row holds a token (else it is staged as zeros)
  uint32_t coff[kW];     // byte offset of the chunk's codes at slice 0
  uint32_t soff[kW];     // byte offset of its scale word at slice 0
  uint32_t shi;          // bit i: chunk i's pair is the word's upper half
  bool two;              // the codes are 2-bit planes: 8-byte chunks at half the offsets
  // the slice in flight
  uint4 av[kA], wv[kW];
  uint32_t sv[kW];

  template <class ActRow, class WRow>
  __device__ __forceinline__ void setup(const MatGeom& g, int K, bool two_bit, ActRow&& act_row, WRow&& wrow) {
    const int rsh = __builtin_ctz((unsigned)g.rpw);
    two = two_bit;
    avalid = 0u;
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, m = u >> kAsh, q = u & ((1 << kAsh) - 1);
      const int r = act_row(m);   // row of the activation matrix, or -1
      aoff[i] = r >= 0 ? (uint32_t)r * (uint32_t)K + (uint32_t)(q * 8) : 0u;
      avalid |= (r >= 0 ? 1u : 0u) << i;
    }
    shi = 0u;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, lr = u >> kNsh, q = u & ((1 << kNsh) - 1);
      const int row = wrow(lr), t = row >> rsh, ri = row & ((1 << rsh) - 1);
      coff[i] = (uint32_t)(row * g.cw + q) * 16u;
      soff[i] = (uint32_t)((t >> 1) * g.su + ri * g.cw + q) * 4u;
      shi |= (uint32_t)(t & 1) << i;
    }
  }
  // Every lane loads (a zero row reads the base row and drops it): no branch
  // around the loads, so that they all issue back to back.  The loaded words
  // are not touched until store(): a use right after the loads would make the
  // wave wait for them before it multiplies the slice already staged.
  __device__ __forceinline__ void load(const uint16_t* act, const uint8_t* codes, const uint8_t* scales, int k0) {
#pragma unroll
    for (int i = 0; i < kA; ++i) av[i] = ld16(act + aoff[i] + k0);
    const uint32_t c0 = (uint32_t)(k0 >> 5);
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      if (two) {
        // a slice takes half of each 128-byte line of 2-bit codes and the
        // next slice the other half: a cached load, which the L2 may still
        // hold for the next slice (nontemporal loads were no faster)
        const uint2 v = *reinterpret_cast<const uint2*>(codes + ((coff[i] + c0 * 16u) >> 1));
        wv[i] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        wv[i] = ld16o(codes, coff[i] + c0 * 16u);
      }
      sv[i] = ld32o(scales, soff[i] + c0 * 4u);
    }
  }
  __device__ __forceinline__ void store(SM& s) const {
    constexpr int kPad = SM::kPad, kWStride = SM::kWStride;
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, m = u >> kAsh, q = u & ((1 << kAsh) - 1);
      *reinterpret_cast<uint4*>(&s.act[m * kPad + q * 8]) =
          ((avalid >> i) & 1u) ? av[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const int u = (int)threadIdx.x + kPfThreads * i, lr = u >> kNsh, q = u & ((1 << kNsh) - 1);
      // a 2-bit chunk widens to the e2m1 chunk of the same values here
      *reinterpret_cast<uint4*>(&s.wc[lr * kWStride + q * 16]) = two ? widen_2bit(make_uint2(wv[i].x, wv[i].y)) : wv[i];
      s.wsc[lr][q] = (uint16_t)(sv[i] >> (((shi >> i) & 1u) << 4));
    }
  }
};

// B operand of lane group kb (= lane / 16) from local weight row r, chunk q
// of the staged slice: columns 8 kb .. 8 kb + 7, codes times their block's
// e4m3 scale, as bf16.  Exact: an e2m1 value has at most 2 significant bits
// and an e4m3 scale 4, so the product fits bf16's 8.
template <class SM>
__device__ __forceinline__ uint4 wfrag(const SM& s, int r, int q, int kb) {
  const uint32_t d = *reinterpret_cast<const uint32_t*>(&s.wc[r * SM::kWStride + q * 16 + 4 * kb]);
  const float sc = e4m3f<0>((uint32_t)s.wsc[r][q] >> (kb & 2) * 4);   // block kb / 2 of the chunk
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  return make_uint4(pack_bf16x2(v0.x * sc, v0.y * sc), pack_bf16x2(v1.x * sc, v1.y * sc),
                    pack_bf16x2(v2.x * sc, v2.y * sc), pack_bf16x2(v3.x * sc, v3.y * sc));
}
// A operand of lane (mi, kb) for row block mt, chunk q: activation row
// 16 mt + mi, columns 32 q + 8 kb .. + 8.
template <class SM>
__device__ __forceinline__ uint4 afrag(const SM& s, int mt, int q, int mi, int kb) {
  return *reinterpret_cast<const uint4*>(&s.act[(16 * mt + mi) * SM::kPad + 32 * q + 8 * kb]);
}

// One wave's products over a staged slice of SLICE / 32 chunks: local weight rows
// r0 + mi and r1 + mi (the B operands of lane group kb) against the tile's
// ROWS / 16 row blocks, into acc0 and acc1.  Chunk q + 1's fragments are read
// (and its weights decoded) before chunk q's products are issued, so the
// shared-memory reads and the decoding overlap the matrix cores' work.
template <class SM>
__device__ __forceinline__ void mma_slice(const SM& s, int r0, int r1, int mi, int kb,
                                          f32x4_t (&acc0)[SM::kRows / 16], f32x4_t (&acc1)[SM::kRows / 16]) {
  constexpr int NQ = SM::kSlice / 32, kMT = SM::kRows / 16;
  uint4 av[2][kMT], bv[2][2];
  bv[0][0] = wfrag(s, r0 + mi, 0, kb);
  bv[0][1] = wfrag(s, r1 + mi, 0, kb);
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) av[0][mt] = afrag(s, mt, 0, mi, kb);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = q & 1;
    if (q + 1 < NQ) {
      bv[c ^ 1][0] = wfrag(s, r0 + mi, q + 1, kb);
      bv[c ^ 1][1] = wfrag(s, r1 + mi, q + 1, kb);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) av[c ^ 1][mt] = afrag(s, mt, q + 1, mi, kb);
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      acc0[mt] = mfma32(av[c][mt], bv[c][0], acc0[mt]);
      acc1[mt] = mfma32(av[c][mt], bv[c][1], acc1[mt]);
    }
  }
}

// The group's weights (codes, scales) of matrix `which` (0: W13, 1: W2).
struct GroupW {
  const uint8_t *codes, *scales;
  float ts;
};
__device__ __forceinline__ GroupW group_w(const PrefillArgs& a, int g, int which) {
  const bool routed = g < a.E;
  const int e = routed ? g : g - a.E;
  GroupW w;
  w.codes = (routed ? a.r_codes + (size_t)e * a.r_code_stride : a.s_codes + (size_t)e * a.s_code_stride) +
            (which ? (routed ? a.r_w13_code : a.s_w13_code) : 0);
  w.scales = (routed ? a.r_scales + (size_t)e * a.r_scale_stride : a.s_scales + (size_t)e * a.s_scale_stride) +
             (which ? (routed ? a.r_w13_scale : a.s_w13_scale) : 0);
  w.ts = (routed ? a.r_tscale : a.s_tscale)[2 * e + which];
  return w;
}

// gate/up: workgroup (tile, y) takes intermediates [64 y, 64 y + 64): local
// weight rows 0..63 are their gate rows, 64..127 their up rows; wave w's
// lanes take intermediate 64 y + 16 w + lane % 16.  K = H, a multiple of 256.
template <class SM>
__device__ __forceinline__ void gateup_tile(const PrefillArgs& a, const TileRows& tr, const TileSmem& ts, SM& s,
                                            int yb) {
  constexpr int kMT = SM::kRows / 16, SLICE = SM::kSlice;
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int mi = lane & 15, kb = lane >> 4;
  const GroupW gw = group_w(a, tr.g, 0);
  const int j0 = yb * kGuCols, j = j0 + 16 * wave + mi;
  const uint16_t* xsrc = a.prenorm ? a.xhat : a.x;
  const int H = a.H, I = a.I;
  f32x4_t accg[kMT], accu[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Stage<SM> st;
  st.setup(a.g13, H, a.r2bit && tr.g < a.E, [&](int m) { return ts.tok[m]; },
           [&](int r) { return r < kGuCols ? j0 + r : I + j0 + (r - kGuCols); });
  st.load(xsrc, gw.codes, gw.scales, 0);
  for (int k0 = 0; k0 < H; k0 += SLICE) {
    __syncthreads();   // the previous slice is consumed
    st.store(s);
    __syncthreads();
    if (k0 + SLICE < H) st.load(xsrc, gw.codes, gw.scales, k0 + SLICE);
    mma_slice(s, 16 * wave, kGuCols + 16 * wave, mi, kb, accg, accu);
  }
  // h = SiLU(g) * u at the tile's sorted rows; the lane holds rows 16 mt + 4 kb + i
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * mt + 4 * kb + i;
      if (m < tr.nrows)
        a.h[(size_t)(tr.row0 + m) * I + j] = (uint16_t)f2bf(silu_mul(accg[mt][i] * gw.ts, accu[mt][i] * gw.ts));
    }
}

template <bool LONG>
__global__ __launch_bounds__(kPfThreads) void k_pf_gateup(PrefillArgs a) {
  __shared__ TileSmem ts;
  __shared__ __align__(16) uint8_t raw[kSmemBytes];
  int yb;
  const TileRows tr = tile_rows(a, ts.toff, a.I / kGuCols, yb);
  if (tr.g < 0) return;
  if (threadIdx.x < kTileTok) {
    const int r = (int)threadIdx.x;
    ts.tok[r] = r >= tr.nrows ? -1 : tr.g < a.E ? a.perm[tr.row0 + r] / a.k : tr.r0 + r;
  }
  __syncthreads();   // the token list is written
  if (LONG && tr.nrows > 64) gateup_tile(a, tr, ts, *reinterpret_cast<SmemLong<kSliceLong>*>(raw), yb);
  else gateup_tile(a, tr, ts, *reinterpret_cast<SmemShort*>(raw), yb);
}

// down: workgroup (tile, y) takes outputs [128 y, 128 y + 128) (W2 rows);
// wave w's lanes take outputs 128 y + 32 w + 16 nt + lane % 16, nt = 0, 1.
// K = I, staged in slices of SM::kSlice columns.
template <class SM>
__device__ __forceinline__ void down_tile(const PrefillArgs& a, const TileRows& tr, SM& s, int yb) {
  constexpr int kMT = SM::kRows / 16, SLICE = SM::kSlice;
  const int wave = wave_id(), lane = (int)threadIdx.x & 63;
  const int mi = lane & 15, kb = lane >> 4;
  const GroupW gw = group_w(a, tr.g, 1);
  const int n0 = yb * kDnCols, H = a.H, I = a.I;
  f32x4_t acc[2][kMT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Stage<SM> st;
  st.setup(a.g2, I, a.r2bit && tr.g < a.E, [&](int m) { return m < tr.nrows ? tr.row0 + m : -1; },
           [&](int r) { return n0 + r; });
  st.load(a.h, gw.codes, gw.scales, 0);
  for (int k0 = 0; k0 < I; k0 += SLICE) {
    __syncthreads();
    st.store(s);
    __syncthreads();
    if (k0 + SLICE < I) st.load(a.h, gw.codes, gw.scales, k0 + SLICE);
    mma_slice(s, 32 * wave, 32 * wave + 16, mi, kb, acc[0], acc[1]);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * kb + i;
        if (m < tr.nrows) a.y[(size_t)(tr.row0 + m) * H + n0 + 32 * wave + 16 * nt + mi] = acc[nt][mt][i];
      }
}

// SHORT: the slice of tiles of <= 64 rows, min(I, 256); LS: of longer
// tiles (if the call has any: LONG), min(I, 128).
template <int SHORT, int LS, bool LONG>
__global__ __launch_bounds__(kPfThreads) void k_pf_down(PrefillArgs a) {
  __shared__ TileSmem ts;
  __shared__ __align__(16) uint8_t raw[kSmemBytes];
  static_assert(sizeof(GemmSmem<SHORT, 64>) <= kSmemBytes && sizeof(GemmSmem<LS, 128>) <= kSmemBytes, "fits");
  int yb;
  const TileRows tr = tile_rows(a, ts.toff, a.H / kDnCols, yb);
  if (tr.g < 0) return;
  if (LONG && tr.nrows > 64) down_tile(a, tr, *reinterpret_cast<GemmSmem<LS, 128>*>(raw), yb);
  else down_tile(a, tr, *reinterpret_cast<GemmSmem<SHORT, 64>*>(raw), yb);
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
  // at most ceil(c / 64) <= c / 64 + 1 tiles per group of c rows
  return (T * k + 63) / 64 + E + S * ((T + 63) / 64);
}

template <int SHORT, int LS>
void launch_down(const PrefillArgs& a, bool lng, dim3 grid, hipStream_t st) {
  if (lng) hipLaunchKernelGGL((k_pf_down<SHORT, LS, true>), grid, dim3(kPfThreads), 0, st, a);
  else hipLaunchKernelGGL((k_pf_down<SHORT, LS, false>), grid, dim3(kPfThreads), 0, st, a);
}

int launch_prefill(const PrefillArgs& args, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  PrefillArgs a = args;
  // 128-row tiles once the routed groups average 128 rows: fewer decodes of
  // each weight row per token; below that, more tiles in flight pay better
  const bool lng = (long long)a.T * a.k >= 128LL * a.E;
  a.tile_rows = lng ? 128 : 64;
  const int chunks = (prefill_max_tiles(a.T, a.k, a.E, a.S) + 7) / 8;   // of 8 tiles
  (void)hipGetLastError();
  const int tblocks = (a.T + kRouteTok - 1) / kRouteTok, eblocks = (a.E + 63) / 64;
  const int ygroups = std::min(eblocks, std::max(1, (1024 + tblocks - 1) / tblocks));
  hipLaunchKernelGGL(k_pf_logits, dim3(tblocks, ygroups), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_topk, dim3((a.T + kPfThreads / 64 - 1) / (kPfThreads / 64)), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_count, dim3(a.E), dim3(kPfThreads), 0, st, a);
  hipLaunchKernelGGL(k_pf_place, dim3(a.E), dim3(kPfThreads), 0, st, a);
  const dim3 ggrid(chunks * 8 * (a.I / kGuCols));
  if (lng) hipLaunchKernelGGL(k_pf_gateup<true>, ggrid, dim3(kPfThreads), 0, st, a);
  else hipLaunchKernelGGL(k_pf_gateup<false>, ggrid, dim3(kPfThreads), 0, st, a);
  const dim3 dgrid(chunks * 8 * (a.H / kDnCols));
  if (a.I == 64) launch_down<64, 64>(a, lng, dgrid, st);
  else if (a.I == 128) launch_down<128, 128>(a, lng, dgrid, st);
  else launch_down<kSliceShort, kSliceLong>(a, lng, dgrid, st);
  hipLaunchKernelGGL(k_pf_combine, dim3(a.T), dim3(kPfThreads), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace moe
