// Internal definitions shared by the host side (api.cpp) and the kernel
// (layer.hip) of the MoE decode library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/moe_decode.h"

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

// Lane geometry of one weight matrix [rows][cols] (cols = reduction dim).
//
// A row is cut into chunks of 32 consecutive elements; a lane owns one chunk
// per "wave step" (16 B of e2m1 codes, or 4 x 16 B of bf16, plus 2 e4m3 block
// scales).  Rows longer than 64 chunks are split into `ns` slices of `cw`
// chunks each.  A slice of
// `cw` chunks occupies `lpr` (power of two >= cw) lanes, so one wave step
// covers `rpw` = 64 / lpr rows.  Steps run over rows: step t covers rows
// t*rpw .. t*rpw + rpw - 1.  `su` is the number of 16 B units one wave step
// of one slice stores (= rpw * cw).
struct MatGeom {
  int rows, cols;
  int C;       // chunks per row = cols / 32
  int ns;      // slices per row (1, 2 or 4)
  int cw;      // chunks per row in one slice
  int lpr;     // lanes per row
  int rpw;     // rows per wave step
  int nsteps;  // wave steps per slice = rows / rpw (even)
  int su;      // 16 B units per step per slice = rpw * cw
};

// The geometry of a [rows][cols] matrix (rows % rpw == 0 and nsteps even
// are checked by make_geom; ns = 0 marks a row too long for four slices).
MOE_HD constexpr MatGeom geom_of(int rows, int cols) {
  MatGeom g{};
  g.rows = rows;
  g.cols = cols;
  g.C = cols / 32;
  int ns = 1;
  while (ns <= 4 && (g.C / ns > 64 || g.C % ns)) ns *= 2;
  if (ns > 4) return g;
  g.ns = ns;
  g.cw = g.C / ns;
  int lpr = 1;
  while (lpr < g.cw) lpr *= 2;
  g.lpr = lpr;
  g.rpw = 64 / lpr;
  g.nsteps = rows / g.rpw;
  g.su = g.rpw * g.cw;
  return g;
}

// Returns 0 and fills g, or -1 when the shape has no supported geometry.
MOE_HD inline int make_geom(int rows, int cols, MatGeom* g) {
  if (rows <= 0 || cols <= 0 || cols % 32) return -1;
  const MatGeom m = geom_of(rows, cols);
  if (m.ns == 0 || rows % m.rpw || m.nsteps % 2) return -1;
  *g = m;
  return 0;
}

// Packed position of the 16 B code unit (nvfp4) of slice s, step t, row-in-step
// ri, chunk-in-slice j.
MOE_HD inline size_t code_unit(const MatGeom& g, int s, int t, int ri, int j) {
  return ((size_t)s * g.nsteps + t) * g.su + (size_t)ri * g.cw + j;
}
// Packed byte offset of the 4-byte scale word holding the two block scales of
// steps (t & ~1) and (t | 1) for the same lane; step t's pair starts at byte
// 2 * (t & 1) of that word.
MOE_HD inline size_t scale_word(const MatGeom& g, int s, int t, int ri, int j) {
  return (((size_t)s * (g.nsteps / 2) + t / 2) * g.su + (size_t)ri * g.cw + j) * 4;
}
// Packed position of bf16 unit `sub` (elements 8*sub .. 8*sub+7 of the chunk).
MOE_HD inline size_t bf16_unit(const MatGeom& g, int s, int t, int sub, int ri, int j) {
  return (((size_t)s * g.nsteps + t) * 4 + sub) * g.su + (size_t)ri * g.cw + j;
}

// Unsigned division by a divisor fixed per layer, as a multiply-high, an add
// and a shift (round-up method of Granlund and Montgomery):
// q = (mulhi(n, m) + n) >> s with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1.
// Exact for n < 2^31 (the add stays in 32 bits); moe_layer_create checks
// every divisor it sets up over all n < 2^22.
struct FastDiv {
  uint32_t m, s;
};
MOE_HD inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  FastDiv f;
  f.m = (uint32_t)(((((unsigned long long)1 << s) - d) << 32) / d + 1);
  f.s = s;
  return f;
}
MOE_HD inline uint32_t fastdiv(uint32_t n, FastDiv f) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t t = __umulhi(n, f.m);
#else
  const uint32_t t = (uint32_t)(((unsigned long long)n * f.m) >> 32);
#endif
  return (t + n) >> f.s;
}

// ---------------------------------------------------------------------------
// single-launch layer kernel
// ---------------------------------------------------------------------------

constexpr int kFusedWaves = 4;                    // wavefronts per workgroup
constexpr int kFusedThreads = 64 * kFusedWaves;
constexpr int kLogitLine = 16;                    // 8-byte words per router row (one 128-B line)
constexpr int kMaxPairs = MOE_MAX_BATCH * (MOE_MAX_TOPK + MOE_MAX_SHARED);

// Everything one launch of the single-launch layer kernel needs, by value.
//
// Cross-workgroup data (router logits, SiLU*up activations) moves through
// tagged 8-byte words: the low half holds the value, the high half the call's
// tag (the handle's call counter + 1).  A reader polls a word until its tag
// matches, so no flag, fence or barrier is needed: each word carries its own
// validity, and a word of an older call never matches.
// The per-layer and per-call values that are never compile-time constants.
struct KCommon {
  // inputs (caller-owned device memory)
  const uint16_t* x;         // bf16 [B][H]
  const uint16_t* router_w;  // bf16 [Er][H]
  const float* bias;         // fp32 [E] or null
  const uint16_t* gamma;     // bf16 [H] or null
  const uint8_t* r_codes;    // routed code region
  const uint8_t* r_scales;   // routed scale region
  const float* r_tscale;     // routed tensor scales [E][2]
  const uint8_t* s_codes;    // shared code region
  const uint8_t* s_scales;   // shared scale region
  const float* s_tscale;     // shared tensor scales [S][2]
  uint16_t* out;             // bf16 [B][H]
  // workspace (handle-owned)
  unsigned* epoch;                 // [1] number of completed calls
  unsigned* err;                   // [1] sticky error bits (kErr*)
  unsigned long long* xlog;        // [Er][kLogitLine] logit words
  unsigned long long* xh;          // [maxP][I/2] activation words
  int* topk_ids;                   // [maxB][k] readback
  float* topk_w;                   // [maxB][k]
  float* shared_c;                 // [maxB][S]
  int route, prenorm, residual;
  float eps;
  size_t r_code_stride, r_w13_code, r_scale_stride, r_w13_scale;
  size_t s_code_stride, s_w13_code, s_scale_stride, s_w13_scale;
  // plan
  int G;                           // workgroups (a power of two); all must be resident at once
  int log2G;
  FastDiv dv_gs2;                  // division by the gate/up step pairs of a matrix
  int lds_act;                     // bytes of the activation region (x, then h)
  int lds_acc;                     // bytes of the down-GEMV partial sums
  int spg_max;                     // most down-GEMV steps a workgroup owns
  unsigned long long wait_ticks;   // bound of every wait, in 100 MHz ticks
};

// Layer shape read from the arguments ...
struct DynShape {
  int H, I, E, k, S, Er;
  MatGeom g13, g2;
};
// ... or fixed at compile time (the kernel then folds every shape-derived
// index, stride and branch; the host launches it only for a matching layer).
template <int H_, int I_, int E_, int K_, int S_, int ER_>
struct FixedShape {
  static constexpr int H = H_, I = I_, E = E_, k = K_, S = S_, Er = ER_;
  static constexpr MatGeom g13 = geom_of(2 * I_, H_), g2 = geom_of(H_, I_);
};
// Flint's MoE layer: H = 2048, I = 512, 256 routed experts, top-6, one shared
// expert, sigmoid router over the 256 routed experts.
using FlintShape = FixedShape<2048, 512, 256, 6, 1, 256>;

// Batch size of the call: read from the arguments, or fixed (buckets 1 and 2
// hold exactly that many tokens).
template <int BF> struct BatchField { static constexpr int B = BF; };
template <> struct BatchField<0> { int B; };

// Kernel arguments.  Fields of a fixed shape or batch are static members, so
// the kernel reads a.H, a.B, a.g13.lpr ... the same way in every variant.
template <class SH, int BF>
struct KArgs : KCommon, SH, BatchField<BF> {};

// Everything one launch of the single-launch layer kernel needs, by value
// (host side; the launcher turns it into the variant's KArgs).
//
// Cross-workgroup data (router logits, SiLU*up activations) moves through
// tagged 8-byte words: the low half holds the value, the high half the call's
// tag (the handle's call counter + 1).  A reader polls a word until its tag
// matches, so no flag, fence or barrier is needed: each word carries its own
// validity, and a word of an older call never matches.
struct FusedArgs : KCommon, DynShape {
  int B;
};

template <class SH, int BF>
inline KArgs<SH, BF> kargs_of(const FusedArgs& f) {
  KArgs<SH, BF> k{};
  static_cast<KCommon&>(k) = f;
  if constexpr (std::is_same<SH, DynShape>::value) static_cast<DynShape&>(k) = f;
  if constexpr (BF == 0) k.B = f.B;
  return k;
}

// Shape variant a layer runs with: 1 = FlintShape, 0 = read from the arguments.
// The fixed shape is compiled for equal routed and shared weight types only;
// any other pair runs the variant that reads the shape from the arguments.
inline int fixed_shape_of(int H, int I, int E, int k, int S, int Er, int rwt, int swt) {
  using F = FlintShape;
  return (H == F::H && I == F::I && E == F::E && k == F::k && S == F::S && Er == F::Er && rwt == swt) ? 1 : 0;
}

enum : unsigned { kErrLogitWait = 1u, kErrActWait = 2u, kErrLocalWait = 4u };

// Size of the library's static device scratch array (moe_decode_layer_static):
// the largest workspace a layer may need to run without a handle.
constexpr size_t kStaticScratchBytes = (size_t)1 << 20;
static_assert(kStaticScratchBytes == MOE_STATIC_SCRATCH_BYTES, "scratch size differs from the header's");
// Device address of the static scratch array on `device` (the current
// device), looked up once per device; nullptr on failure.
void* static_scratch(int device);

// Dynamic LDS bytes of the kernel for a plan.
MOE_HD inline int fused_lds_bytes(const KCommon& a) { return a.lds_act + a.lds_acc; }

int launch_fused(const FusedArgs& a, int tb, int rwt, int swt, void* stream);
int launch_fused_debug_h(const FusedArgs& a, uint16_t* h_r, uint16_t* h_s, void* stream);
int fused_occupancy(int shape, int tb, int qx, int rwt, int swt, int lds_bytes, int* blocks_per_cu);
// Whether a kernel variant is compiled for (shape, batch bucket, qx, weight types); host only.
bool fused_variant_exists(int shape, int tb, int qx, int rwt, int swt);
// Router units per thread the kernel is built for at this hidden size (0: none).
int fused_qx(int hidden);

// Batch-1 kernel of the Flint shape with NVFP4 routed and shared experts and
// the sigmoid router: 256 workgroups of 512 threads, all resident at once.
// One launch runs a chain of 1 .. kMaxChain such layers: layer l + 1 takes
// layer l's output as its input.
constexpr int kB1Workgroups = 256;
constexpr int kMaxChain = 16;
static_assert(kMaxChain == MOE_MAX_CHAIN, "chain length differs from the header's");
// What differs between the layers of a chain.
struct ChainLayer {
  const uint16_t* router_w;
  const float* bias;
  const uint16_t* gamma;
  const uint8_t* r_codes;
  const uint8_t* r_scales;
  const float* r_tscale;
  const uint8_t* s_codes;
  const uint8_t* s_scales;
  const float* s_tscale;
  int* topk_ids;   // readback of the layer's handle
  float* topk_w;
  float* shared_c;
  float eps;
  int prenorm, residual;
};
struct B1Args {
  KCommon a;                   // the call's common fields: x, out, workspace, strides, wait bound
  unsigned long long* xx;      // [H / 2] tagged words: a layer's output, the next layer's input
  int n;                       // layers
  int r2bit;                   // routed experts in the 2-bit planes (single layer only)
  ChainLayer L[kMaxChain];
};
// The layer fields of a's single layer as a chain entry.
inline ChainLayer chain_layer_of(const KCommon& a) {
  ChainLayer c;
  c.router_w = a.router_w;
  c.bias = a.bias;
  c.gamma = a.gamma;
  c.r_codes = a.r_codes;
  c.r_scales = a.r_scales;
  c.r_tscale = a.r_tscale;
  c.s_codes = a.s_codes;
  c.s_scales = a.s_scales;
  c.s_tscale = a.s_tscale;
  c.topk_ids = a.topk_ids;
  c.topk_w = a.topk_w;
  c.shared_c = a.shared_c;
  c.eps = a.eps;
  c.prenorm = a.prenorm;
  c.residual = a.residual;
  return c;
}
int launch_b1(const B1Args& a, void* stream);

// Prefill / large-batch path: T tokens as grouped GEMMs on the matrix cores
// (seven launches on one stream).  Shapes it takes: NVFP4 routed and shared
// experts, sigmoid routing, H <= kPfMaxH, E <= kPfMaxE (both tile sizes
// divide them; checked by the library).
constexpr int kPfMaxH = 2048;
constexpr int kPfMaxE = 256;
struct PrefillArgs {
  const uint16_t* x;         // bf16 [T][H]
  uint16_t* out;             // bf16 [T][H]
  const uint16_t* router_w;  // bf16 [E][H]
  const float* bias;         // fp32 [E] or null
  const uint16_t* gamma;     // bf16 [H] (prenorm)
  float eps;
  int prenorm, residual;
  const uint8_t *r_codes, *r_scales;
  const float* r_tscale;
  const uint8_t *s_codes, *s_scales;
  const float* s_tscale;
  size_t r_code_stride, r_w13_code, r_scale_stride, r_w13_scale;
  size_t s_code_stride, s_w13_code, s_scale_stride, s_w13_scale;
  int T, H, I, E, k, S;
  int tile_rows;     // rows per GEMM tile (64 or 128; chosen by launch_prefill)
  int r2bit;         // routed experts in the 2-bit planes (the shared ones are NVFP4)
  MatGeom g13, g2;
  // caller's workspace
  uint16_t* xhat;   // bf16 [T][H] (prenorm only)
  float* logits;    // fp32 [T][E]
  int* ids;         // [T][k] selection order
  float* wts;       // [T][k]
  int* counts;      // [5 E]: pairs per expert, then each counting wave's share [E][4]
  int* offs;        // [E + S + 1] first sorted row of each group
  int* tile_off;    // [E + S + 1] first tile of each group
  int* perm;        // [T k] sorted row -> token * k + slot
  int* inv;         // [T k] token * k + slot -> sorted row
  uint16_t* h;      // bf16 [T k + T S][I] at sorted rows
  float* y;         // fp32 [T k + T S][H] at sorted rows
  int32_t* out_ids; // optional copies of ids / wts (caller's)
  float* out_w;
};
int prefill_max_tiles(int T, int k, int E, int S);
int launch_prefill(const PrefillArgs& a, void* stream);
int b1_occupancy(int* blocks_per_cu);
// Small-batch dense NVFP4 GEMV on a matrix packed with geometry g (ns == 1,
// rows padded to whole step pairs; only the first `rows` outputs are written).
struct DenseArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  const uint16_t* x;   // bf16 [B][cols]
  uint16_t* y;         // bf16 [B][rows]
  int rows, B;
  MatGeom g;
};
int launch_dense(const DenseArgs& a, void* stream);
int dense_grid(const MatGeom& g);

// Batch 2-8 kernel of the same layers: 256 workgroups of 512 threads.
int launch_b8(const KCommon& a, int batch, bool r2bit, void* stream);
int b8_occupancy(int* blocks_per_cu);

}  // namespace moe
