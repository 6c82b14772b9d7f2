// Internal definitions shared by the host side (api.cpp) and the kernels
// (kernels.hip) of the MoE decode library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

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
// chunks each, handled by different wavefronts of a workgroup.  A slice of
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

// Returns 0 and fills g, or -1 when the shape has no supported geometry.
MOE_HD inline int make_geom(int rows, int cols, MatGeom* g) {
  if (rows <= 0 || cols <= 0 || cols % 32) return -1;
  const int C = cols / 32;
  int ns = 1;
  while (C / ns > 64 || C % ns) {
    ns *= 2;
    if (ns > 4) return -1;
  }
  const int cw = C / ns;
  int lpr = 1;
  while (lpr < cw) lpr *= 2;
  const int rpw = 64 / lpr;
  if (rows % rpw) return -1;
  const int nsteps = rows / rpw;
  if (nsteps % 2) return -1;
  g->rows = rows; g->cols = cols; g->C = C; g->ns = ns; g->cw = cw;
  g->lpr = lpr; g->rpw = rpw; g->nsteps = nsteps; g->su = rpw * cw;
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

constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kGateSteps = 2;      // gate (and up) steps per wavefront in gate/up kernels

// Everything the three kernels of one layer call need, passed by value.
struct LayerArgs {
  // inputs
  const uint16_t* x;         // bf16 [B][H]
  const uint16_t* router_w;  // bf16 [Er][H]
  const float* bias;         // fp32 [E] or null
  const uint16_t* gamma;     // bf16 [H] or null
  const uint8_t* r_codes;    // routed code region
  const uint8_t* r_scales;   // routed scale region base
  const float* r_tscale;     // routed tensor scales [E][2]
  const uint8_t* s_codes;    // shared code region
  const uint8_t* s_scales;   // shared scale region base
  const float* s_tscale;     // shared tensor scales [S][2]
  uint16_t* out;             // bf16 [B][H]
  // workspace
  unsigned* counter;         // last-block counter (kept at 0 between calls)
  float* logits;             // [maxB][Er]
  int* rt_nd;                // [1] number of distinct routed experts
  int* rt_ids;               // [maxd] distinct experts, ascending
  unsigned* rt_mask;         // [maxd] token masks
  float* rt_wt;              // [maxd][maxB] combine weight per (slot, token)
  int* topk_ids;             // [maxB][k]
  float* topk_w;             // [maxB][k]
  float* shared_c;           // [maxB][S]
  uint16_t* xhat;            // bf16 [maxB][H] (pre-norm only)
  uint16_t* h_routed;        // bf16 [maxd][maxB][I]
  uint16_t* h_shared;        // bf16 [S][maxB][I]
  // shapes
  int B, maxB, H, I, E, k, S, Er, maxd;
  int route, prenorm, residual;
  float eps;
  MatGeom g13, g2;
  // expert set strides (bytes)
  size_t r_code_stride, r_w13_code, r_scale_stride, r_w13_scale;
  size_t s_code_stride, s_w13_code, s_scale_stride, s_w13_scale;
  // grid bookkeeping
  int n_router_blocks;       // kernel 1: router blocks come first
  int wpe13;                 // workgroups per expert in the gate/up kernels
  int s3;                    // steps per workgroup in the down kernel
};

// Launchers (kernels.hip).  Return a hipError_t as int.
// ev4: null, or 4 hipEvent_t recorded around the three kernels.
int launch_layer(const LayerArgs& a, int tb, int rwt, int swt, void* stream, void* const* ev4);
int launch_debug_h(const LayerArgs& a, uint16_t* h_r, uint16_t* h_s, void* stream);

}  // namespace moe
