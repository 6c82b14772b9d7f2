/*
 * moe_decode.h -- C ABI of the small-batch NVFP4 MoE decode layer for
 * MI355X (gfx950).
 *
 * What the layer computes (for each token b of a batch of at most 8):
 *   xhat  = x                                  (or RMSNorm(x) * gamma, pre-norm layers)
 *   l     = R xhat (+ bias)                    router GEMV over E (+S) experts
 *   route = sigmoid top-k, renormalised        (Flint page, "A 40B MoE that activates
 *                                               2.5B parameters": sigmoid top-6 plus a
 *                                               shared expert)
 *        or softmax over the E+S logits, top-k over the routed E only, weights =
 *           selected probabilities, shared expert s weighted by its own probability
 *                                              (Inkling page, "Model Architecture":
 *                                               the expert sink)
 *   h_e   = SiLU(W13_e[:I] xhat) * (W13_e[I:] xhat)     per selected/shared expert
 *   out   = sum_e w_e W2_e h_e  (+ x for pre-norm residual layers)
 * Only the chosen experts' weight bytes are fetched, and routing and the expert
 * combine run inside the same launch as the GEMVs around them (Flint page, "From
 * 1,096 kernels to 346": the small-batch MoE kernels and the low-latency decode path).
 *
 * Weight formats
 *   NVFP4: e2m1 codes, one e4m3 scale per 16 consecutive elements of a row, one fp32
 *          scale per matrix ("Frontier MoE on consumer Blackwell (SM120)", section
 *          "GLM-5.2": e2m1 x e4m3 block-16 x per-tensor scale_2).  Activations are
 *          bf16 (W4A16, Flint page, "A 40B MoE ...").
 *   BF16:  plain bf16 weights.
 *   Canonical (unpacked) order of an NVFP4 matrix [R, K]: codes uint8 [R][K/2], element
 *   2j of a row in the low nibble of byte j, 2j+1 in the high nibble; scales uint8
 *   [R][K/16].  Each expert has W13 [2I][H] (rows 0..I-1 gate, I..2I-1 up) and
 *   W2 [H][I].  The packers below move these bytes into the kernel layout without
 *   changing any of them (repack at load time, Flint page, "A 40B MoE ...": the GGUF
 *   blocks are repacked losslessly at load).
 *
 * Conventions
 *   * Every function returns a moe_status (0 = success); no exceptions cross the ABI.
 *   * "device" pointers are HIP device memory owned by the caller; "host" pointers are
 *     ordinary host memory owned by the caller.  The library owns only the workspace a
 *     layer handle allocates at creation.
 *   * `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *     enqueued asynchronously; moe_decode_layer performs no allocation, no host
 *     synchronisation and no copy to the host.
 *   * Argument errors are detected on the host before anything is enqueued.  Kernel
 *     faults surface at the caller's next synchronisation of the stream.  NaN/Inf in
 *     inputs propagate; they are not checked.
 *   * A handle's workspace is shared by all calls made with it: calls on one handle
 *     must be ordered (one stream, or explicit dependencies).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* limits of this implementation */
#define MOE_MAX_BATCH 8      /* the low-latency decode path serves up to 8 requests  */
#define MOE_MAX_ROUTED 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_SHARED 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null/negative/inconsistent argument                   */
  MOE_ERR_UNSUPPORTED = -2, /* shape, dtype or routing combination not implemented    */
  MOE_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned                */
  MOE_ERR_BATCH = -4,       /* batch outside [1, max_batch]                           */
  MOE_ERR_LAUNCH = -5,      /* a kernel launch or async copy was rejected by HIP      */
  MOE_ERR_DEVICE = -6,      /* device allocation / query failed (e.g. no GPU)         */
  MOE_ERR_STATE = -7        /* readback before any moe_decode_layer call on a handle  */
} moe_status;

/* MOE_W_2BIT: the SM120 page's sign-symmetric 2-bit expert planes ("How it fits - 2-bit
 * experts at FP4 quality"): W = LEVEL[q] * e4m3 block-16 scale * fp32 tensor scale,
 * LEVEL = {-4, -1, 1, 4} for q = 0..3; canonical codes uint8 [rows][cols/4], element 4j+i
 * in bits 2i..2i+1 of byte j; scales and tensor scales as NVFP4.  Routed experts only,
 * on the Flint shape (batch 1 to 8, NVFP4 shared expert, sigmoid routing, a device with
 * the 256 compute units the dedicated kernels take); moe_requant_2bit makes the planes
 * from NVFP4 experts.                                                                  */
typedef enum { MOE_W_NVFP4 = 0, MOE_W_BF16 = 1, MOE_W_2BIT = 2 } moe_wtype;

/* The two expert sets of a layer.  The routed set lives in two buffers (moe_decode_layer's
 * expert_packed = its code region, scales = its scale region); the shared set in one
 * (shared_w: code region, then the scale region at shared_scale_offset).              */
typedef enum { MOE_SET_ROUTED = 0, MOE_SET_SHARED = 1 } moe_set;

typedef enum {
  MOE_ROUTE_SIGMOID_TOPK = 0, /* s = sigmoid(l + bias), top-k of s, w = s / sum_topk s, shared c = 1 */
  MOE_ROUTE_SOFTMAX_SINK = 1  /* p = softmax(l[0..E+S)), top-k of p[0..E), w = p, shared c_s = p[E+s] */
} moe_route;

/* Layer description.  Shapes: hidden H, inter I, n_routed E, top_k k, n_shared S.
 * Requirements (else MOE_ERR_UNSUPPORTED): H % 32 == 0, I % 32 == 0, H <= 8192,
 * I <= 2048, 1 <= k <= min(E, 16), E <= 512, 0 <= S <= 4, 1 <= max_batch <= 8,
 * plus the layout conditions moe_layer_validate checks.  The router has E rows
 * (sigmoid) or E + S rows (sink: rows E..E+S-1 score the shared experts).          */
typedef struct {
  int hidden;
  int inter;
  int n_routed;
  int top_k;
  int n_shared;
  int max_batch;
  int routed_wtype;          /* moe_wtype                                                  */
  int shared_wtype;          /* moe_wtype; BF16 routed with NVFP4 shared is unsupported     */
  int route;                 /* moe_route                                                  */
  const float* router_bias;  /* device fp32 [E] added to the routed logits, or NULL.        */
                             /* Sigmoid routing only.  Must outlive the handle.            */
  const void* prenorm_gamma; /* device bf16 [H], or NULL.  Non-NULL turns on the pre-norm   */
                             /* prologue xhat = bf16(x / sqrt(mean(x^2) + eps) * gamma).     */
  float rms_eps;             /* epsilon of the pre-norm (e.g. 1e-6)                         */
  int add_residual;          /* non-zero: out = x + MoE(xhat)                               */
} moe_layer_desc;

typedef struct moe_layer* moe_layer_t;

/* Byte layout of a set of n experts of one weight type, as the packers write it.
 * A set lives in two regions:
 *   code region : expert e at e * code_stride: packed W13 (w13_code_bytes) then packed
 *                 W2.  NVFP4: the e2m1 codes.  BF16: the bf16 weights.
 *   scale region: NVFP4 only.  Expert e at e * scale_stride: packed W13 block scales
 *                 (w13_scale_bytes) then packed W2 block scales; then, at
 *                 tensor_scale_offset, fp32 [n][2] = (W13 scale, W2 scale) per expert.
 *                 BF16: empty (scale_region_bytes = 0).
 * moe_decode_layer takes the routed set's code region as `expert_packed` and its scale
 * region as `scales`; the shared set is one buffer `shared_w` holding its code region
 * at offset 0 and its scale region at offset shared_scale_offset.                   */
typedef struct {
  size_t w13_code_bytes;
  size_t w2_code_bytes;
  size_t code_stride;
  size_t code_region_bytes;
  size_t w13_scale_bytes;
  size_t w2_scale_bytes;
  size_t scale_stride;
  size_t tensor_scale_offset;
  size_t scale_region_bytes;
  size_t shared_scale_offset; /* where the scale region starts inside a one-buffer set */
  size_t shared_total_bytes;  /* code region + padding + scale region                   */
} moe_expert_layout;

/* ---- host-only queries (no device access) -------------------------------------- */

/* Version of this header's ABI (MOE_ABI_VERSION).  Host only, never fails.          */
int moe_abi_version(void);
/* Static text for a moe_status value (unknown values get "unknown status").          */
const char* moe_status_str(int status);

/* Checks a description without touching the device: shapes and limits, the dtype /
 * routing combination (Flint page, "A 40B MoE that activates 2.5B parameters": sigmoid
 * top-6 plus a shared expert; Inkling page, "Model Architecture": the expert sink) and
 * that a kernel is compiled for it at every batch up to max_batch.  Device pointers
 * inside it are not dereferenced.  A description this accepts is accepted by
 * moe_layer_create unless the device itself fails (MOE_ERR_DEVICE) or cannot hold the
 * launch (MOE_ERR_UNSUPPORTED from the occupancy check).                              */
int moe_layer_validate(const moe_layer_desc* desc);

/* Byte layout of one expert set (MOE_SET_ROUTED or MOE_SET_SHARED) of the layer desc
 * describes (see moe_expert_layout): the sizes a caller allocates for moe_pack_experts'
 * outputs.  NVFP4 sizes follow the format's three parts ("Frontier MoE on consumer
 * Blackwell (SM120)", section "GLM-5.2": e2m1 codes, e4m3 per 16-element block, one fp32
 * per tensor).  Checks desc as moe_layer_validate does.                             */
int moe_expert_layout_query(const moe_layer_desc* desc, int set, moe_expert_layout* out);

/* ---- packers (host memory, lossless, load time) ----------------------------------- */
/* The Flint page ("A 40B MoE that activates 2.5B parameters") repacks its checkpoint's
 * NVFP4 blocks losslessly at load time into the order its kernels read; these do the
 * same for the gfx950 kernels.  All buffers are host memory owned by the caller.      */

/* Experts [first, first + count) of one expert set of the layer desc describes, from
 * canonical bytes into the set's packed buffers, every offset and the order inside them
 * chosen by the library (moe_expert_layout_query).
 *   NVFP4: w13 uint8 [count][2I][H/2], w13_scales uint8 [count][2I][H/16],
 *          w2 uint8 [count][H][I/2],   w2_scales uint8 [count][H][I/16],
 *          tensor_scales fp32 [count][2] = (W13, W2) per expert, or NULL for 1.0.
 *   BF16:  w13 uint16 [count][2I][H], w2 uint16 [count][H][I]; the scale and
 *          tensor-scale arguments are ignored (may be NULL).
 * MOE_SET_ROUTED: region holds code_region_bytes, scale_region scale_region_bytes
 * (NVFP4; ignored for BF16).  MOE_SET_SHARED: region holds shared_total_bytes and
 * scale_region is ignored.  Bytes of other experts are left as they are, so a set can
 * be packed a few experts at a time.  Lossless: every byte (-0 codes, zero and NaN
 * scale bytes) is kept.  MOE_ERR_INVALID_ARG for a null required pointer or a range
 * outside the set; the errors of moe_layer_validate for desc.                         */
int moe_pack_experts(const moe_layer_desc* desc, int set, int first, int count,
                     const void* w13, const void* w13_scales, const void* w2,
                     const void* w2_scales, const float* tensor_scales, void* region,
                     void* scale_region);
/* Exact inverse of moe_pack_experts (data flowing the other way; tensor_scales may be
 * NULL to skip them).                                                                  */
int moe_unpack_experts(const moe_layer_desc* desc, int set, int first, int count,
                       const void* region, const void* scale_region, void* w13,
                       void* w13_scales, void* w2, void* w2_scales, float* tensor_scales);

/* One canonical NVFP4 matrix [rows][cols] -> the kernel layout (the building block of
 * moe_pack_experts).
 * codes: uint8 [rows][cols/2] in, rows*cols/2 bytes out; scales:
 * uint8 [rows][cols/16] in, rows*cols/16 bytes out.  A permutation of 16-byte code
 * units and 2-byte scale pairs.  rows/cols must describe a W13 ([2I][H]) or W2
 * ([H][I]) matrix of a valid layer.                                                  */
int moe_pack_nvfp4(int rows, int cols, const uint8_t* codes, const uint8_t* scales,
                   uint8_t* codes_out, uint8_t* scales_out);
/* Exact inverse of moe_pack_nvfp4. */
int moe_unpack_nvfp4(int rows, int cols, const uint8_t* codes_packed,
                     const uint8_t* scales_packed, uint8_t* codes, uint8_t* scales);
/* One canonical bf16 matrix [rows][cols] (uint16 bit patterns) -> kernel layout, and
 * its inverse.  A permutation of 16-byte units.                                       */
int moe_pack_bf16(int rows, int cols, const uint16_t* w, uint16_t* w_out);
int moe_unpack_bf16(int rows, int cols, const uint16_t* w_packed, uint16_t* w);

/* Re-quantises one canonical NVFP4 matrix [rows][cols] (codes uint8 [rows][cols/2],
 * e4m3 scales [rows][cols/16]) to the 2-bit planes (codes2 uint8 [rows][cols/4], new
 * e4m3 scales2 [rows][cols/16]); the matrix's fp32 tensor scale is kept.  SM120 page,
 * "How it fits - 2-bit experts at FP4 quality": the sign-symmetric codebook {-4, -1, 1,
 * 4}, re-quantised from NVFP4 after an exact float64 dequantisation.  Each 16-element
 * block v (e2m1 x e4m3, exact in float64) gets the non-negative finite e4m3 scale s
 * (bytes 0x00..0x7E) with the least sum over the block, in element order, of
 * (v_i - LEVEL[q_i] s)^2, each q_i the nearest level (|v| = 2.5 s takes 1; the level's
 * sign is v's sign bit); equal errors take the smaller scale.  Host only, no device
 * access; cols % 16 == 0.                                                             */
int moe_requant_2bit(int rows, int cols, const uint8_t* codes, const uint8_t* scales,
                     uint8_t* codes2, uint8_t* scales2);

/* ---- small-batch dense NVFP4 GEMV ---------------------------------------------------- */
/* The Flint page ("From 1,096 kernels to 346") runs a small-batch dense GEMV on the same
 * packed NVFP4 weights as its other kernels: the attention projections (GQA with 32
 * query and 4 KV heads at hidden 2048) and the dense MLP of layers 0 and 1 ("A 40B MoE
 * that activates 2.5B parameters").  Here one matrix W [rows][cols] (cols the reduction)
 * is packed with the experts' layout and y = x W^T is computed for 1-8 bf16 tokens.
 * Limits: 1 <= rows <= 1048576, 32 <= cols <= 2048, cols a multiple of 32.           */
typedef struct {
  int rows, cols;
  int packed_rows;            /* rows rounded up to whole scale-word step pairs; the   */
                              /* rows past `rows` are packed as zeros                  */
  size_t code_bytes;          /* code region: packed e2m1 codes                         */
  size_t scale_bytes;         /* packed e4m3 block scales, at the start of the scale    */
                              /* region                                                 */
  size_t tensor_scale_offset; /* the fp32 per-tensor scale, inside the scale region     */
  size_t scale_region_bytes;
} moe_dense_layout;
/* Host only.  MOE_ERR_INVALID_ARG for a shape outside the limits or out == NULL.       */
int moe_dense_layout_query(int rows, int cols, moe_dense_layout* out);
/* Canonical NVFP4 matrix -> its packed regions (host memory, caller-owned):
 * codes uint8 [rows][cols/2], scales uint8 [rows][cols/16] (e4m3, block 16 along cols),
 * tensor_scale the fp32 per-tensor scale ("Frontier MoE on consumer Blackwell (SM120)",
 * section "GLM-5.2").  Lossless; MOE_ERR_INVALID_ARG for a null pointer or bad shape. */
int moe_pack_dense(int rows, int cols, const void* codes, const void* scales, float tensor_scale,
                   void* code_region, void* scale_region);
/* Exact inverse of moe_pack_dense (tensor_scale may be NULL to skip it).              */
int moe_unpack_dense(int rows, int cols, const void* code_region, const void* scale_region,
                     void* codes, void* scales, float* tensor_scale);
/* y[b][n] = sum_k W[n][k] x[b][k], rounded once to bf16, for 1 <= batch <= 8:
 *   code_region, scale_region  device, as moe_pack_dense wrote them (16-byte aligned)
 *   x  device bf16 [batch][cols], y  device bf16 [batch][rows] (16-byte aligned, not
 *   overlapping x).
 * Enqueues one kernel on `stream` (a hipStream_t, NULL for the default stream); returns
 * without waiting.  Allocates nothing.  MOE_ERR_INVALID_ARG / MOE_ERR_BATCH /
 * MOE_ERR_ALIGNMENT for bad arguments (nothing is enqueued), MOE_ERR_LAUNCH if the
 * launch fails.                                                                        */
int moe_dense_gemv(int rows, int cols, const void* code_region, const void* scale_region,
                   const void* x, void* y, int batch, void* stream);

/* ---- layer handle ------------------------------------------------------------------ */

/* Validates desc (moe_layer_validate), plans the launch for the current device and
 * allocates the handle's device workspace there, once: the cross-workgroup exchange
 * words, the call counter and the routing readback (the layer of the Flint page, "A 40B
 * MoE that activates 2.5B parameters", or the Inkling expert sink, "Model
 * Architecture").  No later call allocates.  *out is NULL on failure; MOE_ERR_DEVICE
 * if no device is usable.  The router bias and pre-norm gamma pointers in desc are
 * kept (not copied) and must outlive the handle.                                     */
int moe_layer_create(const moe_layer_desc* desc, moe_layer_t* out);
/* Frees the handle's workspace.  The caller must have synchronised every stream that
 * used it.  MOE_ERR_INVALID_ARG for NULL.                                             */
int moe_layer_destroy(moe_layer_t layer);

/* One MoE decode layer for `batch` tokens (1 <= batch <= max_batch).
 *   x             device bf16 [batch][H] (16-byte aligned)
 *   router_w      device bf16 [E_r][H] row-major, E_r = E (sigmoid) or E + S (sink)
 *   expert_packed device, routed set's code region (moe_expert_layout)
 *   scales        device, routed set's scale region (NULL allowed for BF16 experts)
 *   shared_w      device, shared set (code region, then scale region at
 *                 shared_scale_offset); NULL allowed when n_shared == 0
 *   out           device bf16 [batch][H]; must not overlap x
 * Enqueues ONE kernel on `stream` whose workgroups (moe_layer_grid) are all resident at
 * once and hand data to each other in device memory: router GEMV, routing (every
 * workgroup computes the same top-k from the gathered logits), the shared and the
 * selected experts' gate/up GEMV with SiLU*up, and the down GEMV of every selected and
 * shared expert with the weighted, fixed-order combine (+ residual).  The Flint page
 * ("From 1,096 kernels to 346") fuses routing and the combine into the neighbouring
 * GEMVs, and no expert outside the top-k has its bytes fetched; this call does the same in one
 * launch.  Deterministic: no floating-point atomics; the result does not depend on
 * scheduling.  Every cross-workgroup wait is bounded (0.2 s): if the grid cannot be
 * resident at once (for example another such call of a different handle runs
 * concurrently on another stream), the kernel still ends, sets an error bit
 * (moe_layer_error) and its output is undefined.  Calls on one handle must be ordered.*/
int moe_decode_layer(moe_layer_t layer, const void* x, const void* router_w,
                     const void* expert_packed, const void* scales, const void* shared_w,
                     void* out, int batch, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same layer call as
 * moe_decode_layer, on the same kernels, without a handle: desc (host, validated as
 * moe_layer_validate does) replaces the handle, and the call's workspace (exchange
 * words, call counter, routing copy) lives in a static device array of the library,
 * MOE_STATIC_SCRATCH_BYTES per device, held by every device the library runs on until
 * the process ends.  A description whose workspace does not fit is rejected with
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  The call performs no hipMalloc,
 * hipFree or other allocation (the launch plan of a shape is made on its first call on a
 * device and kept in a fixed table).  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (streams without an
 * order between them) race and their outputs are undefined.  err_flags: optional device
 * word (4-byte aligned) into which the call ORs the wait bits moe_layer_error would
 * report; the caller clears it; NULL discards them.  x, router_w, expert_packed,
 * scales, shared_w, out, batch and stream as for moe_decode_layer.                    */
#define MOE_STATIC_SCRATCH_BYTES (1u << 20)
int moe_decode_layer_static(const moe_layer_desc* desc, const void* x, const void* router_w,
                            const void* expert_packed, const void* scales, const void* shared_w,
                            void* out, int batch, unsigned* err_flags, void* stream);

/* Routing of the last moe_decode_layer call on this handle, copied on `stream` into
 * device buffers: ids int32 [batch][k] and w fp32 [batch][k] in selection order
 * (descending score, ties to the lower index); c fp32 [batch][S] shared coefficients
 * (sigmoid top-k renormalised: Flint page, "A 40B MoE that activates 2.5B parameters";
 * sink probabilities: Inkling page, "Model Architecture").  Any pointer may be NULL to
 * skip it.  MOE_ERR_STATE before the first call.                                      */
int moe_layer_routing(moe_layer_t layer, int32_t* ids, float* w, float* c, void* stream);

/* Profiling hook for benchmarks (the per-kernel timing the SM120 page, "SM120 decode
 * kernels", reports for its decode kernels).  events: n_events hipEvent_t handles (as void*), n_events a
 * positive multiple of 2; the pointer array is copied, the events stay owned by the caller and
 * must outlive the setting.  Every later moe_decode_layer call number c on this handle records
 * events[2*(c mod n_events/2) + 0] before its kernel and events[... + 1] after it, on its
 * stream.  events = NULL (or n_events = 0) turns the hook off.  Not meant for calls under
 * stream capture.                                                                            */
int moe_layer_set_profiling(moe_layer_t layer, void* const* events, int n_events);

/* Test hook: the SiLU*up activations h = SiLU(gate) * up of the last call (the
 * SiLU-gated expert MLP of the Flint page, "From 1,096 kernels to 346"), bf16, gathered
 * on `stream` into device buffers h_routed [batch][k][I] (selection order) and h_shared
 * [batch][S][I].  Either pointer may be NULL.  MOE_ERR_STATE before the first call.  */
int moe_layer_debug_h(moe_layer_t layer, void* h_routed, void* h_shared, void* stream);

/* A chain of n_layers (1 <= n_layers <= MOE_MAX_CHAIN) decode layers in ONE launch: layer
 * l + 1 takes layer l's output (bf16) as its x, and the launch writes the last layer's
 * output to `out`.  This is the Flint page's low-latency path across layers ("From 1,096
 * kernels to 346": each kernel loads its weights while the previous one still runs,
 * through programmatic dependent launch): inside the launch, layer l + 1's router row
 * and shared expert load while layer l finishes, and the output rows travel to every
 * workgroup as tagged words in the first layer's workspace.
 *   layers                  host array of n_layers handles with the same shape, weight
 *                           types and routing (their own pre-norm γ, bias, residual flag
 *                           and readback buffers apply); all created on one device
 *   x, out                  device bf16 [batch][H] (16-byte aligned, not overlapping)
 *   router_w, expert_packed, scales, shared_w   host arrays of n_layers device
 *                           pointers, each as for moe_decode_layer
 * Batch 1 on layers that run the batch-1 kernel dedicated to the Flint shape
 * (moe_layer_set_path reports MOE_PATH_DEDICATED for layers[0]); MOE_ERR_UNSUPPORTED
 * otherwise (call moe_decode_layer per layer then).  Uses layers[0]'s workspace and
 * call counter (the launch takes n_layers of its tags); after it moe_layer_routing works
 * on every layer's handle and moe_layer_debug_h on none.  Allocates nothing.          */
#define MOE_MAX_CHAIN 16
int moe_decode_chain(const moe_layer_t* layers, int n_layers, const void* x,
                     const void* const* router_w, const void* const* expert_packed,
                     const void* const* scales, const void* const* shared_w, void* out,
                     int batch, void* stream);

/* ---- prefill / large batch ------------------------------------------------------
 * The same layer for T tokens at once (prompt processing), as grouped GEMMs on the
 * matrix cores instead of the decode kernels' GEMVs.  The Flint page ("From 1,096
 * kernels to 346") counts the MoE kernel work as the largest prefill gain, and the SM120
 * page ("How it fits - 2-bit experts at FP4 quality") replaces the [tokens * top_k,
 * hidden] fp32 scatter buffer of the expert outputs by a direct, deterministic
 * gather/reduce; both are what this call does:
 *   route   the router GEMM (bf16, fp32 sums) of every token, its top-k and weights
 *           (the decode kernels' selection rule and weights);
 *   group   the (token, slot) pairs sorted by expert, tokens in order within an expert;
 *   gate/up per expert, its tokens' rows times the decoded NVFP4 gate and up rows,
 *           h = SiLU(g) * up in bf16; each shared expert takes all T tokens;
 *   down    y = W2 h in fp32 at the same sorted rows;
 *   combine out[t] = sum of the token's shared experts' y, then its routed slots' w * y in
 *           selection order (each times its W2 tensor scale), (+ x), one bf16 rounding.
 * Shapes it takes (else MOE_ERR_UNSUPPORTED): NVFP4 or 2-bit routed and NVFP4 shared
 * experts (a 2-bit expert's chunks widen to e2m1 as they are staged), sigmoid
 * routing, H <= 2048 with H % 256 == 0, I = 64, 128 or a multiple of 256,
 * E <= 256 with E % 16 == 0.  1 <= tokens <= MOE_PREFILL_MAX_TOKENS and
 * tokens * (k + S) * I < 2^32 (else MOE_ERR_BATCH).                                   */
#define MOE_PREFILL_MAX_TOKENS 65536

/* Bytes of device workspace moe_prefill_layer needs for `tokens` tokens on this layer
 * (logits, the selection, the sorted pairs, h and y: about tokens * (k + S) * (2 I + 4 H)
 * bytes).  Host only.                                                                 */
int moe_prefill_workspace_bytes(moe_layer_t layer, int tokens, size_t* bytes);

/* Enqueues the prefill of `tokens` tokens on `stream` (seven kernels, no host sync, no
 * allocation).  x, router_w, expert_packed, scales, shared_w as for moe_decode_layer;
 * x and out bf16 [tokens][H], out must not overlap x.  workspace: device, 16-byte
 * aligned, at least moe_prefill_workspace_bytes(layer, tokens) bytes, owned by the
 * caller and not read after the call's kernels end.  topk_ids / topk_w: optional device
 * int32 / fp32 [tokens][k] copies of the selection (selection order) and its weights,
 * or NULL.  Deterministic: fixed summation orders, no atomics.  The layer's handle
 * workspace is not used: prefill calls do not disturb the decode calls' state.        */
int moe_prefill_layer(moe_layer_t layer, const void* x, const void* router_w,
                      const void* expert_packed, const void* scales, const void* shared_w,
                      void* out, int tokens, void* workspace, size_t workspace_bytes,
                      int32_t* topk_ids, float* topk_w, void* stream);

/* Test hook: which kernels run the handle's later calls.  MOE_PATH_AUTO (the default)
 * takes the kernels dedicated to the Flint shape where the layer has them (NVFP4 or
 * 2-bit routed and NVFP4 shared experts, sigmoid router, a device with at least 256
 * compute units): the batch-1 kernel with a wavefront per expert, and the batch 2-8
 * kernel; every other layer runs the general kernel.  MOE_PATH_GENERAL always takes the
 * general kernel, and is refused (MOE_ERR_UNSUPPORTED) for a 2-bit layer, which has no
 * general kernel.  Both compute the same layer (their sums run in different orders).
 * Returns the path
 * now in force through *active (may be NULL): MOE_PATH_DEDICATED or MOE_PATH_GENERAL.
 * Host-only; affects no call already made.                                           */
enum moe_path { MOE_PATH_AUTO = 0, MOE_PATH_GENERAL = 1, MOE_PATH_DEDICATED = 2 };
int moe_layer_set_path(moe_layer_t layer, int path, int* active);

/* Sticky error bits of the handle's calls so far, read synchronously (waits for the
 * device): 1 = a workgroup gave up waiting for router logits, 2 = for activations (the
 * grid was not resident at once), 4 = a wavefront gave up waiting for another of its
 * workgroup (batch-1 kernel).  clear != 0 resets them.
 * After a non-zero result the handle's later outputs are undefined until
 * moe_layer_reset.  These waits replace the kernel boundaries of the Flint page's
 * chained low-latency kernels ("From 1,096 kernels to 346").                         */
int moe_layer_error(moe_layer_t layer, unsigned* flags, int clear);

/* Waits for the device and returns the handle's workspace to its state after
 * moe_layer_create (call counter 0, no error bits, no last call).  Host-synchronous;
 * MOE_ERR_DEVICE if the device fails.                                                */
int moe_layer_reset(moe_layer_t layer);

/* Launch plan of the handle: workgroups of its kernel (all resident at once, the one
 * launch that stands for the Flint page's chain of layer kernels, "From 1,096 kernels
 * to 346") and the shared-memory bytes each uses at max_batch.  Either pointer may be
 * NULL.  Host only.                                                                   */
int moe_layer_grid(moe_layer_t layer, int* workgroups, int* lds_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
