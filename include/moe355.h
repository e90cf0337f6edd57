/*
 * libmoe355 -- fused Mixture-of-Experts layer forward for AMD Instinct MI355X
 * (CDNA4, gfx950).  C ABI.
 *
 * The method: the five-stage FusedMoE chain of Tencent's HPC-Ops
 * ("HPC-Ops" overview page, sections "Main functions" and "Technical
 * principles"): routing index -> Gate-Up GEMM -> activation quantisation ->
 * Down GEMM -> top-k weighted combine, with the split-BF16 router GEMM as an
 * optional front end, for a Hy4-preview style block (PR #54160 report,
 * "Features and motivation": 256 routed experts, top-8, plus one shared
 * expert).
 *
 * Conventions for every call
 *  - Array pointers are DEVICE pointers unless stated otherwise; arrays are
 *    row-major and contiguous.  bf16 is carried as uint16_t bit patterns,
 *    FP8 as uint8_t codes in OCP E4M3FN (max 448, no infinities).
 *  - The caller allocates and owns every buffer, including workspaces whose
 *    size the *_workspace_bytes queries return.  The library allocates no
 *    device memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Calls are asynchronous on that stream.
 *  - Every call validates its arguments on the host before enqueuing
 *    anything and returns a status: on error nothing is launched.  A call
 *    with T == 0 (or zero rows) returns MOE_OK and enqueues nothing.  No C++
 *    exception crosses the ABI.  Shapes outside the compiled envelope are
 *    refused with MOE_EUNSUPPORTED; there is no silent fallback path.
 *  - Stateless and re-entrant.  For fixed inputs and shapes every output is
 *    bitwise identical from run to run (no floating-point atomics).
 *
 * Symbols used below: T tokens, H hidden size, E routed experts, k experts
 * per token, I expert intermediate size, S in {0,1} shared experts.
 * P = T*k routed (token, rank) pairs, pair index p = t*k + j.
 * R = P + S*T rows in "slot space": slots [0,P) are grouped by expert
 * (group e owns slots [offsets[e], offsets[e+1])), slots [P, P+T) belong to
 * the shared expert (group E) in token order.
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE355_ABI_VERSION 4

enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* NULL required pointer, negative size, k > E, overlapping outputs */
  MOE_EUNSUPPORTED = 2,  /* outside the envelope: H or I not a multiple of 128, E > 1024,
                            k > 32, R >= 2^31, unknown dtype */
  MOE_EWORKSPACE = 3,    /* workspace NULL or smaller than the query returned */
  MOE_EDEVICE = 4        /* a HIP error reported right after a launch */
};

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };  /* y_dtype */
enum { MOE_W_BF16 = 0, MOE_W_FP8 = 1, MOE_W_MXFP8 = 2, MOE_W_FP8_TENSOR = 3 };   /* moe_experts_t.wtype */

int moe_abi_version(void);
const char* moe_status_string(int status);

/* ------------------------------------------------------------------ router
 * Split-BF16 router (HPC-Ops page, "Router GEMM" in main functions and
 * technical principles): fp32 router weights are split offline into a high
 * bf16 part and a residual bf16 part with scale 1/256, and the logits are two
 * bf16 GEMMs combined linearly in one kernel with one FMA in the epilogue.
 *
 * moe_router_split (offline):  w fp32 [E,H] -> w_hi, w_lo bf16 [E,H] with
 *   w_hi = bf16_rne(w), w_lo = bf16_rne((w - w_hi) * 256).
 * moe_router_gemm:  x bf16 [T,H], w_hi, w_lo [E,H] -> logits fp32 [T,E],
 *   logits = fma(x.w_lo^T, 1/256, x.w_hi^T), both products accumulated in
 *   fp32 on the bf16 matrix cores; x is read once.  H % 128 == 0, E <= 1024.
 */
int moe_router_split(const float* w, uint16_t* w_hi, uint16_t* w_lo, int E, int H, void* stream);
int moe_router_gemm(const uint16_t* x, const uint16_t* w_hi, const uint16_t* w_lo, float* logits,
                    int64_t T, int H, int E, void* stream);

/* ------------------------------------------------------------------ stage 1: route
 * Routing index (HPC-Ops page, FusedMoE stage 1).  Per token t:
 *   l'[e] = logits[t,e] + bias[e] (fp32 add) if bias != NULL and
 *           (bias_rows == NULL or bias_rows[t] != 0), else logits[t,e];
 *   topk_ids[t, 0..k-1] = the k experts with the largest l', ordered by
 *           value descending, ties to the lower expert id;
 *   topk_w[t, j] = exp(l'_j - l'_0) / sum_i exp(l'_i - l'_0)  (softmax over
 *           the k selected values; no capacity limit, nothing dropped).
 * logits fp32 [T,E]; bias fp32 [E] or NULL; bias_rows uint8 [T] or NULL;
 * topk_ids int32 [T,k]; topk_w fp32 [T,k].  1 <= k <= min(E, 32), E <= 1024.
 */
int moe_route(const float* logits, const float* bias, const uint8_t* bias_rows, int64_t T, int E,
              int k, int32_t* topk_ids, float* topk_w, void* stream);

/* ------------------------------------------------------------------ stage 1b: align
 * Per-expert histogram in LDS, exclusive prefix sum, and a contiguous output
 * interval per expert (HPC-Ops page, technical principles: FusedMoE routing
 * stage).  Slots inside an interval follow ascending pair index, hence
 * ascending token (a token's k experts are distinct).
 *   counts int32 [E]; offsets int32 [E+2]: offsets[e] = sum_{e'<e} counts[e'],
 *   offsets[E] = P, offsets[E+1] = P + shared*T;
 *   slot_pair int32 [P]: pair stored in slot s; pair_slot int32 [P]: inverse.
 * ws: device scratch of moe_align_workspace_bytes(T, E, k) bytes (may be 0;
 * ws may then be NULL).  topk_ids must hold valid ids in [0,E) with k
 * distinct ids per token (the output of moe_route); other input is undefined
 * behaviour.
 */
size_t moe_align_workspace_bytes(int64_t T, int E, int k);
int moe_align(const int32_t* topk_ids, int64_t T, int E, int k, int shared, int32_t* counts,
              int32_t* offsets, int32_t* slot_pair, int32_t* pair_slot, void* ws, size_t ws_bytes,
              void* stream);

/* ------------------------------------------------------------------ FP8 helpers
 * OCP E4M3FN, round to nearest even, saturating at +-448.  Scale of a
 * group/block = amax / 448 in fp32 (1 when amax == 0); code = e4m3(fp32(v / s)).
 * moe_quant_rows_fp8: activations, per row per group of 128 columns
 *   (x bf16 [rows,cols] -> q [rows,cols], s fp32 [rows, cols/128]).
 * moe_quant_blocks_fp8 (offline): weights with 128x128 block scales, the
 *   checkpoint format named in the PR #54160 report (implementation item 4)
 *   (w bf16 [mats,rows,cols] -> q [mats,rows,cols], s fp32 [mats, rows/128, cols/128]).
 * rows/cols of a block-quantised matrix and cols of a row-quantised one must be
 * multiples of 128.
 */
int moe_quant_rows_fp8(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s, void* stream);
int moe_quant_blocks_fp8(const uint16_t* w, int64_t mats, int rows, int cols, uint8_t* q, float* s,
                         void* stream);

/* ------------------------------------------------------------------ MXFP8 helper
 * MXFP8, the microscaling FP8 format the PR #54160 report lists beside the
 * 128x128 blockwise scales (implementation item 4), as the OCP Microscaling
 * definition gives it: per row, every 32 consecutive columns share an E8M0
 * scale byte X + 127 with X = floor(log2(amax)) - 8 clamped to [-127, 127]
 * (-127 for an all-zero block); codes are E4M3FN(v * 2^-X), round to nearest
 * even, saturating at +-448.
 * moe_quant_rows_mxfp8: x bf16 [rows,cols] -> q [rows,cols], s uint8
 *   [rows, cols/32].  Used for activations (K along the columns) and, offline,
 *   for weights stored with K along the rows' columns (w1, w3 as [E*I, H], w2
 *   as [E*H, I]).  cols must be a multiple of 32; x 16-byte and q 8-byte
 *   aligned; x, q and s must not overlap.
 */
int moe_quant_rows_mxfp8(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* s, void* stream);

/* ------------------------------------------------------------------ per-tensor FP8 helpers
 * The per-tensor FP8 mode of the HPC-Ops page's GroupGEMM (main functions:
 * per-tensor as well as block-wise FP8): one fp32 scale per tensor.  x holds
 * mats tensors of n values each (dtype MOE_DTYPE_BF16 or MOE_DTYPE_F32).
 * moe_tensor_amax: amax[m] = max |x| over tensor m (fp32).  The call zeroes
 *   amax first; the result does not depend on the order of the partial
 *   maxima.
 * moe_quant_tensor_fp8: s[m] = amax[m] / 448 in fp32 (1 when amax[m] == 0),
 *   q = e4m3(fp32(v / s[m])) (round to nearest even, saturating), from an amax
 *   computed by moe_tensor_amax or by the per-tensor Gate-Up GEMM.
 * Used offline for expert weights (w1, w3, w2 as E tensors of I*H values, the
 * shared ones as 1), on the hot path for x (1 tensor of T*H values) and for
 * h (1 tensor of R*I fp32 values).  n must be a multiple of 128 and
 * mats <= 65535 (MOE_EUNSUPPORTED); x 16-byte, q 8-byte, amax and s 4-byte
 * aligned; q and s must overlap neither x nor each other (MOE_EINVAL).
 */
int moe_tensor_amax(const void* x, int dtype, int64_t mats, int64_t n, float* amax, void* stream);
int moe_quant_tensor_fp8(const void* x, int dtype, int64_t mats, int64_t n, const float* amax, uint8_t* q, float* s,
                         void* stream);

/* ------------------------------------------------------------------ experts
 * SwiGLU experts: h = SiLU(x.w1^T) * (x.w3^T) (w1 = gate, w3 = up),
 * y = h.w2^T.  Routed: w1, w3 [E,I,H], w2 [E,H,I].  Shared expert (if
 * has_shared): sw1, sw3 [I,H], sw2 [H,I].  wtype MOE_W_BF16: bf16 weights,
 * scale pointers ignored.  wtype MOE_W_FP8: e4m3 codes plus fp32 128x128 block
 * scales s1, s3 [E,I/128,H/128], s2 [E,H/128,I/128], ss1, ss3 [I/128,H/128],
 * ss2 [H/128,I/128].  wtype MOE_W_MXFP8: e4m3 codes plus uint8 E8M0 scales per
 * weight row per 32 K (moe_quant_rows_mxfp8): s1, s3 [E,I,H/32], s2
 * [E,H,I/32], ss1, ss3 [I,H/32], ss2 [H,I/32].  wtype MOE_W_FP8_TENSOR: e4m3
 * codes plus one fp32 scale per matrix (moe_quant_tensor_fp8): s1, s3, s2 [E],
 * ss1, ss3, ss2 [1].  MXFP8 and per-tensor scale pointers must be 4-byte
 * aligned (MOE_EINVAL otherwise) and H a multiple of 256 (MOE_EUNSUPPORTED
 * otherwise).  For these two types x [T,H] and h [R,I] must also each hold
 * fewer than 2^31 elements, and H, I be below 2^23 (MOE_EUNSUPPORTED
 * otherwise); bf16 and block-scaled fp8 take any such shape.  The struct
 * itself is host memory; the pointers in it are device pointers.
 */
typedef struct moe_experts_t {
  int wtype;
  int E, H, I, has_shared;
  const void *w1, *w3, *w2;
  const void *s1, *s3, *s2;     /* fp32 (MOE_W_FP8, MOE_W_FP8_TENSOR) or uint8 E8M0 (MOE_W_MXFP8) */
  const void *sw1, *sw3, *sw2;
  const void *ss1, *ss3, *ss2;
} moe_experts_t;

/* ------------------------------------------------------------------ stages 2-3: Gate-Up GEMM
 * Grouped Gate-Up GEMM with SwiGLU (and, for FP8, the activation
 * requantisation stage fused into its epilogue).  For every slot s of group
 * g (HPC-Ops page, technical principles: the Gate-Up GEMM reads the input
 * directly through the routing index, with no separate gather copy):
 *   t = slot_pair[s] / k for routed slots, t = s - P for shared slots;
 *   h[s] = SiLU(x[t].w1[g]^T) * (x[t].w3[g]^T), fp32 accumulation.
 * bf16: x bf16 [T,H], xs NULL, h bf16 [R,I], hs NULL.
 * fp8:  x e4m3 [T,H] with xs fp32 [T,H/128] (moe_quant_rows_fp8); partial
 *   sums over each 128-wide K block are scaled by xs[t,kb] * s[g,n/128,kb];
 *   h is requantised per row per 128 columns into h e4m3 [R,I] and hs fp32
 *   [R,I/128] with the same rule as moe_quant_rows_fp8.
 * mxfp8: x e4m3 [T,H] with xs uint8 [T,H/32] (moe_quant_rows_mxfp8, 4-byte
 *   aligned); the matrix cores apply the E8M0 scales of both operands per 32 K;
 *   h is requantised per row per 32 columns with the same rule as
 *   moe_quant_rows_mxfp8 into h e4m3 [R,I] and hs uint8 [R,I/32].
 * per-tensor fp8: x e4m3 [T,H] with xs fp32 [1] (moe_quant_tensor_fp8 of the
 *   whole x); the code products summed over the whole K are scaled by
 *   xs[0] * s1[g] (s3[g] for the up half).  A per-tensor scale needs the amax
 *   of the whole h before any code, so this stage writes h unquantised, fp32
 *   [R,I], and hs fp32 [1] receives max |h|; moe_quant_tensor_fp8(h,
 *   MOE_DTYPE_F32, 1, R*I, hs, ...) then gives the codes and scale that
 *   moe_gemm2 takes.  xs and hs 4-byte aligned.
 * offsets, slot_pair: from moe_align.
 * ws: device scratch of moe_gemm_workspace_bytes bytes, 4-byte aligned; its
 *   contents need not be initialised (the call clears what it uses, on its
 *   stream).  The tiled Gate-Up kernels (bf16, MXFP8, per-tensor) may keep
 *   one counter per XCD in it, at which the workgroups of that XCD meet after
 *   every round of tiles so that tiles sharing a weight tile stream it
 *   through L2 together (used where groups average 1.5 row tiles or more).
 *   The waits are bounded, so the workspace affects timing only, never
 *   results; calls that may run concurrently should still use separate
 *   workspaces.  The per-tensor Gate-Up also clears the h amax word in hs.
 *   ws NULL or smaller than the query: MOE_EWORKSPACE; ws overlapping x or h
 *   or misaligned: MOE_EINVAL.
 */
size_t moe_gemm_workspace_bytes(const moe_experts_t* ex, int64_t T, int k);
int moe_gemm13(const moe_experts_t* ex, const void* x, const void* xs, const int32_t* offsets,
               const int32_t* slot_pair, int64_t T, int k, void* h, void* hs, void* ws,
               size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ stage 4: Down GEMM
 * y[s] = h[s].w2[g]^T for every slot s of group g (fp32 accumulation; fp8
 * partial sums per 128-wide K block scaled by hs[s,kb] * s2[g,n/128,kb];
 * mxfp8: hs uint8 [R,I/32], 4-byte aligned, scales applied per 32 K;
 * per-tensor fp8: h e4m3 [R,I], hs fp32 [1], sums over the whole K scaled by
 * hs[0] * s2[g]).
 * y is fp32 (y_dtype MOE_DTYPE_F32) or bf16 (MOE_DTYPE_BF16), [R,H].
 * ws, ws_bytes: reserved, unused (NULL and 0 are accepted).
 */
int moe_gemm2(const moe_experts_t* ex, const void* h, const void* hs, const int32_t* offsets,
              int64_t T, int k, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ stage 5: combine
 * Top-k weighted combine (HPC-Ops page, FusedMoE stage 5):
 *   out[t] = sum_{j=0..k-1} topk_w[t,j] * y[pair_slot[t*k+j]] + has_shared * y[P+t],
 * summed in that fixed order in fp32 and rounded once to bf16 (no atomics).
 * y [R,H] fp32 or bf16; out bf16 [T,H].
 */
int moe_combine(const void* y, int y_dtype, const int32_t* pair_slot, const float* topk_w, int64_t T,
                int k, int H, int has_shared, uint16_t* out, void* stream);

/* ------------------------------------------------------------------ combine + residual + RMSNorm
 * The combine above fused with a residual add and RMSNorm: the single-GPU half
 * of the HPC-Ops page's fused AllReduce+Norm (technical principles:
 * RMSNorm(AllReduce(x) + residual, weight); the all-reduce is the identity on
 * one GPU).  Per token t:
 *   s = combine(t) + residual[t]      (fp32; the combine sum is not rounded first)
 *   res_out[t] = bf16(s)              (optional, NULL to skip; may be residual itself)
 *   out[t] = bf16(s / sqrt(mean_H(s^2) + eps) * weight)
 * residual, out, res_out bf16 [T,H]; weight bf16 [H]; eps finite and >= 0.
 * H must be a multiple of 128 and at most 32768.  All arrays 16-byte aligned;
 * out overlaps nothing; res_out overlaps nothing except being exactly residual.
 */
int moe_combine_rmsnorm(const void* y, int y_dtype, const int32_t* pair_slot, const float* topk_w, int64_t T,
                        int k, int H, int has_shared, const uint16_t* residual, const uint16_t* weight, float eps,
                        uint16_t* out, uint16_t* res_out, void* stream);

/* ------------------------------------------------------------------ the whole chain
 * Convenience entry point that enqueues the chain on one stream:
 * [router_gemm] -> route -> align -> [quant x] -> gemm13 -> [quant h] -> gemm2 -> combine
 * (x and, for per-tensor FP8, h quantised as the weight type prescribes).
 * Either logits (fp32 [T,E]) or the split router weights (router_hi/lo bf16
 * [E,H]) must be given.  x bf16 [T,H]; out bf16 [T,H].  Every intermediate
 * lives in the caller's workspace (moe_forward_workspace_bytes bytes); the
 * layout of the workspace is private.  topk_ids/topk_w may be NULL; if given
 * ([T,k] each) the routing result is also copied there.
 */
typedef struct moe_forward_args_t {
  int64_t T;
  int k;
  int y_dtype;
  const uint16_t* x;
  const float* logits;
  const uint16_t* router_hi;
  const uint16_t* router_lo;
  const float* bias;
  const uint8_t* bias_rows;
  uint16_t* out;
  int32_t* topk_ids;
  float* topk_w;
} moe_forward_args_t;

size_t moe_forward_workspace_bytes(const moe_experts_t* ex, int64_t T, int k, int y_dtype);
int moe_forward(const moe_experts_t* ex, const moe_forward_args_t* args, void* ws, size_t ws_bytes,
                void* stream);

/* ------------------------------------------------------------------ the chain without a workspace
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): moe_forward
 * with every intermediate in a fixed device scratch array the library owns,
 * MOE_NOALLOC_SCRATCH_BYTES on each device it runs on (held until the process
 * ends).  The caller passes inputs and outputs only; the call allocates
 * nothing.  Same arguments (minus the workspace), checks, kernels and result
 * bits as moe_forward.  A shape whose moe_forward_workspace_bytes exceeds
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_EUNSUPPORTED with nothing enqueued
 * (e.g. decode-sized batches of 64 tokens at H = 6144 fit; prefill batches do
 * not).  Every call on a device uses that device's one scratch array: calls
 * that overlap on one device (other streams, other threads) race and give
 * undefined results; the caller must order them.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_experts_t* ex, const moe_forward_args_t* args, void* stream);

/* ------------------------------------------------------------------ the chain in one launch
 * Same arguments, workspace and result as moe_forward, bitwise: the stages run
 * as phases of one persistent kernel that hands out work items in chain order
 * from a counter in the workspace and signals readiness through device-side
 * counters (route -> align -> each 16-row chunk's Gate-Up tiles -> that
 * chunk's Down tiles -> each token's combine), the single-launch analogue of
 * the HPC-Ops page's PDL-chained FusedMoE stages (main functions: FusedMoE;
 * technical principles: PDL).  A Down tile fetches its first weight stages
 * before it waits for its h rows.  Enqueues a small clear kernel, then the
 * chain kernel ([router_gemm] first when logits is NULL).
 * Envelope: wtype MOE_W_BF16 and at most 16 routed rows per expert on average
 * (T*k <= 16*E); anything else returns MOE_EUNSUPPORTED with nothing enqueued.
 * When it pays (measured on MI355X): only for small batches launched eagerly,
 * where the host's launch rate is the bottleneck (16 tokens, H 256, E 8, top-2:
 * about 23 us against 38-45 us for five eager stage launches).  With the
 * stages replayed from a HIP graph, or from decode-sized batches on (64 tokens,
 * H 4096, E 256, top-8: 1.58 ms against 1.32 ms), moe_forward is faster: the
 * chain's device-side hand-overs cost more than graph launches, and its one
 * register allocation, sized for Gate-Up, leaves the Down phase fewer bytes in
 * flight than the stand-alone Down kernel.
 *
 * Residency: the chain kernel's grid is sized to what the device holds at
 * once, and it completes only if all of its workgroups are resident together
 * (waves wait on items that other waves of the grid hold).  The caller must
 * therefore not run other kernels on the device while the chain runs.  The
 * library orders its own chains: on each device, every call's stream first
 * waits for the previous call's chain (an event the library keeps), so chains
 * on different streams never overlap.  Calls made during a stream capture are
 * not ordered this way (the captured graph's own order applies); the caller
 * must not replay such a graph beside another chain.  If the device is
 * shared anyway, every device-side wait ends after about 0.67 s: the call has
 * already returned MOE_OK, out is undefined, and moe_forward_persistent_status
 * reports MOE_EDEVICE.  Two calls that share a workspace must not run
 * concurrently.
 */
int moe_forward_persistent(const moe_experts_t* ex, const moe_forward_args_t* args, void* ws, size_t ws_bytes,
                           void* stream);

/* Waits for `stream`, then reports whether the last moe_forward_persistent
 * call on workspace `ws` completed: MOE_OK, or MOE_EDEVICE when a device-side
 * wait ran out of time (about half a second; it means a device fault or a
 * bug, and out is then undefined).  MOE_EINVAL for a NULL workspace.
 */
int moe_forward_persistent_status(const void* ws, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_H */
