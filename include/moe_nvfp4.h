/*
 * moe_nvfp4.h - fused Mixture-of-Experts layer with NVFP4 expert weights, for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What the layer computes (the page "Serving Solar Open 2 on DGX Spark",
 * backend.ai, 2026-07):
 *   - section "Solar Open 2 개요": routed experts plus one shared expert, top-k
 *     routing (320 routed, 1 shared, top-8 in the served model);
 *   - section "수정 사항 › b12x에서의 Expert Parallelism 구현 추가": each device
 *     holds a contiguous shard [local_expert_offset, local_expert_offset +
 *     num_local_experts) of the routed experts; globally routed expert ids are
 *     mapped to shard-relative indices and token-expert pairs outside the shard
 *     are dropped; the output is this shard's partial sum, which the caller adds
 *     up across shards with an ordinary all-reduce; the weight tensors of a
 *     shard may start at any expert (every expert's codes and scales span a
 *     multiple of 16 bytes, so a slice of an aligned tensor stays aligned); one
 *     scratch pool serves every layer;
 *   - section "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기": expert
 *     weights are packed FP4 codes, FP8 (E4M3) block scales clamped to 448 and a
 *     per-expert fp32 global scale, with gate and up projections fused into one
 *     weight (w13).
 *
 * Forward, per token t with hidden row x_t (bf16, d_model wide):
 *   logits_e = x_t . gate_w[e]            for ALL num_experts experts (global)
 *   ids      = the top_k experts by logit, descending (equal logits: lower id)
 *   w_j      = softmax over the top_k selected logits (= full softmax renormalised)
 *   keep pair (t, j) iff 0 <= ids_j - local_expert_offset < num_local_experts
 *   h_t      = x_t (W4A16)  or  NVFP4-quantize-dequantize(x_t) (W4A4, static W4A4)
 *   expert MLP:  u = W13 h (2*d_ff outputs), a = silu(u[0:F]) * u[F:2F],
 *                (W4A4: a = NVFP4-quantize-dequantize(a)),  y = W2 a
 *   out_t    = sum over kept pairs of w_j * y  +  has_shared * y_shared(h_t)
 * Weights are never renormalised inside a shard, so the shards' outputs sum to
 * the unsharded output.
 *
 * NVFP4 (NVIDIA's format): an element is an E2M1 code (4 bits, bit 3 = sign,
 * values {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}); two codes per byte, the
 * even element in the low nibble; one E4M3fn scale byte per 16 consecutive
 * elements along the reduction (K) axis; one fp32 global scale per tensor.  A
 * weight decodes as  code * e4m3(scale) * global  (global is a multiplier).
 * W4A4 activations use the same element/scale format with no global scale:
 * scale = E4M3_rne_saturating(block_amax / 6), code = E2M1_rne_saturating(x / scale).
 * Static W4A4 (the page's third fused-MoE backend variant, "static" NVFP4 W4A4:
 * a calibrated activation scale fixed ahead of time) gives each of the two
 * quantization points a per-layer fp32 activation global g_a (act_global13 for
 * h, act_global2 for a), applied like a weight's global:
 * scale = E4M3(block_amax / (6 g_a)), code = E2M1(x / (scale g_a)), value =
 * code * scale * g_a; blocks beyond 6 * 448 * g_a saturate.
 *
 * Numerics: code * scale is exact in bf16 (and in f16); the GEMMs run on bf16
 * MFMA (W4A16) or f16 MFMA on the tiled path in W4A4, where both operands are
 * such products, with fp32 accumulation, and apply the fp32 global scale after
 * accumulation.  Routing is exact: up to 128 tokens the logits are fp64 sums of
 * the exact bf16 x bf16 products (fp64 matrix cores); beyond, bf16-MFMA logits
 * carry a rigorous error bound, and every expert that could be on either side
 * of the top-k boundary is re-scored in fp64.  Either way the result is
 * deterministic.
 *
 * Conventions of every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP), caller-owned, row-major,
 *     dense; bf16 tensors, FP4 codes and E4M3 scales 16-byte aligned, fp32 and
 *     int32 tensors 4-byte aligned (MOE_NVFP4_ERR_INVALID_ARG otherwise for the
 *     weights).
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream); no
 *     host synchronisation, no allocation, no hidden global state.  Inputs are
 *     never modified.
 *   - The workspace is caller-owned device memory of at least
 *     moe_nvfp4_workspace_size() bytes (256-byte aligned); its contents are
 *     undefined after a call; calls that share a workspace must not overlap.
 *   - Argument errors are reported before anything is enqueued.  A HIP launch
 *     failure returns MOE_NVFP4_ERR_HIP.  No exception crosses the ABI.
 *     moe_nvfp4_last_error() gives a message for the calling thread.
 *
 * Three layout choices differ from the most literal form of the operation
 * (logits = hidden x gate_w with gate_w as a [d_model][E] matrix; one array of
 * (w13, w2) global-scale pairs; any d_ff that is a multiple of the 16-element
 * block):
 *   - gate_w is [E][d_model], one contiguous row per routed expert, so that the
 *     router streams each expert's row along K like the token rows (the [d][E]
 *     matrix is its transpose; the logits are the same);
 *   - the global scales are two fp32 arrays, w13_global[n] and w2_global[n],
 *     one per GEMM, instead of one interleaved [n][2] array: each GEMM reads
 *     one contiguous array, and a shard's slice is a pointer offset in each;
 *   - d_model and d_ff must be multiples of 128 (not only of 16): both kernel
 *     paths cover 128 SwiGLU columns (and 128 K elements) per unit of work.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_NVFP4_W4A16 = 0,   /* NVFP4 weights, bf16 activations                     */
    MOE_NVFP4_W4A4  = 1,   /* NVFP4 weights, activations NVFP4-quantized online   */
    MOE_NVFP4_W4A4_STATIC = 2  /* as W4A4, with calibrated activation globals      */
} moe_nvfp4_mode;

typedef enum {
    MOE_NVFP4_OK = 0,
    MOE_NVFP4_ERR_INVALID_ARG = 1,        /* null pointer, bad offset/count, unknown mode */
    MOE_NVFP4_ERR_UNSUPPORTED_SHAPE = 2,  /* dims outside what the kernels tile          */
    MOE_NVFP4_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_NVFP4_ERR_ARCH = 4,               /* device is not gfx950                         */
    MOE_NVFP4_ERR_HIP = 5                 /* a HIP runtime call or launch failed          */
} moe_nvfp4_status;

/* Kernel path.  AUTO picks from the expected number of local pairs per local
 * expert, T * top_k / num_experts (the shard's expected load, not the global
 * one), with crossovers measured on the 4096 x 1024 layer:
 *   W4A16 with d_model % 256 == 0: block-diagonal weight streaming (DECODE) up
 *     to 3.9, dense weight streaming (MID) up to 64, tiles (PREFILL) above;
 *   W4A4 with d_model and d_ff multiples of 256, at most 8192 (the activations
 *     then travel as NVFP4): DECODE up to 5, MID up to 18, PREFILL above;
 *   W4A4 with d_model and d_ff multiples of 256 above 8192: DECODE up to 6,
 *     PREFILL above;
 *   any other shape: DECODE up to 9, PREFILL above.
 * AUTO never takes MICRO.  Every path gives results within the stated
 * tolerances; they are not bit-identical to each other. */
typedef enum {
    MOE_NVFP4_PATH_AUTO = 0,
    MOE_NVFP4_PATH_DECODE = 1,   /* weight streaming, block-diagonal MFMA, 4-16-row tiles */
    MOE_NVFP4_PATH_PREFILL = 2,  /* 256 x 256 MFMA tiles                                  */
    MOE_NVFP4_PATH_MID = 3,      /* weight streaming, dense MFMA, 16/32-row tiles; needs
                                    d_model % 256 == 0 (else UNSUPPORTED_SHAPE)          */
    MOE_NVFP4_PATH_MICRO = 4     /* the whole layer in one persistent launch (one
                                    workgroup per CU, grid barriers) for 1..16 tokens;
                                    needs d_model, d_ff <= 4096, d_model % 256 == 0, and
                                    the device otherwise idle for the launch's duration
                                    (its barriers wait for every CU's workgroup).  The
                                    waits are bounded: if one expires the kernel still
                                    ends, but `out` is then undefined (the 32-bit word
                                    at byte offset 4 of the workspace is then non-zero) */
} moe_nvfp4_path;

typedef struct {
    int32_t num_tokens;           /* T >= 0                                             */
    int32_t d_model;              /* d: multiple of 128, 128..16384                      */
    int32_t d_ff;                 /* F: multiple of 128, 128..16384                      */
    int32_t num_experts;          /* E: routed experts of the whole model, 1..1024       */
    int32_t top_k;                /* k: 1..min(E, 32)                                    */
    int32_t local_expert_offset;  /* o >= 0: global id of this shard's first expert      */
    int32_t num_local_experts;    /* L >= 1, o + L <= E                                  */
    int32_t has_shared;           /* 1: this call adds the shared expert (weight 1)      */
    int32_t mode;                 /* moe_nvfp4_mode                                      */
    int32_t path;                 /* moe_nvfp4_path                                      */
    float act_global13;           /* static W4A4: activation global of h (GEMM1 input);  */
    float act_global2;            /*   of a (GEMM2 input); finite, 2^-100..2^100.        */
                                  /*   Ignored in the other modes.                       */
} moe_nvfp4_problem;

/* NVFP4 weights of n experts (n = num_local_experts, or 1 for the shared
 * expert), expert-major.  w13 rows [0, F) are the gate projection, rows [F, 2F)
 * the up projection. */
typedef struct {
    const uint8_t *w13;         /* [n][2F][d/2]   E2M1 codes                       */
    const uint8_t *w13_scale;   /* [n][2F][d/16]  E4M3 block scales                */
    const float   *w13_global;  /* [n]            fp32 global scale (multiplier)   */
    const uint8_t *w2;          /* [n][d][F/2]    E2M1 codes                       */
    const uint8_t *w2_scale;    /* [n][d][F/16]   E4M3 block scales                */
    const float   *w2_global;   /* [n]                                             */
} moe_nvfp4_weights;

/* Bytes of workspace moe_nvfp4_forward / moe_nvfp4_route need for `p`.
 * Device-free.  Returns OK, or INVALID_ARG / UNSUPPORTED_SHAPE for a bad problem. */
int moe_nvfp4_workspace_size(const moe_nvfp4_problem *p, size_t *bytes);

/* Device-free validation of a problem against a workspace size and a device
 * architecture name (e.g. "gfx950:sramecc+:xnack-"; NULL skips the check).
 * Returns the status moe_nvfp4_forward would return for these arguments
 * (given non-null tensor pointers). */
int moe_nvfp4_validate(const moe_nvfp4_problem *p, size_t workspace_bytes, const char *arch);

/* The kernel path moe_nvfp4_forward takes for `p` (p->path itself unless it
 * is AUTO, else the rule above resolves it).  Device-free.  Writes it to
 * *path and returns OK, or INVALID_ARG / UNSUPPORTED_SHAPE for a bad problem. */
int moe_nvfp4_resolved_path(const moe_nvfp4_problem *p, int32_t *path);

/* The fused layer: out = this shard's partial sum (bf16 [T][d], fully
 * overwritten; a token with no local pair gets the shared term or 0).
 *   hidden  bf16 [T][d]
 *   gate_w  bf16 [E][d]     router weight, one row per routed expert (global)
 *   local   weights of experts o .. o+L-1 (pointers to the shard's first expert)
 *   shared  weights of the shared expert (n = 1); NULL iff has_shared == 0
 */
int moe_nvfp4_forward(const moe_nvfp4_problem *p, const void *hidden, const void *gate_w,
                      const moe_nvfp4_weights *local, const moe_nvfp4_weights *shared,
                      void *workspace, size_t workspace_bytes, void *out, void *stream);

/* moe_nvfp4_forward that also records caller-owned HIP events (hipEvent_t; NULL
 * entries are skipped) on `stream` at the boundaries of the layer's kernels, for
 * per-kernel timing with hipEventElapsedTime:
 *   events[0] before routing          events[1] after routing + permutation
 *   events[2] after the W4A4 hidden quantizer (== events[1] for W4A16)
 *   events[3] after GEMM1 + SwiGLU    events[4] after GEMM2    events[5] after combine
 * num_events may be 0..6; the computation is identical to moe_nvfp4_forward. */
int moe_nvfp4_forward_timed(const moe_nvfp4_problem *p, const void *hidden, const void *gate_w,
                            const moe_nvfp4_weights *local, const moe_nvfp4_weights *shared,
                            void *workspace, size_t workspace_bytes, void *out, void *stream,
                            void *const *events, int num_events);

/* moe_nvfp4_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the scratch is a library-owned device array of
 * MOE_NVFP4_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held from the first call
 * on a device until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the caller passes inputs and outputs
 * as for moe_nvfp4_forward, and the result is the same.
 *   - A problem whose workspace (moe_nvfp4_workspace_size) exceeds the scratch
 *     returns MOE_NVFP4_ERR_WORKSPACE_TOO_SMALL before anything is enqueued
 *     (e.g. the 4096 x 1024, 320-expert layer fits up to a few hundred tokens).
 *   - Every call on one device shares that device's scratch: calls that overlap
 *     on one device (other streams, other host threads) race and must be
 *     serialized by the caller.  Nothing is assumed of the scratch's previous
 *     contents: each call clears what it needs with kernels.
 * Other statuses as for moe_nvfp4_forward. */
#define MOE_NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_nvfp4_forward_noalloc(const moe_nvfp4_problem *p, const void *hidden, const void *gate_w,
                              const moe_nvfp4_weights *local, const moe_nvfp4_weights *shared,
                              void *out, void *stream);

/* Routing and permutation only (the first steps of the forward), for checking:
 *   topk_ids  int32 [T][k]   global expert ids, slot 0 = largest logit
 *   topk_w    fp32  [T][k]   routing weights (sum to 1 per token)
 *   counts    int32 [L]      kept pairs per local expert
 *   offsets   int32 [L+1]    exclusive scan of counts; offsets[L] = P
 *   perm      int32 [T*k]    first P entries: kept pair ids t*k+j sorted by
 *                            (local expert, token); the rest is left untouched
 * Any of topk_ids/topk_w/counts/offsets/perm may be NULL to skip that output. */
int moe_nvfp4_route(const moe_nvfp4_problem *p, const void *hidden, const void *gate_w,
                    int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets,
                    int32_t *perm, void *workspace, size_t workspace_bytes, void *stream);

/* NVFP4 quantization of n weight tensors (the preparation of inputs that the
 * forward consumes; rule of the workload recipe):
 *   global[i] = amax(tensor i) / (6 * 448)  (1 if the tensor is all zero), fp32
 *   scale     = E4M3_rne_sat(block_amax / (6 * global))      (fp32 arithmetic)
 *   code      = E2M1_rne_sat(w / (scale * global))            (0 where scale = 0)
 *   w       bf16 [n][R][C]   (C multiple of 16)
 *   codes   u8   [n][R][C/2];  scales u8 [n][R][C/16];  global fp32 [n]       */
int moe_nvfp4_quantize_weights(const void *w, int32_t n, int32_t R, int32_t C, uint8_t *codes,
                               uint8_t *scales, float *global, void *stream);

/* W4A4 activation quantizer alone (the step the forward applies to `hidden`):
 *   scale = E4M3_rne_sat(block_amax / 6), code = E2M1_rne_sat(x / scale)
 *   x bf16 [R][C] (C multiple of 16) -> codes u8 [R][C/2], scales u8 [R][C/16]  */
int moe_nvfp4_quantize_activations(const void *x, int32_t R, int32_t C, uint8_t *codes,
                                   uint8_t *scales, void *stream);

/* Static W4A4 activation quantizer alone, with the calibrated global g (finite,
 * 2^-100..2^100; g = 1 gives moe_nvfp4_quantize_activations):
 *   scale = E4M3_rne_sat(block_amax / (6 g)), code = E2M1_rne_sat(x / (scale g)),
 *   fp32 products and correctly rounded divisions; a block whose scale is 0
 *   gets zero codes.  Shapes as above. */
int moe_nvfp4_quantize_activations_static(const void *x, int32_t R, int32_t C, float g, uint8_t *codes,
                                          uint8_t *scales, void *stream);

/* Checkpoint preparation (the page "Serving Solar Open 2 on DGX Spark", section
 * "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기": pre-quantized NVFP4
 * checkpoints hold packed FP4 weights, FP8 block scales and per-expert global
 * scales, in one of two conventions for the global scale; the loader reads
 * either, handles the fused gate/up row order and slices the scales of an
 * expert shard).  The prepared tensors are the layout moe_nvfp4_weights
 * describes.
 *
 * Global scale conventions of a checkpoint tensor:
 *   MULTIPLIER  w = e2m1 * e4m3 * g          (g stored as is)
 *   INVERSE     w = e2m1 * e4m3 / g_stored   (prepared g = fp32(1 / g_stored),
 *                                             one correctly rounded division)
 * Gate/up row order of a checkpoint's fused w13:
 *   GATE_UP     rows [0, F) gate, [F, 2F) up  (copied as is)
 *   UP_GATE     rows [0, F) up,   [F, 2F) gate (the two halves are swapped)
 * Codes and block scales are copied bit for bit (no re-rounding). */
typedef enum { MOE_NVFP4_GLOBAL_MULTIPLIER = 0, MOE_NVFP4_GLOBAL_INVERSE = 1 } moe_nvfp4_global_convention;
typedef enum { MOE_NVFP4_GATE_UP = 0, MOE_NVFP4_UP_GATE = 1 } moe_nvfp4_w13_order;

/* A checkpoint's expert tensors (device pointers; num_experts experts,
 * expert-major, the moe_nvfp4_weights shapes, w13 in w13_order). */
typedef struct {
    const uint8_t *w13;         /* [E][2F][d/2]                                     */
    const uint8_t *w13_scale;   /* [E][2F][d/16]                                    */
    const float   *w13_global;  /* [E] in global_convention                          */
    const uint8_t *w2;          /* [E][d][F/2]                                      */
    const uint8_t *w2_scale;    /* [E][d][F/16]                                     */
    const float   *w2_global;   /* [E] in global_convention                          */
    int32_t num_experts, d_model, d_ff;
    int32_t global_convention;  /* moe_nvfp4_global_convention                        */
    int32_t w13_order;          /* moe_nvfp4_w13_order                                */
} moe_nvfp4_checkpoint;

/* Writes experts [first_expert, first_expert + count) of `ck` into `dst`
 * (caller-owned device tensors for `count` experts, the moe_nvfp4_weights
 * layout; they must not overlap the checkpoint's).  d_model and d_ff follow the
 * forward's rules; 0 <= first_expert, first_expert + count <= num_experts,
 * count <= 65535 (count == 0 enqueues nothing); pointers as in the forward
 * (16-byte aligned codes and scales, 4-byte aligned globals).  Enqueued on
 * `stream`; returns INVALID_ARG / UNSUPPORTED_SHAPE before enqueuing anything,
 * ARCH when the current device is not gfx950, HIP when a launch fails. */
int moe_nvfp4_prepare(const moe_nvfp4_checkpoint *ck, int32_t first_expert, int32_t count,
                      const moe_nvfp4_weights *dst, void *stream);

/* Static description of a status code. */
const char *moe_nvfp4_strerror(int status);

/* Message describing the last error returned on the calling thread ("" if none). */
const char *moe_nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
