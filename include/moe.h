/*
 * moe.h -- C ABI of libmoe_mi355x.so: one small-batch decode Mixture-of-Experts layer
 * on one AMD Instinct MI355X (gfx950).
 *
 * The layer (what every page describes for its model):
 *   - an FP32 router GEMV with sigmoid top-k selection ("Inkling 2 Small on vLLM:
 *     Day-0 Support", accuracy evaluation: FP32 router; "Day 0 support for Mistral
 *     Large 4 on vLLM", breakable CUDA graphs and fusions: FP32 router GEMM;
 *     "vLLM Day-0 support for Recursive's Flint", architecture: sigmoid top-6 of 256
 *     experts plus one shared expert), or softmax top-k (Mistral Large 4 page, ROCm
 *     implementation details: the fused decode's softmax top-4 router);
 *   - gate/up and down projections that read only the selected experts' weights
 *     (Flint page, optimization strategy: small-batch MoE kernels), with SwiGLU;
 *   - block-scaled weights: NVFP4 (Inkling page, mixed-precision MoE), OCP MXFP4 and
 *     MXFP8 (Mistral Large 4 page, AMD section and ROCm implementation details);
 *   - optional in-kernel activation quantization: NVFP4 "Four Over Six" (Inkling page,
 *     Four-Over-Six NVFP4; MoE with fused activation quantization) or FP8-E4M3 with
 *     one scale per token (Mistral Large 4 page, MXFP4 experts, a8w4);
 *   - a weighted combine of the routed outputs plus the shared expert (Flint page,
 *     low-latency decode path: routing and expert combine fused into the GEMVs);
 *   - at load time, BF16 weights requantized to MXFP4 (Mistral Large 4 page, ROCm
 *     implementation details: experts requantized to MXFP4 one layer at a time) or NVFP4.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller (e.g. a torch tensor's
 *     data_ptr()). The library never allocates, frees or synchronizes inside
 *     moe_route, moe_expert_forward, moe_forward, quantize_nvfp4_4o6,
 *     moe_requant_mxfp4, moe_requant_mxfp8 or moe_requant_nvfp4; they enqueue
 *     kernels on `stream` and return.
 *   - Every entry returns a moe_status_t and never throws. Arguments are validated
 *     before anything is launched; on error nothing is enqueued and moe_last_error()
 *     returns a message (thread-local) naming every problem found.
 *   - A launch failure reported by the HIP runtime maps to MOE_ELAUNCH.
 *   - BF16 values are passed as uint16_t bit patterns; FP8 / E8M0 bytes as uint8_t.
 *   - Results are deterministic: repeated calls on the same inputs give identical bits.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, size, alignment            */
  MOE_EUNSUPPORTED = -2,  /* valid request this library does not implement          */
  MOE_EWORKSPACE = -3,    /* workspace missing or smaller than moe_workspace_bytes  */
  MOE_ELAUNCH = -4        /* the HIP runtime refused or failed a kernel launch      */
} moe_status_t;

/* Storage format of a weight tensor [rows][K], K contiguous. */
typedef enum {
  MOE_W_BF16 = 0,   /* codes: uint16 BF16 [rows][K]; no scales                         */
  MOE_W_NVFP4 = 1,  /* codes: E2M1 nibbles [rows][K/2], element 2i in the low nibble;
                       scales: E4M3 bytes [rows][K/16]; gscale: one FP32 per tensor    */
  MOE_W_MXFP4 = 2,  /* codes as NVFP4; scales: E8M0 bytes [rows][K/32]; no gscale       */
  MOE_W_MXFP8 = 3   /* codes: E4M3 bytes [rows][K]; scales: E8M0 bytes [rows][K/32]     */
} moe_wfmt_t;

/* Format the routed experts' activations (x before gate/up, h before down) take. */
typedef enum {
  MOE_A_BF16 = 0,        /* x used as given (BF16); h kept in FP32                      */
  MOE_A_NVFP4_4O6 = 1,   /* NVFP4 with a per-row FP32 global scale amax/2688 and a
                            Four-Over-Six E4M3 scale per 16 elements (NVFP4 weights only) */
  MOE_A_FP8_TOKEN = 2,   /* FP8-E4M3 with one FP32 scale amax/448 per row (MX weights)  */
  MOE_A_MXFP4 = 3,       /* OCP MXFP4 (a4w4): E2M1 with one E8M0 scale per 32 elements,
                            shared exponent floor(log2(block amax)) - 2 (MX weights; the
                            Mistral Large 4 page's ROCm specialized decode runs a4w4)      */
  MOE_A_MXFP8 = 4        /* OCP MXFP8: E4M3 with one E8M0 scale per 32, exponent
                            floor(log2(block amax)) - 8 (MX weights; the Inkling page's
                            MXFP8 layers quantize activations to their own format)       */
} moe_afmt_t;

/* How the router turns the selected logits into combine weights (the experts are always
 * the k largest selection keys, ties to the lower index):
 *   MOE_SCORE_SIGMOID: w_j = sigmoid(l_j) / sum sigmoid(l_j') over the selected
 *                      (the sigmoid top-k of the Flint and Inkling pages);
 *   MOE_SCORE_SOFTMAX: w_j = exp(l_j) / sum exp(l_j') over the selected, i.e. the
 *                      softmax over all experts renormalised to the selection (the
 *                      softmax top-k router of the Mistral Large 4 page's ROCm decode).
 * l is the logit plus the bias, or the bare logit with bias_select_only. */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score_t;

/* One stacked weight set: n experts x [rows][K]. Expert e's codes start at
 * codes + e * rows * (bytes per row); scales and gscale likewise. */
typedef struct {
  const void *codes;       /* see moe_wfmt_t; 16-byte aligned                           */
  const uint8_t *scales;   /* NVFP4 / MX: see moe_wfmt_t (NVFP4 16-byte, MX 4-byte
                              aligned); BF16: NULL                                       */
  const float *gscale;     /* NVFP4 only: FP32 [n][2] for w13 (gate, up), [n][1] for w2 */
} moe_weights_t;

/* Sizes: H, I and I_shared multiples of 32. With NVFP4 weights the GEMV walks also need
 * each K (H for gate/up, I or I_shared for down) to be a multiple of 256, or small enough
 * that a row's pieces form one batch of the walk; other sizes are refused
 * (MOE_EUNSUPPORTED, reported by moe_layer_check). */
typedef struct {
  int32_t H;            /* hidden size (K of gate/up, rows of down); multiple of 32      */
  int32_t I;            /* routed expert intermediate size; multiple of 32               */
  int32_t E;            /* routed experts, 1..1024                                       */
  int32_t k;            /* experts per token, 1..min(E, 16)                              */
  int32_t has_shared;   /* 1: one shared expert added with weight 1 to every token        */
  int32_t I_shared;     /* shared expert intermediate size; multiple of 32                */
  int32_t wfmt;         /* moe_wfmt_t of the routed experts                               */
  int32_t shared_wfmt;  /* moe_wfmt_t of the shared expert                                */
  int32_t afmt;         /* moe_afmt_t of the routed experts (the shared expert: BF16 x,
                           FP32 h)                                                        */
  const float *router_w;     /* FP32 [E][H]                                              */
  const float *router_bias;  /* FP32 [E], added to the logits before selection and
                                weighting (see bias_select_only), or NULL                 */
  moe_weights_t w13;    /* routed gate/up: [E][2I][H], gate rows 0..I-1 then up rows      */
  moe_weights_t w2;     /* routed down: [E][H][I]                                         */
  moe_weights_t sh13;   /* shared gate/up: [1][2*I_shared][H] (ignored if !has_shared)    */
  moe_weights_t sh2;    /* shared down: [1][H][I_shared]                                  */
  int32_t router_score;     /* moe_score_t                                               */
  int32_t bias_select_only; /* 1: router_bias enters the selection keys only; the weights
                               use the bare logits. 0: both                              */
} moe_layer_t;

/* Layout of the quantized-token buffer `xq` for T tokens (see moe_xq_bytes):
 *   MOE_A_NVFP4_4O6: codes [T][H/2] | scales E4M3 [T][H/16] | g FP32 [T]
 *   MOE_A_FP8_TOKEN: codes E4M3 [T][H] | s FP32 [T]
 *   MOE_A_MXFP4:     codes E2M1 [T][H/2] (element 2i in the low nibble) | scales E8M0 [T][H/32]
 *   MOE_A_MXFP8:     codes E4M3 [T][H] | scales E8M0 [T][H/32]
 * Each part starts at a 256-byte boundary from the start of xq. */

/* Optional per-call debug outputs and controls of moe_expert_forward (any pointer may
 * be NULL). Pair p = t*k + j is token t's j-th selected expert; rows T*k + t hold token
 * t's shared expert. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GROUPED = 2 } moe_path_t;
typedef struct {
  float *h;             /* FP32 [T*k + T*has_shared][max(I, I_shared)]: SwiGLU outputs   */
  uint8_t *hq_codes;    /* quantized routed h: NVFP4 / MXFP4 [T*k][I/2], FP8 / MXFP8
                           [T*k][I]                                                       */
  uint8_t *hq_scales;   /* NVFP4: E4M3 [T*k][I/16]; MX: E8M0 [T*k][I/32]                  */
  float *hq_scale;      /* NVFP4: g [T*k]; FP8 per token: s [T*k]; MX: unused             */
  int32_t path;         /* moe_path_t: which expert kernels run. AUTO picks the grouped
                           (MFMA, 32 tokens per unit) kernels from 8 tokens on with a BF16
                           shared expert, from 24 with BF16 or MXFP8 routed weights, and
                           from 32 with 4-bit weights when units hold many tokens (a
                           shared expert, or T*k >= E); else the GEMV kernels (4 tokens
                           per unit). GROUPED is refused where the shapes do not tile or
                           a workgroup would need more than 80 KB of LDS (the expert
                           tables grow with T*k and E); AUTO then runs the GEMV kernels  */
} moe_debug_t;

/* Host only; no device access. Checks every constraint the kernels rely on for a
 * layer run with up to max_tokens tokens (default-deny: anything not known to work
 * is refused) and writes every violated one, ';'-separated, into why (if non-NULL).
 * This follows the refuse-at-startup-with-every-reason rule of the Mistral Large 4
 * page's ROCm implementation details (specialized decode, default deny). */
moe_status_t moe_layer_check(const moe_layer_t *L, int32_t max_tokens, char *why,
                             size_t why_len);

/* Bytes of device workspace a layer needs for calls with up to max_tokens tokens;
 * 0 if moe_layer_check fails. */
size_t moe_workspace_bytes(const moe_layer_t *L, int32_t max_tokens);

/* Bytes of the xq buffer for T tokens (0 for MOE_A_BF16). */
size_t moe_xq_bytes(const moe_layer_t *L, int32_t T);

/* Enqueues a fill kernel that zeroes ws. Call once after allocating a workspace
 * (and after any call that returned an error mid-way). Every successful call leaves
 * the workspace's counters at zero again. One workspace must not be used by calls
 * that may overlap (different streams). */
moe_status_t moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Router ("Inkling 2 Small on vLLM: Day-0 Support", accuracy evaluation: the router
 * runs in FP32; "vLLM Day-0 support for Recursive's Flint", architecture: sigmoid top-6
 * routing over 256 experts; "Day 0 support for Mistral Large 4 on vLLM", ROCm
 * implementation details: softmax top-4 router; Inkling page, MoE with fused activation
 * quantization: tokens quantized to the expert layer's format in the producing kernel).
 * logits = x * router_w^T in FP32, keys = logits + bias; per token the k
 * largest keys, largest first, ties to the lower expert index; topk_w = the
 * router_score of the selected keys (or bare logits with bias_select_only),
 * renormalized to sum to 1 (FP32). With afmt != MOE_A_BF16 also quantizes every token
 * into xq (layout above) in the same launch.
 *   x_bf16   [T][H] BF16, device.      topk_ids [T][k] int32, device (output).
 *   topk_w   [T][k] FP32 (output).     xq: NULL for MOE_A_BF16, else moe_xq_bytes.
 *   0 <= T <= the max_tokens ws was sized for; T = 0 enqueues nothing. */
moe_status_t moe_route(const moe_layer_t *L, const uint16_t *x_bf16, int32_t T,
                       int32_t *topk_ids, float *topk_w, void *xq, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* Experts and combine ("vLLM Day-0 support for Recursive's Flint", optimization
 * strategy: small-batch MoE kernels that read only the selected experts' weights, with
 * routing and the expert combine fused into the neighbouring GEMVs; Inkling page, MoE
 * with fused activation quantization: the SwiGLU output is quantized before the down
 * projection; Flint and Mistral Large 4 architecture sections: one shared expert added
 * with weight 1). For every selected (token, expert) pair, and for the shared
 * expert, h = silu(Wg x) * (Wu x) (x quantized per afmt for routed experts; the
 * shared expert takes x_bf16), h re-quantized per afmt for routed experts, o = Wd h;
 * y[t] = sum_j topk_w[t][j] * o[t, j] + o_shared[t], FP32 accumulation, BF16 output
 * (round to nearest even). Reads only the experts named in topk_ids.
 *   x_bf16 [T][H]; xq as written by moe_route (ignored for MOE_A_BF16);
 *   topk_ids [T][k]: the k entries of a row must be distinct and in [0, E) (as
 *   moe_route writes them); for a row that breaks this, that token's y is unspecified
 *   (every access stays in bounds and the other tokens are unaffected).
 *   topk_w [T][k]; y_bf16 [T][H] (output).
 *   dbg: NULL or debug outputs. */
moe_status_t moe_expert_forward(const moe_layer_t *L, const uint16_t *x_bf16,
                                const void *xq, int32_t T, const int32_t *topk_ids,
                                const float *topk_w, uint16_t *y_bf16, void *ws,
                                size_t ws_bytes, const moe_debug_t *dbg,
                                hipStream_t stream);

/* The whole layer in one call: moe_route then moe_expert_forward, with the arguments,
 * layouts, results and checks of both (topk_ids / topk_w are outputs; xq is written
 * and read). Where the experts run the GEMV kernels in pair mode (T*k <= 64, not the
 * grouped kernels), the top-k runs inside the gate/up kernel's prologue, from the
 * router logits in ws, instead of in a launch of its own: the same selection and
 * weights as moe_route (the Flint page's low-latency decode path, routing fused into
 * the neighbouring kernels). Arguments are all validated before the first launch. */
moe_status_t moe_forward(const moe_layer_t *L, const uint16_t *x_bf16, int32_t T,
                         int32_t *topk_ids, float *topk_w, void *xq, uint16_t *y_bf16,
                         void *ws, size_t ws_bytes, const moe_debug_t *dbg,
                         hipStream_t stream);

/* RMSNorm of the residual stream before the layer (weight gamma, BF16 [H]; eps >= 0). */
typedef struct {
  const uint16_t *gamma;
  float eps;
} moe_norm_t;

/* The layer with its neighbouring steps of a pre-norm transformer block fused in ("Day 0
 * support for Mistral Large 4 on vLLM", fusions of the decode round: the residual add
 * and the RMSNorm run in one kernel with the all-reduce; "Inkling 2 Small on vLLM: Day-0
 * Support", kernel fusion: the memory-bound steps between sublayers are folded into
 * neighbouring kernels). With r = resid_in [T][H] (BF16):
 *   x_out     = RMSNorm(r) = r / sqrt(mean_h r^2 + eps) * gamma, in FP32 (the squares
 *               summed in a fixed order), rounded to BF16; the router launch computes it
 *   topk_ids, topk_w, xq, and y = the layer on x_out, exactly as moe_forward;
 *   resid_out = r + y, summed in FP32 and rounded once to BF16 (y is not rounded first);
 *               the kernel that writes y writes this instead.
 * No launch is added to moe_forward's. resid_out may be resid_in (updated in place);
 * x_out must not overlap resid_in. resid_in, x_out and gamma 16-byte aligned. Other
 * arguments, checks and errors as moe_forward. */
moe_status_t moe_forward_fused(const moe_layer_t *L, const moe_norm_t *norm, const uint16_t *resid_in,
                               int32_t T, uint16_t *x_out, int32_t *topk_ids, float *topk_w, void *xq,
                               uint16_t *resid_out, void *ws, size_t ws_bytes, const moe_debug_t *dbg,
                               hipStream_t stream);

/* moe_forward without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The same arguments, results and checks as moe_forward, minus ws and
 * ws_bytes: the workspace is a static array inside this library, one copy per GPU of
 * moe_noalloc_scratch_bytes() bytes (16 MiB), held until the process ends. Its device
 * address is looked up (hipGetSymbolAddress) on the first call on each device, so make
 * that first call outside graph capture. The call allocates nothing. A call whose
 * workspace would exceed the scratch (moe_workspace_bytes(L, T) > 16 MiB, e.g. the
 * Flint-shaped layer past about 200 tokens) fails with MOE_EWORKSPACE and enqueues
 * nothing. Every call on one GPU uses the same scratch and leaves the last call's
 * intermediates in it (nothing in it needs clearing: each call's kernels read only what
 * earlier kernels of the same call wrote), so calls that may overlap on one GPU (other
 * streams, other threads) race and must be serialized by the caller. */
moe_status_t moe_forward_noalloc(const moe_layer_t *L, const uint16_t *x_bf16, int32_t T,
                                 int32_t *topk_ids, float *topk_w, void *xq, uint16_t *y_bf16,
                                 const moe_debug_t *dbg, hipStream_t stream);
size_t moe_noalloc_scratch_bytes(void);

/* Four-Over-Six NVFP4 quantization of rows x[rows][cols] (BF16), cols % 16 == 0
 * ("Inkling 2 Small on vLLM: Day-0 Support", mixed-precision MoE and Four-Over-Six
 * NVFP4): per row g = amax/2688 (FP32); per 16-block with max m and c in {6, 4}:
 * S_c = E4M3((m/g)/c), codes E2M1(x/(S_c*g)); keep c = 4 only if its FP32 sum of
 * |x - decoded| (pairwise tree 8,4,2,1) is strictly lower. An all-zero row gives
 * g = 0, zero scales and sign-only codes. Outputs: codes [rows][cols/2] (element 2i
 * in the low nibble), scales [rows][cols/16], gscale [rows], choice [rows][cols/16]
 * in {4, 6} (NULL to skip). Bit-exact with the stated FP32 operation order. */
moe_status_t quantize_nvfp4_4o6(const uint16_t *x_bf16, int32_t rows, int32_t cols,
                                uint8_t *codes, uint8_t *scales, float *gscale,
                                uint8_t *choice, hipStream_t stream);

/* Load-time weight requantization to MXFP4 (MOE_W_MXFP4 layout), following the load
 * path of the Mistral Large 4 page's ROCm implementation details (each expert
 * dequantized to BF16, then requantized to E2M1 values with one E8M0 scale per 32).
 * Per 32-element block, the OCP MX v1.0 rule: shared exponent floor(log2(block amax))
 * - 2, clamped to [-127, 127], scale byte = exponent + 127; elements = value *
 * 2^-exponent (exact), rounded to E2M1 with ties to even, saturating at 6, sign kept
 * (so -0 gives code 8). An all-zero block takes scale byte 0.
 *   w_bf16 [rows][cols] BF16, device, 16-byte aligned; cols a positive multiple of 32.
 *   codes  [rows][cols/2] (element 2i in the low nibble), 16-byte aligned (output).
 *   scales [rows][cols/32] E8M0 bytes (output).
 *   rows = 0 enqueues nothing. Asynchronous on stream; caller-owned buffers. A stack
 *   of experts is one call with rows = experts * rows per expert. */
moe_status_t moe_requant_mxfp4(const uint16_t *w_bf16, int64_t rows, int32_t cols,
                               uint8_t *codes, uint8_t *scales, hipStream_t stream);

/* Load-time requantization of block-scaled FP8 weights to MXFP4 (MOE_W_MXFP4 layout): the
 * checkpoint the Mistral Large 4 page's loader reads (ROCm implementation details: block-FP8
 * expert weights with their block scales, each expert dequantized to BF16 and requantized
 * to MXFP4). Element (r, c) is E4M3(w_fp8[r][c]) times block_scales[r / block_rows]
 * [c / block_cols], one FP32 product rounded to nearest even, then rounded to BF16 (nearest
 * even); the BF16 rows then take the moe_requant_mxfp4 rule, bit for bit.
 *   w_fp8 [rows][cols] E4M3 bytes (OCP), device, 16-byte aligned; cols a positive
 *   multiple of 32; NaN codes (0x7F, 0xFF) and products beyond BF16's range are outside
 *   the contract (their blocks' outputs are unspecified).
 *   block_scales [ceil(rows / block_rows)][ceil(cols / block_cols)] FP32, device; the
 *   edge blocks may be ragged; block_rows, block_cols >= 1 (128 x 128 in common
 *   checkpoints; block_cols need not be a multiple of 32).
 *   codes [rows][cols/2] (element 2i in the low nibble), 16-byte aligned; scales
 *   [rows][cols/32] E8M0 bytes (outputs). rows = 0 enqueues nothing; at most 2^31
 *   32-blocks per call. A stack of experts is one call when the rows per expert are a
 *   multiple of block_rows (the scale grid then stacks the same way), else one call per
 *   expert. Asynchronous on stream; caller-owned buffers. */
moe_status_t moe_requant_fp8_block_mxfp4(const uint8_t *w_fp8, const float *block_scales,
                                         int64_t rows, int32_t cols, int32_t block_rows,
                                         int32_t block_cols, uint8_t *codes, uint8_t *scales,
                                         hipStream_t stream);

/* Load-time weight requantization to MXFP8 (MOE_W_MXFP8 layout), for MXFP8 expert layers
 * (Inkling page, mixed-precision MoE: MXFP8 expert layers): the same OCP MX v1.0 rule as
 * moe_requant_mxfp4 with E4M3 elements, i.e. shared exponent floor(log2(block amax)) - 8,
 * clamped to [-127, 127], elements E4M3 (nearest-even, saturating at 448, sign kept).
 *   w_bf16 [rows][cols] BF16, device, 16-byte aligned; cols a positive multiple of 32.
 *   codes  [rows][cols] E4M3 bytes, 16-byte aligned; scales [rows][cols/32] E8M0 bytes.
 *   rows = 0 enqueues nothing. */
moe_status_t moe_requant_mxfp8(const uint16_t *w_bf16, int64_t rows, int32_t cols,
                               uint8_t *codes, uint8_t *scales, hipStream_t stream);

/* Load-time weight requantization to NVFP4 (MOE_W_NVFP4 layout), the load path's other
 * target: ntensors tensors of [rows][cols], each with its own FP32 scale (gate, up and
 * down of every expert are separate tensors, so a w13 stack is 2E tensors of I rows in
 * gscale order [E][2], a w2 stack E tensors of H rows). Per tensor, in FP32: a = max
 * |x|; g = a / 2688; per 16-block with maximum m: S = E4M3((m / g) / 6) (nearest-even,
 * saturating at 448), elements E2M1(x / (S * g)) (nearest-even, saturating at 6); a
 * zero S * g or an all-zero tensor gives sign-only codes (and g = 0, scale bytes 0).
 *   w_bf16 [ntensors][rows][cols] BF16, device, 16-byte aligned; cols a positive
 *   multiple of 16. codes [ntensors][rows][cols/2] (element 2i in the low nibble),
 *   8-byte aligned; scales [ntensors][rows][cols/16] E4M3 bytes; gscale [ntensors]
 *   FP32 (outputs). 0 <= ntensors <= 65535; ntensors = 0 or rows = 0 enqueues nothing.
 *   Three launches in stream order (chunk maxima, kept in the code bytes until the last
 *   launch overwrites them; tensor scales; quantization). */
moe_status_t moe_requant_nvfp4(const uint16_t *w_bf16, int32_t ntensors, int64_t rows,
                               int32_t cols, uint8_t *codes, uint8_t *scales,
                               float *gscale, hipStream_t stream);

/* Diagnostics: per-kernel device time.
 * Between moe_profile_begin() and moe_profile_end(), every kernel the library launches
 * is bracketed by a start/stop event pair taken by the dispatch itself
 * (hipExtLaunchKernel), on the stream it runs on. moe_profile_end() waits for those
 * events, fills up to max_entries records (one per kernel kind that ran: route, topk,
 * gateup, hquant, down, combine, quantize_nvfp4, fill) with the launch count
 * and summed milliseconds, ends the session
 * and returns the number of records written. Meant for measurement runs; do not use
 * while capturing a stream into a graph. One process-wide session. */
typedef struct {
  const char *name;
  int32_t launches;
  double total_ms;
} moe_kernel_time_t;
moe_status_t moe_profile_begin(void);
int32_t moe_profile_end(moe_kernel_time_t *out, int32_t max_entries);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *moe_last_error(void);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
