/*
 * moe_mi355x.h -- C ABI of the routed mixture-of-experts expert-FFN hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * Pages cited by title and section:
 *   [GATE-PR]  "Enable and fuse the Inkling MoE gate epilogue on Intel XPU"
 *              (sglang PR #36385)
 *   [CLAMP-PR] "[Moe] Fix flashinfer_trtllm silently dropping swiglu_limit
 *              clamped SwiGLU activation" (sglang PR #39920)
 *   [OAI-PR]   "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE"
 *              (DeepGEMM PR #445)
 *   [INT4-PR]  "sm100: Fused INT4 grouped + SiLU Triton kernel"
 *              (batchgen PR #239)
 *   [LORA-AOT] "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT -- SwiGLU LoRA
 *              up-delta units, EP scale lookups" (release notes); it serves
 *              NVFP4 expert weights with distinct gate/up global scales
 *
 * Conventions for every entry point:
 *   - Every array argument is DEVICE memory owned by the caller (plain
 *     pointers; the descriptors moe_weights / moe_lora / moe_layer /
 *     moe_act_params themselves are HOST structs read during the call).
 *     The library keeps no pointer after a call returns, allocates no device
 *     or host memory, and never synchronises except in
 *     moe_read_device_error. `stream` is a hipStream_t (NULL = default).
 *   - Work is enqueued asynchronously on `stream`; outputs are valid once the
 *     stream reaches that point.
 *   - Host-detectable problems return a negative moe_status and enqueue
 *     nothing. Launch failures return MOE_ERR_HIP (moe_last_error() has the
 *     HIP message). Data-dependent problems found on the device (a routing
 *     id outside [0, num_experts_global)) OR a MOE_DEVERR_* bit into a
 *     caller-owned int32 `err_word` (the caller zeroes it), skip the bad
 *     pair and leave every valid pair unaffected.
 *   - Row-major layouts; a "[G][N][K]" weight is G matrices of N output rows
 *     by K input columns.
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or not a multiple */
  MOE_ERR_FORMAT = -3,      /* unknown weight format or format mismatch */
  MOE_ERR_LOCAL_RANGE = -4, /* missing/invalid local expert range */
  MOE_ERR_PARAM = -5,       /* non-finite or out-of-range scalar parameter */
  MOE_ERR_WORKSPACE = -6,   /* workspace NULL or too small */
  MOE_ERR_HIP = -8,         /* a HIP launch or runtime call failed */
  MOE_ERR_SCRATCH = -9      /* the call needs more than the static scratch of
                               moe_forward_no_workspace holds */
} moe_status;

typedef enum {
  MOE_W_BF16 = 0,      /* bf16 [G][N][K]; scale NULL */
  MOE_W_FP8_B128 = 1,  /* OCP e4m3fn [G][N][K]; scale fp32 [G][N/128][K/128]
                          (w = q * scale, 128x128 blocks) [CLAMP-PR
                          "Modifications": blockwise 128x128 FP8] */
  MOE_W_INT4_G32 = 2,  /* u8 [G][N][K/2] (byte j of a row: low nibble k=2j,
                          high nibble k=2j+1); scale bf16 [G][N][K/32];
                          w = (nibble - 8) * scale [INT4-PR commit text] */
  MOE_W_NVFP4 = 3,     /* e2m1 codes packed like INT4, u8 [G][N][K/2];
                          scale e4m3fn u8 [G][N][K/16]; w = e2m1(code) *
                          e4m3(scale) * gscale [LORA-AOT "Changes since
                          1b699bf": per-half NVFP4 global scales]. e2m1:
                          sign bit 3, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
                          NaN scale codes (0x7F, 0xFF) set
                          MOE_DEVERR_W4_SCALE. */
  MOE_W_MXFP4 = 4,     /* e2m1 codes as NVFP4; scale e8m0 u8 [G][N][K/32];
                          w = e2m1(code) * 2^(scale - 127). Exact for scale
                          exponents 104..128 (2^-23 .. 2); a call that meets
                          another exponent sets MOE_DEVERR_W4_SCALE (its
                          outputs are then not valid). */
  MOE_W_MXFP4_A8 = 5   /* W4A8: the weights exactly as MOE_W_MXFP4, but the
                          activations enter GEMM1 as MXFP8 (see
                          moe_quantize_act_mxfp8) and GEMM1 runs on the
                          block-scaled matrix instructions, which take the
                          whole e8m0 range (code 0xFF, NaN, sets
                          MOE_DEVERR_W4_SCALE). Its 128-deep sums are
                          accurate to about 2e-5 of their sum of |products|
                          (not fp32-accurate); h is bf16 and GEMM2 is the
                          MOE_W_MXFP4 one. A choice of this library: the
                          pages fix no activation format for 4-bit weights. */
} moe_wfmt;

/* err_word bits */
#define MOE_DEVERR_GLOBAL_ID_OOB 0x1 /* a routing id < 0 or >= num_experts_global */
#define MOE_DEVERR_F16_RANGE 0x2     /* 4-bit layer: a bf16 activation x or h with
                                        |v| > 65504 (or not finite), beyond the f16
                                        operands of its matrix cores; the outputs
                                        of that call are not valid */
#define MOE_DEVERR_W4_SCALE 0x4      /* 4-bit layer: a weight scale outside the
                                        range the kernels expand exactly: INT4 a
                                        nonzero |scale| outside [2^-13, 2^13),
                                        NVFP4 a NaN e4m3 code, MXFP4 an exponent
                                        outside 104..128; outputs not valid */

/* Parameterized SwiGLU [CLAMP-PR "Modifications"; OAI-PR "Summary",
 * "Compatibility"]:
 *   g' = min(g, limit), u' = clamp(u, -limit, limit),
 *   h  = g' * sigmoid(alpha * g') * (u' + beta).
 * Defaults alpha = 1, beta = 0, limit = +INFINITY (no clamp) give
 * silu(g) * u. alpha and beta must be finite, limit > 0 (may be +inf). */
typedef struct {
  float alpha, beta, limit;
} moe_act_params;

/* One stacked expert weight (W13 = fused [gate | up], or W2 = down). */
typedef struct {
  int fmt;              /* moe_wfmt */
  int n_groups;         /* G: stacked matrices (local experts [+ shared]) */
  int N, K;             /* each matrix is [N][K]: W13 N = 2I, K = H;
                           W2 N = H, K = I */
  const void *q;        /* codes, layout per moe_wfmt */
  const void *scale;    /* scales, layout per moe_wfmt (NULL for BF16) */
  const float *gscale;  /* nullable. W13: fp32 [G][2] = (gate, up)
                           per-expert global scales multiplying the dequantised
                           gate rows 0..I-1 and up rows I..2I-1; the "true
                           units" of [LORA-AOT "Changes since 1b699bf"].
                           W2: NVFP4 / MXFP4 only (else MOE_ERR_FORMAT),
                           fp32 [G], one per expert. */
} moe_weights;
/* Alignment (MOE_ERR_PARAM): 4-bit codes 16 bytes; INT4 and NVFP4 scales
 * 2 bytes. Activations of 4-bit layers enter the matrix cores as f16:
 * exact for |x| in [2^-14, 65504] (and h alike); larger magnitudes set
 * MOE_DEVERR_F16_RANGE, smaller ones lose low bits (an absolute error below
 * 2^-25 per element). */

/* Rank-r LoRA of the local experts [LORA-AOT "Changes since 1b699bf"].
 * On the fused gate/up projection ("lora"): z = x A_e^T (fp32),
 * delta = scale * z B_e^T, added to g and u after each half's own global
 * scale, before the clamp.  A: bf16 [n_groups][rank][H], B: bf16
 * [n_groups][2I][rank].
 * On the down projection ("lora_down"): its input is activation_lora_input,
 * the SwiGLU output h in those true units rounded to bf16 (before any FP8
 * re-quantisation); z2 = h A2_e^T (fp32), y += scale * z2 B2_e^T, added to
 * the expert's output row before the routing-weighted combine.  A2: bf16
 * [n_groups][rank][I], B2: bf16 [n_groups][H][rank].
 * The shared expert (group E_loc) carries no LoRA.
 * A batch of adapters (n_adapters > 1; the page's harness serves eight
 * rank-16 adapters at once): A and B gain a leading adapter dimension,
 * [n_adapters][n_groups][...], and adapter_ids (device int32 [T], per call)
 * gives each token's adapter; a token whose id is outside [0, n_adapters)
 * gets no delta. n_adapters 0 or 1: one adapter for every token,
 * adapter_ids unused. A and B must be 16-byte aligned (MOE_ERR_PARAM). */
typedef struct {
  int rank;             /* 1..32 */
  int n_groups;         /* adapters for groups 0..n_groups-1 (the local
                           routed experts); later groups have none */
  float scale;
  const void *A;
  const void *B;
  int n_adapters;       /* 0..1024 */
  const int *adapter_ids;
} moe_lora;

/* ---------------------------------------------------------------- route -- */
/* Sigmoid-gate top-k with log-sigmoid renormalisation and shared-sink
 * columns [GATE-PR "2. Correctness", "3. Performance", router-epilogue
 * commit message]. Per token row t of `logits` (fp32, row stride `ld`
 * elements, ld >= n_routed + n_sink):
 *   - top_k passes of masked argmax over the n_routed leading columns,
 *     ranked on the raw logit when sel_bias is NULL (sigmoid is monotone),
 *     else on the fp32 key sigmoid(x) + sel_bias[c] (sel_bias fp32
 *     [n_routed]; the sink columns take no bias and never rank); equal keys
 *     resolve to the lower column index;
 *   - the winners carry their RAW logits: lp = logsigmoid of the k winners'
 *     raw logits and of the n_sink trailing sink columns; w = exp(lp -
 *     logsumexp(lp)) * route_scale * global_scale (finite when every logit
 *     is far below -104).
 * Outputs: topk_ids int32 [T][top_k] (global column ids, selection order),
 * topk_w fp32 [T][top_k], sink_w fp32 [T][n_sink] (NULL iff n_sink == 0),
 * packed int32 [T][top_k] or NULL: (id << 16) | bf16 bits of topk_w
 * (round to nearest even); a consumer takes the id as p >> 16 and the
 * weight from p & 0xFFFF.
 * Limits: 1 <= top_k <= n_routed, top_k + n_sink <= 64,
 * n_routed + n_sink <= 1024, T >= 0. Logits are assumed finite. */
int moe_route(const float *logits, long T, long ld, int n_routed, int n_sink,
              int top_k, const float *sel_bias, float route_scale,
              float global_scale, int *topk_ids, float *topk_w, float *sink_w,
              int *packed, void *stream);

/* ----------------------------------------------------------- gate route -- */
/* The router GEMM fused with the epilogue of moe_route [GATE-PR: the
 * "258-column gate GEMM" whose fp32 [T, N + S] rows feed the epilogue;
 * router-epilogue commit message]. logits[t][c] = sum_h x[t][h] * wg[c][h]
 * for c < n_routed + n_sink, bf16 operands, fp32 accumulation (in an order
 * of the kernel's choosing), then exactly the moe_route epilogue on those
 * rows (selection bias, raw-logit carry, sinks, scales, packed output).
 *   x_bf16   bf16 [T][H], row-major, 16-byte aligned;
 *   wg_bf16  bf16 [n_routed + n_sink][H] (routed rows first, then the sink
 *            rows), 16-byte aligned;
 *   logits   fp32 [T][n_routed + n_sink] or NULL (the gate rows, if the
 *            caller wants them);
 *   topk_ids, topk_w, sink_w, packed, sel_bias as for moe_route;
 *   ws       device workspace of moe_gate_route_workspace_size(T, H,
 *            n_routed, n_sink) bytes (0 when T is large enough for the
 *            single fused launch; NULL allowed then).
 * Limits: H a multiple of 32, 1 <= top_k <= n_routed, top_k + n_sink <= 16,
 * n_routed + n_sink <= 512, T >= 0 (T = 0 is a no-op). Errors: SHAPE for
 * the limits, NULL for a missing required pointer, PARAM for non-finite
 * scales or misaligned x / wg, WORKSPACE for a missing or short ws. */
size_t moe_gate_route_workspace_size(long T, int H, int n_routed, int n_sink);
int moe_gate_route(const void *x_bf16, const void *wg_bf16, long T, int H,
                   int n_routed, int n_sink, int top_k, const float *sel_bias,
                   float route_scale, float global_scale, float *logits,
                   int *topk_ids, float *topk_w, float *sink_w, int *packed,
                   void *ws, size_t ws_bytes, void *stream);

/* -------------------------------------------------------------- permute -- */
/* Expert-parallel rebase and grouping of (token, slot) pairs by local expert
 * [LORA-AOT "Changes since 1b699bf": ids are global, per-expert tables are
 * rank-local, rebase by local_expert_offset and bounds-check against the
 * local count; INT4-PR: per-expert sorted-token dispatch].
 *   pair id p = t*top_k + j; e = topk_ids[p] - local_expert_offset; the pair
 *   is local iff 0 <= e < num_local_experts. With shared_expert = 1 an
 *   always-on group G-1 = num_local_experts holds pairs p = T*top_k + t.
 *   Groups are laid out in order, pairs inside a group by ascending p.
 * Outputs: offsets int32 [G+1] (group g owns sorted rows
 * offsets[g]..offsets[g+1]-1), sorted_pair int32 [P_cap] (pair id of each
 * sorted row), pair_row int32 [T*top_k + shared*T] (sorted row of each pair
 * or -1), with P_cap = T*top_k + shared*T and G = num_local_experts +
 * shared_expert. Ids outside [0, num_experts_global) set
 * MOE_DEVERR_GLOBAL_ID_OOB in *err_word and are skipped.
 * Errors: MOE_ERR_LOCAL_RANGE unless num_local_experts >= 1,
 * local_expert_offset >= 0 and offset + num_local_experts <=
 * num_experts_global; MOE_ERR_SHAPE if G > 1024 or T*top_k >= 2^30.
 * Workspace: moe_permute_workspace_size(T, top_k, G) bytes. */
int moe_permute(const int *topk_ids, long T, int top_k, int num_experts_global,
                int local_expert_offset, int num_local_experts,
                int shared_expert, int *offsets, int *sorted_pair,
                int *pair_row, int *err_word, void *ws, size_t ws_bytes,
                void *stream);
size_t moe_permute_workspace_size(long T, int top_k, int n_groups);

/* -------------------------------------------------- activation quantise -- */
/* Per token and per 128-column group: amax in fp32, s = amax / 448 (s = 1
 * when amax == 0), q = e4m3fn(round-to-nearest-even(x / s)) saturated to
 * +-448 [CLAMP-PR "Modifications": the activation side of blockwise FP8].
 * x bf16 [T][H] -> xq e4m3fn [T][H], xs fp32 [T][H/128]. H % 128 == 0. */
int moe_quantize_act_fp8(const void *x_bf16, long T, int H, void *xq,
                         float *xs, void *stream);

/* MXFP8 activations, the GEMM1 input of MOE_W_MXFP4_A8 layers: per token and
 * per 32 columns, amax in fp32, e = the smallest integer with
 * amax <= 448 * 2^e (raised to -127 when smaller, e.g. an all-zero group),
 * xe = e + 127 (e8m0), xq = e4m3fn(round-to-nearest-even(x / 2^e)) (never
 * beyond 448, so never saturated). x bf16 [T][H] -> xq e4m3fn [T][H] +
 * xe u8 [T][H/32]. H % 128 == 0. */
int moe_quantize_act_mxfp8(const void *x_bf16, long T, int H, void *xq,
                           void *xe, void *stream);

/* ------------------------------------------------ grouped GEMM1 + SwiGLU -- */
/* err_word of the GEMM entry points: device int32, ORed with the
 * MOE_DEVERR_F16_RANGE / MOE_DEVERR_W4_SCALE bits a 4-bit layer meets
 * (required for 4-bit weights: MOE_ERR_NULL without it; nullable, and
 * never written, for BF16 and FP8 weights). */
/* For each group g and each of its sorted rows r (token t of pair
 * sorted_pair[r]):  [g | u] = x_t W13_g^T  (fp32 accumulation;
 * FP8: per 128-K block partial sums times xs[t][kb] * scale[g][nb][kb]),
 * times gscale[g] (gate, up) when given, plus the LoRA delta when given,
 * then the parameterized SwiGLU `act` -> h[r][0..I-1].
 *   FP8 weights: x = xq e4m3fn [T][H] with xs fp32 [T][H/128]; h is
 *     re-quantised like moe_quantize_act_fp8 per row and 128 columns:
 *     h e4m3fn [P_cap][I], hs fp32 [P_cap][I/128].
 *   MXFP4_A8 weights: x = xq e4m3fn [T][H] with xs = xe u8 [T][H/32]
 *     (moe_quantize_act_mxfp8); h bf16 as below, hs NULL.
 *   BF16 / other 4-bit (INT4, NVFP4, MXFP4) weights: x bf16 [T][H] (xs NULL);
 *     h bf16 [P_cap][I] (round-to-nearest-even), hs NULL.
 * x_bf16 bf16 [T][H] is the LoRA input (NULL without LoRA).
 * h_lora (FP8 weights only, else it must be NULL: MOE_ERR_PARAM), nullable:
 * bf16 [P_cap][I], the SwiGLU output before the re-quantisation (round to
 * nearest even), i.e. the down-LoRA input; BF16 / 4-bit layers pass h itself
 * to moe_grouped_gemm2_combine instead.
 * offsets / sorted_pair come from moe_permute for the same (T, top_k);
 * w13->n_groups = G, w13->N = 2I, w13->K = H. p_cap = rows allocated in h.
 * Limits: H % 128 == 0 and I % 128 == 0. Workspace:
 * moe_gemm1_workspace_size(w13, p_cap, lora) bytes: the LoRA z rows; for
 * FP8 / 4-bit weights at decode sizes (few enough tiles of 32 rows x 128 h
 * columns that one tile per workgroup would leave CUs idle) the fp32
 * partial sums of a split-K schedule (4 * p_cap * 2I floats), which spreads
 * the K blocks of those tiles over all CUs and reduces them in a fixed
 * order; for 4-bit weights other than MXFP4_A8 the f16 copy of the
 * activations (p_cap * H * 2 bytes, T <= p_cap). Returns 0 for a NULL w13 or N not a multiple of 256. */
int moe_grouped_gemm1_act(const moe_weights *w13, const void *x,
                          const void *xs, const void *x_bf16, long T, int H,
                          int I, int top_k, long p_cap, const int *offsets,
                          const int *sorted_pair, const moe_act_params *act,
                          const moe_lora *lora, void *h, float *hs,
                          void *h_lora, int *err_word, void *ws,
                          size_t ws_bytes, void *stream);
size_t moe_gemm1_workspace_size(const moe_weights *w13, long p_cap,
                                const moe_lora *lora);

/* ---------------------------------------- grouped GEMM2 + weighted combine -- */
/* y[r] = h[r] W2_g^T (fp32; FP8 per 128-K block partial sums times
 * hs[r][kb] * scale[g][nb][kb]; FP4 times w2->gscale[g] when given) for
 * every sorted row, plus with lora_down
 * the down-LoRA delta scale * (h_lora[r] A2_g^T) B2_g^T for groups
 * g < lora_down->n_groups (h_lora bf16 [P_cap][I]: GEMM1's h_lora output
 * for FP8 weights, h itself for BF16 / 4-bit weights). For FP8 and 4-bit
 * weights the rows y pass to the combine in block floating point: one
 * power-of-two scale per row and 16 columns and an int16 multiple of it per
 * value, rounded to nearest (error at most 2^-15 of the run's largest
 * magnitude; a value that is not finite becomes NaN); BF16 layers keep
 * fp32 rows. Then
 *   out[t][:] = sum_{j < top_k, pair_row[t*top_k+j] >= 0} topk_w[t][j] *
 *               y[pair_row[t*top_k+j]]   (ascending j, fp32)
 *             + shared_w * y[pair_row[T*top_k + t]]   (if shared_expert)
 * [INT4-PR: slot-specific routing-weight reduction, fp32 accumulation].
 * Every out element is written (0 for a token with no local pair).
 * w2->N = H, w2->K = I. out fp32 [T][H]. Limits: 1 <= top_k <= 64
 * (MOE_ERR_SHAPE). err_word as for moe_grouped_gemm1_act. Workspace:
 * moe_gemm2_workspace_size(w2, p_cap, lora_down) bytes: the y rows (and
 * their scale exponents), or
 * for FP8 / 4-bit weights at decode sizes their split-K partial sums
 * (4 * p_cap * H floats, reduced by the combine in a fixed order; the
 * down-LoRA delta enters the first partial of each tile), then the
 * down-LoRA z2 rows (p_cap * rank floats, plus p_cap ints with a batch of
 * adapters). sorted_pair (moe_permute's) is needed with lora_down only (it
 * maps rows to tokens for the adapter ids). Errors: NULL for a lora_down
 * without h_lora or sorted_pair. Returns 0 for a NULL w2. */
int moe_grouped_gemm2_combine(const moe_weights *w2, const void *h,
                              const float *hs, const void *h_lora,
                              const moe_lora *lora_down, long T, int H, int I,
                              int top_k, int shared_expert, long p_cap,
                              const int *offsets, const int *sorted_pair,
                              const int *pair_row, const float *topk_w,
                              float shared_w, float *out, int *err_word,
                              void *ws, size_t ws_bytes, void *stream);
size_t moe_gemm2_workspace_size(const moe_weights *w2, long p_cap,
                                const moe_lora *lora_down);

/* ---------------------------------------------------------- whole layer -- */
typedef struct {
  int H, I;
  int num_experts_global;   /* routed experts E (logit columns 0..E-1) */
  int num_local_experts;    /* experts held here, global ids
                               [offset, offset + num_local_experts) */
  int local_expert_offset;
  int shared_expert;        /* 0 | 1: always-on group num_local_experts */
  int top_k, n_sink;        /* n_sink trailing sink logit columns */
  float route_scale, global_scale, shared_w;
  moe_weights w13, w2;      /* n_groups = num_local_experts + shared_expert */
  moe_act_params act;
  const moe_lora *lora;     /* nullable: LoRA on [gate | up] */
  const moe_lora *lora_down;/* nullable: LoRA on the down projection, input
                               the true-units SwiGLU output (see moe_lora) */
} moe_layer;

/* One call of the whole path on `stream`: moe_route -> moe_permute ->
 * (FP8) moe_quantize_act_fp8 | (MXFP4_A8) moe_quantize_act_mxfp8 ->
 * moe_grouped_gemm1_act ->
 * moe_grouped_gemm2_combine. x_bf16 bf16 [T][H]; logits fp32 [T][ld_logits]
 * with ld_logits >= num_experts_global + n_sink. Outputs out fp32 [T][H],
 * topk_ids/topk_w [T][top_k], sink_w [T][n_sink] (NULL iff n_sink == 0),
 * err_word as in moe_permute and the GEMM entry points. Workspace: moe_workspace_size(layer, T_max)
 * bytes, T <= T_max. Errors: those of the steps, checked before any launch. */
int moe_forward(const moe_layer *layer, const void *x_bf16,
                const float *logits, long T, long ld_logits, float *out,
                int *topk_ids, float *topk_w, float *sink_w, int *err_word,
                void *ws, size_t ws_bytes, void *stream);
size_t moe_workspace_size(const moe_layer *layer, long T_max);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and the same kernels, with the workspace taken from
 * a static device array of MOE_SCRATCH_BYTES that the library holds on
 * every GPU it runs on, from module load until the process ends. Arguments
 * as for moe_forward without ws / ws_bytes; the caller still passes (and
 * owns) every input and output. The device is the current one; its
 * array's address is looked up on the first call there. A layer and T whose
 * moe_workspace_size exceeds MOE_SCRATCH_BYTES return MOE_ERR_SCRATCH
 * (moe_scratch_error() says how much was needed) and launch nothing; 32 MiB
 * holds every layer here at T <= 64. Calls on one GPU share its array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * ordered by the caller. Nothing in the array has to start at zero (each
 * call writes every workspace byte before reading it). */
#define MOE_SCRATCH_BYTES (32u << 20)
int moe_forward_no_workspace(const moe_layer *layer, const void *x_bf16,
                             const float *logits, long T, long ld_logits,
                             float *out, int *topk_ids, float *topk_w,
                             float *sink_w, int *err_word, void *stream);
/* Message of the calling thread's last moe_forward_no_workspace refusal
 * ("" if none). */
const char *moe_scratch_error(void);

/* --------------------------------------------------------------- misc -- */
/* Synchronises `stream`, then copies *err_word (device) to *host_bits. */
int moe_read_device_error(const int *err_word, int *host_bits, void *stream);
const char *moe_status_string(int status);
/* Last HIP error message of the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
