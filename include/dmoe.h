/*
 * libdmoe: the hot path of one dots3-note preview mixture-of-experts layer on
 * an AMD Instinct MI355X (gfx950).
 *
 * The layer (model card "dots-studio/dots3-note-prev", Model Overview table;
 * Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig parameters): 256 routed
 * experts plus 1 shared expert, top-8 token-choice routing with renormalised
 * weights, hidden size 5120, per-expert SwiGLU FFN of width 1536, in BF16 or in
 * fine-grained FP8 (E4M3 weights with one FP32 scale per 128x128 block and
 * dynamically quantised 1x128 activations, including weight dimensions that
 * are not multiples of 128: Transformers PR #47844, implementation and
 * validation lists).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All data pointers are DEVICE pointers unless stated otherwise; the caller
 *   owns every buffer (including workspaces). The library never allocates,
 *   frees or synchronises; it enqueues kernels on `stream` and returns.
 * - Matrices are row-major with an explicit pitch ("ld", in elements).
 *   BF16 values are passed as their 16-bit patterns (uint16_t).
 * - Arguments are validated on the host before anything is enqueued; an
 *   invalid call returns a non-zero status, enqueues nothing and writes
 *   nothing. dmoe_last_error() then describes the problem (per thread).
 * - Launch failures are reported as DMOE_ERR_HIP. Faults inside kernels
 *   surface at the caller's next synchronisation, as with any HIP call.
 * - Device buffers must be 16-byte aligned and pitches multiples of 8
 *   elements (16 for FP8 codes) unless stated otherwise.
 * - Outputs must not alias inputs. Calls on different streams may run
 *   concurrently when their buffers are disjoint. Results are bitwise
 *   reproducible run to run.
 * - No entry point reads device memory from the host, so every call can be
 *   captured into a HIP graph. Grids are sized from host-known bounds and
 *   kernels read the actual counts on the device.
 * - The grouped GEMMs address each operand as a base pointer plus a 32-bit
 *   byte offset: the activation rows a call can read, one expert's weight
 *   block and the activation scales must each span at most 4 GiB. Entry
 *   points return DMOE_ERR_UNSUPPORTED when the sizes they are given break
 *   this; for a gathered operand (row_token) the caller keeps the rows it
 *   names within the first 4 GiB of `a`.
 *
 * Weight layout (produced once, before timing, by the preparation calls)
 * ------------------------------------------------------------------
 * Expert e's gate and up weights are [F_pad, ldw] blocks at
 * w + e * F_pad * ldw, F_pad = round_up(F, 128); down weights are [H, ldw]
 * blocks at w + e * H * ldw with ldw >= round_up(F, 128). Rows F..F_pad-1 and
 * columns past the valid width are zero (codes 0x00 or BF16 +0). FP8 block
 * scales are dense [E_loc][ceil(rows/128)][ceil(cols/128)] FP32 arrays over the
 * valid (unpadded) rows and columns. The hidden size H must be a multiple of
 * 128 (5120 on the pages).
 */
#ifndef DMOE_H
#define DMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef int32_t dmoe_status;
#define DMOE_OK 0
#define DMOE_ERR_INVALID_ARG 1 /* bad size, null pointer, out-of-range index */
#define DMOE_ERR_ALIGNMENT 2   /* pointer or pitch not aligned as required */
#define DMOE_ERR_UNSUPPORTED 3 /* valid request this build does not implement */
#define DMOE_ERR_WORKSPACE 4   /* workspace null or smaller than required */
#define DMOE_ERR_HIP 5         /* a HIP launch or runtime call failed */

#define DMOE_BF16 1
#define DMOE_FP8_E4M3 2

#define DMOE_ABI_VERSION 2

/* Router scoring functions (dmoe_layer_desc.scoring). */
#define DMOE_SCORING_SOFTMAX 0
#define DMOE_SCORING_SIGMOID 1

/* Text of the last error on this thread ("" if none). Host pointer, valid
 * until the next call on the same thread. */
const char* dmoe_last_error(void);

/* DMOE_ABI_VERSION of the built library. */
int32_t dmoe_abi_version(void);

/*
 * Router logits, FP32: logits[t, e] = sum_h f32(x[t, h]) * w_r[e, h].
 * x: [T, ldx] BF16; w_r: [E, H] FP32 dense; logits: [T, E] FP32 dense.
 * The sum is accumulated in FP32 on matrix cores (each product exact); its
 * order differs from a sequential sum, so results agree with an exact sum to
 * FP32 accumulation error, not bit for bit.
 * Requires 1 <= E <= 1024, H % 128 == 0, T >= 0 (T == 0 is a no-op).
 * Source: Transformers documentation "Dots 3 Note Preview", model outputs,
 * router_logits entry (shape (batch*seq, num_experts)); Transformers PR #47844 "Add dots3-note Preview model support",
 * implementation list (routing in FP32).
 */
dmoe_status dmoe_router_logits(const uint16_t* x, int64_t ldx, const float* w_r, int32_t T, int32_t H,
                               int32_t E, float* logits, hipStream_t stream);

/*
 * Top-K routing (Dots3NoteTextConfig: num_experts_per_tok, norm_topk_prob,
 * routed_scaling_factor = 1, n_group = topk_group = 1).
 * For each token: the K largest logits, equal values going to the lower expert
 * index, -0.0 treated as +0.0; slot k holds the expert of rank k.
 * topk_w[t, k] = exp(l_k - l_max) / sum_{j in top-K} exp(l_j - l_max), i.e. the
 * softmax over all E experts renormalised over the selected K, rounded to FP32.
 * logits: [T, E] FP32 (finite values; NaN behaviour is undefined);
 * topk_ids: [T, K] int32; topk_w: [T, K] FP32.
 * Requires 1 <= K <= E <= 1024, K <= 64.
 * Source: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
 * num_experts_per_tok, norm_topk_prob, routed_scaling_factor, n_group,
 * topk_group. The scoring function and the tie rule are not stated there:
 * softmax (the conditional-generation forward calls its router output
 * post-softmax) and lower index first are this library's readings.
 */
dmoe_status dmoe_route(const float* logits, int32_t T, int32_t E, int32_t K, int32_t* topk_ids, float* topk_w,
                       hipStream_t stream);

/*
 * Top-K routing with the other Dots3NoteTextConfig routing knobs (n_group,
 * topk_group, norm_topk_prob, routed_scaling_factor):
 * - n_group > 1: the E experts form n_group groups of E / n_group consecutive
 *   experts; a group's score is its largest logit; the topk_group groups with
 *   the largest scores are kept (equal scores: the lower group) and the K
 *   experts are the top-K (same tie rule) of the kept groups' experts. The
 *   docs fix only that the selected experts lie within topk_group groups; the
 *   group's best expert as its score is this library's reading.
 * - renormalize != 0: weights as dmoe_route; 0: the softmax over all E experts
 *   of each selected expert, not renormalised.
 * - weights are multiplied by routed_scaling_factor before the FP32 rounding.
 * n_group 0 or 1: ungrouped; topk_group 0: every group. Requires n_group <= 64,
 * E % n_group == 0, 1 <= topk_group <= n_group, K <= topk_group * E / n_group,
 * and a positive finite routed_scaling_factor; otherwise as dmoe_route.
 * dmoe_route(...) is dmoe_route_grouped(..., 1, 1, 1, 1.0f, ...).
 * Source: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
 * n_group, topk_group, norm_topk_prob, routed_scaling_factor.
 */
dmoe_status dmoe_route_grouped(const float* logits, int32_t T, int32_t E, int32_t K, int32_t n_group,
                               int32_t topk_group, int32_t renormalize, float routed_scaling_factor,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Sigmoid scoring with a selection-only correction bias: the bias-balanced
 * router the Transformers documentation ("Dots 3 Note Preview", model outputs, aux_loss entry)
 * name for DeepSeek-V3 and derived models.
 *   s[e] = f32(1 / (1 + exp(-l[e])))  (evaluated in double, rounded once)
 *   b[e] = f32(s[e] + score_bias[e])  (score_bias may be NULL: no bias)
 * Selection as dmoe_route_grouped on b, except that a group's score is
 * f32(b1 + b2), its two largest b (b1 alone for one-expert groups). Weights
 * are the unbiased s of the selected experts, divided by their sum when
 * renormalize != 0, times routed_scaling_factor, rounded to FP32.
 * score_bias: [E] FP32 device array. Same requirements as dmoe_route_grouped.
 * Source: Transformers documentation "Dots 3 Note Preview", model outputs, aux_loss
 * entry (routers that balance their experts with a bias).
 */
dmoe_status dmoe_route_sigmoid(const float* logits, const float* score_bias, int32_t T, int32_t E, int32_t K,
                               int32_t n_group, int32_t topk_group, int32_t renormalize, float routed_scaling_factor,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Expert-contiguous permutation of the (token, slot) pairs routed to this
 * GPU's experts [e0, e0 + E_loc): a stable counting sort over the flat pair
 * index t*K + k, so rows are ordered by (local expert, token).
 * Outputs: offsets [E_loc + 1] (offsets[E_loc] = M, the number of local
 * pairs); row_token [T*K] and row_slot [T*K] (entries [0, M) written);
 * token_row [T*K] (row of pair (t, k), or -1 if its expert is not local).
 * Expert ids outside [e0, e0 + E_loc) are simply not local.
 * ws: device workspace of at least dmoe_permute_ws_bytes(T, K, E_loc) bytes.
 * Source: the pages do not describe how the MoE runner lays out its rows
 * (SGLang cookbook "Dots3-Note", Configuration Tips, MoE runner paragraph,
 * names grouped expert GEMMs only). Reading: a stable counting sort by local
 * expert, which makes every table unique and is all a grouped GEMM needs.
 */
size_t dmoe_permute_ws_bytes(int32_t T, int32_t K, int32_t E_loc);
dmoe_status dmoe_permute(const int32_t* topk_ids, int32_t T, int32_t K, int32_t e0, int32_t E_loc,
                         int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* token_row, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * Dynamic 1x128 activation quantisation to E4M3 (PR #47844: dynamic
 * activations; partial blocks per its validation list).
 * For row r and column slice j = [128j, min(128j + 128, cols)):
 *   amax = max |x|, s = f32(amax / 448) (correctly rounded),
 *   q = E4M3 round-to-nearest-even of f32(x / s), saturated to +-448,
 *   sign bit of x / s kept; if s == 0 every code of the slice is 0x00.
 * x: [rows, ldx] BF16; q: [rows, ldq] uint8 codes (columns [cols, round_up(cols,
 * 128)) are written as 0x00 and must fit in ldq); scales: [rows, lds] FP32
 * with ceil(cols/128) valid entries per row. Requires cols % 8 == 0.
 * Source: Transformers PR #47844 "Add dots3-note Preview model support", implementation list
 * (fine-grained FP8: E4M3 with dynamically quantised activations) and
 * Validation list (partial blocks). The 1x128 slice, amax/448 and
 * round-to-nearest-even are this library's reading of "dynamic activations".
 */
dmoe_status dmoe_quant_act(const uint16_t* x, int32_t rows, int32_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                           float* scales, int64_t lds, hipStream_t stream);

/*
 * Weight preparation (not part of the timed layer): 128x128 block quantisation
 * of one FP32 weight matrix w [rows, ldw] to E4M3 codes, with the same
 * amax/448 rule over each block's valid elements.
 * q: [round_up(rows, 128), ldq] codes, ldq >= round_up(cols, 128); padding rows
 * and columns are written as 0x00. scales: [ceil(rows/128), ceil(cols/128)]
 * FP32 dense. Requires cols % 4 == 0, ldw % 4 == 0.
 * Source: Transformers PR #47844 "Add dots3-note Preview model support", implementation list
 * (E4M3 weights with one scale per 128x128 block) and the authors' reply on
 * partial weight blocks.
 */
dmoe_status dmoe_quant_weight_blocks(const float* w, int32_t rows, int32_t cols, int64_t ldw, uint8_t* q,
                                     int64_t ldq, float* scales, hipStream_t stream);

/*
 * Grouped gate/up projection with fused SwiGLU over the permuted rows:
 * for local expert e and row r in [offsets[e], offsets[e+1]):
 *   a_r = a[row_token[r]] (or a[r] when row_token is NULL),
 *   g = a_r . Wg_e^T, u = a_r . Wu_e^T, h[r, :] = bf16(silu(g) * u).
 * BF16: a is [*, lda] BF16, weights BF16, FP32 accumulation.
 * FP8: a is [*, lda] E4M3 codes with scales a_scales [*, ldas] (one per 128
 * columns), weights E4M3 with block scales; each 128-wide K slice's code
 * product is scaled by a_scale * w_scale and added in FP32.
 * h: [max_rows, ldh] BF16, ldh >= round_up(F, 128); columns [F, round_up(F,
 * 128)) are written as 0. Rows past offsets[E_loc] are not written.
 * max_rows: host-side upper bound on offsets[E_loc] (T*K for routed rows); it
 * sizes the grid and the tile schedule, so it must not be below the real row
 * count (rows past the capacity it implies are not computed).
 * row_token: every row it names satisfies (row + 1) * lda * element size <=
 * 4 GiB (without row_token the check is max_rows * lda * element size, done
 * here); DMOE_ERR_UNSUPPORTED when an expert's weights span more than 4 GiB.
 * ws: at least dmoe_gemm_ws_bytes(max_rows, E_loc).
 * Source: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
 * hidden_act (silu), mlp_bias (no bias on gate_proj, up_proj, down_proj),
 * moe_intermediate_size; model card "dots-studio/dots3-note-prev", Model
 * Overview table (256 experts of width 1536 on hidden 5120); Transformers PR #47844 "Add dots3-note Preview model support",
 * implementation list (fine-grained FP8 GEMMs with 128x128 weight blocks).
 */
size_t dmoe_gemm_ws_bytes(int32_t max_rows, int32_t E_loc);
dmoe_status dmoe_grouped_gemm_gateup(int32_t dtype, const void* a, int64_t lda, const float* a_scales,
                                     int64_t ldas, const int32_t* row_token, const int32_t* offsets,
                                     int32_t E_loc, int32_t max_rows, const void* w_gate, const void* w_up,
                                     int64_t ldw, const float* w_scales_gate, const float* w_scales_up, int32_t H,
                                     int32_t F, uint16_t* h, int64_t ldh, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * Grouped down projection: o[r, :] = bf16(h_r . Wd_e^T) for the rows of each
 * local expert, with the same FP8 block-scale rule over K = F (the last K
 * slice may be partial; padded columns of h and Wd are zero).
 * h: [max_rows, ldh] BF16 or E4M3 codes (+ h_scales [max_rows, ldhs]);
 * o: [max_rows, ldo] BF16.
 * Source: as dmoe_grouped_gemm_gateup (down_proj of the same expert). On the
 * FP8 path h is quantised like any activation before this call (Transformers PR #47844 "Add dots3-note Preview model support",
 * implementation list: dynamically quantised activations).
 */
dmoe_status dmoe_grouped_gemm_down(int32_t dtype, const void* h, int64_t ldh, const float* h_scales, int64_t ldhs,
                                   const int32_t* offsets, int32_t E_loc, int32_t max_rows, const void* w_down,
                                   int64_t ldw, const float* w_scales_down, int32_t F, int32_t H, uint16_t* o,
                                   int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Shared expert (Dots3NoteTextConfig n_shared_experts = 1,
 * shared_experts_intermediate_size): s_out[t] = bf16(down(q(bf16(silu(gate a_t)
 * * up a_t)))) for tokens t in [0, T_s), i.e. the routed expert computation
 * with one group of T_s rows and the identity row map. a/a_scales as in the
 * gate/up call; weights in the single-expert layout above; s_out [T_s, lds_out].
 * ws: at least dmoe_shared_expert_ws_bytes(dtype, T_s, H, F_s).
 * Source: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
 * n_shared_experts (1) and shared_experts_intermediate_size; model card
 * "dots-studio/dots3-note-prev", Model Overview table (1 shared expert). Its
 * output enters the sum with weight 1 (the config gives it no gate).
 */
size_t dmoe_shared_expert_ws_bytes(int32_t dtype, int32_t T_s, int32_t H, int32_t F_s);
dmoe_status dmoe_shared_expert(int32_t dtype, const void* a, int64_t lda, const float* a_scales, int64_t ldas,
                               int32_t T_s, const void* w_gate, const void* w_up, const void* w_down,
                               int64_t ldw_gu, int64_t ldw_d, const float* w_scales_gate,
                               const float* w_scales_up, const float* w_scales_down, int32_t H, int32_t F_s,
                               uint16_t* s_out, int64_t lds_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Deterministic gather combine:
 *   y[t] = bf16( sum_{k=0..K-1, token_row[t,k] >= 0} topk_w[t,k] * o[token_row[t,k]]
 *                + (t < T_s ? s_out[t] : 0) ),
 * accumulated in FP32 in slot order, no atomics. s_out may be NULL (T_s
 * ignored). o: [*, ldo] BF16; y: [T, ldy] BF16. Requires 1 <= K <= 64 and
 * H % 8 == 0.
 * Source: Transformers documentation "Dots 3 Note Preview", Dots3NoteTextConfig
 * norm_topk_prob and routed_scaling_factor (the weights applied here) and
 * n_shared_experts (the shared output, added with weight 1). The pages fix no
 * summation order; FP32 in slot order is this library's reading.
 */
dmoe_status dmoe_combine(const uint16_t* o, int64_t ldo, const int32_t* token_row, const float* topk_w,
                         const uint16_t* s_out, int64_t lds, int32_t T_s, int32_t T, int32_t K, int32_t H,
                         uint16_t* y, int64_t ldy, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Whole layer: router logits (unless given) -> route -> permute -> [FP8:
 * quantise x] -> gate/up + SwiGLU -> [FP8: quantise h] -> down -> shared
 * expert -> combine. One stream, no host synchronisation.
 * ------------------------------------------------------------------------- */
typedef struct dmoe_layer_desc {
  int32_t T;            /* tokens */
  int32_t H;            /* hidden size, multiple of 128 */
  int32_t F;            /* routed expert FFN width */
  int32_t F_s;          /* shared expert FFN width (0: no shared expert) */
  int32_t E;            /* routed experts in the model */
  int32_t E_loc;        /* experts held here: [e0, e0 + E_loc) */
  int32_t e0;
  int32_t K;            /* experts per token */
  int32_t T_s;          /* the shared expert runs on tokens [0, T_s) */
  int32_t dtype;        /* DMOE_BF16 or DMOE_FP8_E4M3 */
  int32_t logits_given; /* 1: ptrs.logits is an input; 0: computed from x and w_router */
  /* Routing options as in dmoe_route_grouped; zero values select the defaults. */
  int32_t n_group;              /* 0 or 1: ungrouped */
  int32_t topk_group;           /* 0: every group */
  int32_t no_renormalize;       /* 0: renormalise over the selected experts (norm_topk_prob) */
  float routed_scaling_factor;  /* 0: 1.0 */
  int32_t scoring;              /* DMOE_SCORING_SOFTMAX (0) or DMOE_SCORING_SIGMOID (ptrs.score_bias) */
} dmoe_layer_desc;

typedef struct dmoe_layer_ptrs {
  const uint16_t* x; /* [T, ldx] BF16 */
  int64_t ldx;
  const float* w_router; /* [E, H] FP32 (when logits are computed) */
  float* logits;         /* [T, E] FP32: output, or input when logits_given */
  const float* score_bias; /* [E] FP32 selection bias for sigmoid scoring, or NULL */
  const void* w_gate;    /* routed experts, layout above */
  const void* w_up;
  const void* w_down;
  int64_t ldw_gu, ldw_d;
  const float* ws_gate; /* FP8 block scales (NULL for BF16) */
  const float* ws_up;
  const float* ws_down;
  const void* sw_gate; /* shared expert, same layout with one expert */
  const void* sw_up;
  const void* sw_down;
  int64_t ldsw_gu, ldsw_d;
  const float* sws_gate;
  const float* sws_up;
  const float* sws_down;
  int32_t* topk_ids; /* [T, K] output */
  float* topk_w;     /* [T, K] output */
  uint16_t* y;       /* [T, ldy] BF16 output */
  int64_t ldy;
} dmoe_layer_ptrs;

/*
 * Whole layer on one stream: the steps above in order, reading desc and ptrs
 * (host structs, not retained). ws: device workspace of at least
 * dmoe_forward_ws_bytes(desc) bytes, 16-byte aligned; its contents after the
 * call can be inspected with dmoe_forward_ws_offset. dmoe_forward_ws_bytes
 * returns 0 for an invalid desc.
 * Source: the MoE block as Transformers documentation "Dots 3 Note Preview"
 * configures it (Dots3NoteTextConfig n_routed_experts 256, n_shared_experts
 * 1, num_experts_per_tok 8, hidden_size 5120, moe_intermediate_size 1536) and
 * the model card "dots-studio/dots3-note-prev", Model Overview table; FP8 as
 * in Transformers PR #47844 "Add dots3-note Preview model support", implementation list. The pages
 * describe no workspace: its layout is this library's own.
 */
size_t dmoe_forward_ws_bytes(const dmoe_layer_desc* desc);
dmoe_status dmoe_forward(const dmoe_layer_desc* desc, const dmoe_layer_ptrs* ptrs, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * dmoe_forward, recording caller-created events between its stages so a
 * profiler or benchmark can time each stage on the stream it runs on.
 * stage_events: host array of DMOE_STAGES + 1 hipEvent_t; event i is recorded
 * before stage i and event DMOE_STAGES after the last one. Stages, in order:
 * 0 router logits (empty when logits are given; with T <= 256 and
 * H % 1024 == 0 it leaves four partial sums over K in the workspace, which
 * stage 1 adds and stores in ptrs.logits), 1 route, 2 permute and tile
 * schedule, 3 quantise x (FP8), 4 gate/up + SwiGLU, 5 quantise h (FP8),
 * 6 down, 7 shared expert, 8 combine. A NULL entry is skipped (each recorded
 * event is a stream marker that costs a few microseconds of queue time).
 * Recording events adds stream markers only; the results are identical to
 * dmoe_forward.
 * Source: as dmoe_forward.
 */
#define DMOE_STAGES 9
dmoe_status dmoe_forward_timed(const dmoe_layer_desc* desc, const dmoe_layer_ptrs* ptrs, void* ws, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t* stage_events);

/*
 * Views into the forward workspace, for inspection after dmoe_forward (host
 * byte offsets from ws; -1 if the buffer does not exist for this desc):
 * 0 offsets, 1 row_token, 2 row_slot, 3 token_row, 4 x codes, 5 x scales,
 * 6 h (BF16; not written for FP8 when the gate/up launch quantises h itself,
 * see dmoe_forward_gateup_kernel), 7 h codes, 8 h scales, 9 o, 10 shared output.
 */
int64_t dmoe_forward_ws_offset(const dmoe_layer_desc* desc, int32_t which);

/*
 * Name of the GEMM kernel that the layer's gate/up launch runs for this desc:
 * "gemm_stage_kernel" (weight streaming, few rows per expert), "gemm_tile_kernel"
 * or "gemm_wide_kernel" (a static string; NULL for an invalid desc). For
 * profiling and reports; no GPU work. With FP8 the wide kernel quantises h in
 * its epilogue, so workspace view 6 (BF16 h) is then not written.
 */
const char* dmoe_forward_gateup_kernel(const dmoe_layer_desc* desc);

/*
 * Name of the GEMM kernel that the layer's down launch (routed experts, and
 * the shared expert when it runs as an extra group of the routed launches, as
 * it does when F_s == F) runs for this desc, from the same three (a static
 * string; NULL for an invalid desc). For profiling and reports; no GPU work.
 */
const char* dmoe_forward_down_kernel(const dmoe_layer_desc* desc);

/*
 * dmoe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is a fixed device array inside the
 * library of DMOE_NOALLOC_WS_BYTES (24 MiB): each GPU the library runs on
 * holds its own copy until the process ends. That covers
 * dmoe_forward_ws_bytes(desc) of the full-size layer (H 5120, F 1536, 256
 * experts, top-8) up to 128 tokens in BF16 and FP8 (17.5 MiB); a layer that
 * needs more returns DMOE_ERR_WORKSPACE and enqueues nothing. The call
 * allocates and frees nothing. The array's device address is looked up once
 * per device (the device of `stream`, or the current device for the null
 * stream) on the first call there. Every call on one GPU shares the array and
 * it keeps the last call's contents (dmoe_forward_ws_offset offsets index into
 * it); calls that overlap on one GPU, from several streams or threads, race
 * on it and must be serialised by the caller. Results equal dmoe_forward's
 * bit for bit.
 */
#define DMOE_NOALLOC_WS_BYTES (24u << 20)
dmoe_status dmoe_forward_noalloc(const dmoe_layer_desc* desc, const dmoe_layer_ptrs* ptrs, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DMOE_H */
