/*
 * moe.h - C ABI of the MI355X (gfx950) sparse Mixture-of-Experts MLP block.
 *
 * The block is the Qwen3-MoE / Qwen3-VL-MoE expert layer:
 *   y = sum over the token's top-k experts of w_i * expert_i(x)  [+ sigmoid(w_s . x) * shared(x)]
 * ("27. Mixture of experts", sections "The router", "The shared expert" and "Dispatch";
 *  "Qwen3-VL + MoE: train to deploy", section "What a mixture-of-experts layer is", its equation).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned by the caller.
 *    The library never allocates or frees device memory and keeps no state between calls.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *    Outputs are valid once that stream has completed. There is no host synchronisation.
 *  - Validation runs on the host before anything is enqueued. A call that returns an error has
 *    enqueued nothing, except MOE_ERR_HIP, which reports a failed launch (hipGetLastError).
 *    moe_last_error() then gives a message naming the offending argument.
 *  - n_tokens == 0 is a successful no-op (after the configuration itself is validated).
 *  - Inputs are assumed finite; what NaN or Inf routing selects is unspecified.
 *  - Calls on one stream are ordered; concurrent calls on different streams must not share
 *    output or workspace buffers.
 *
 * Layouts (the stacked-expert layout of "27. Mixture of experts", section "Dispatch", class Experts,
 * whose linear layers read weights as [out, in], so every GEMM operand is contiguous along K):
 *   x           [N, D]
 *   w_router    [E, D]             logits = x W_r^T, no bias
 *   gate_up     [E, 2I, D]         rows [0, I) gate, rows [I, 2I) up
 *   down        [E, D, I]
 *   shared_gate_up [2I_s, D], shared_down [D, I_s], w_shared_gate [D]
 * dtype (moe_config.dtype) applies to x and every weight; routing outputs are always fp32
 * weights and int32 expert ids; the per-assignment expert outputs are fp32 or an fp16 form (see
 * "Expert outputs").
 *
 * Packed weights (moe_config.weight_layout = MOE_LAYOUT_PACKED): gate_up, down, shared_gate_up,
 * shared_down and, when n_experts is a multiple of 16, w_router (as a [1, E, D] stack) instead hold
 * the output of moe_pack_weights, a one-time rearrangement (at model load) of each [G, R, K] matrix
 * into 16 x 32 blocks of 1 KB stored in the order the matrix cores read them, so that every weight
 * load is one contiguous kilobyte. With another n_experts, w_router keeps the row layout. The values
 * are the same; results are bitwise identical to the row layout. bf16 only, with hidden, inter and
 * shared_inter multiples of 128. w_shared_gate is a vector and keeps its layout.
 *
 * Quantised experts (moe_config.weight_layout = MOE_LAYOUT_Q8, MOE_LAYOUT_Q4 or MOE_LAYOUT_F8;
 * weight-only quantisation of the experts with the router kept in bf16: "Qwen3-VL-MoE" Keras port,
 * section "Lower memory"; "27. Mixture of experts", section "Dispatch" and stretch exercise 3;
 * "Qwen3-VL + MoE: train to deploy", the FP8 copy of the 30B model): gate_up,
 * down, shared_gate_up and shared_down each hold a quantised stack made by moe_quantize_weights
 * (with the same n_groups, rows and cols the expert entry points see), w_router is packed (or not)
 * as for MOE_LAYOUT_PACKED and w_shared_gate keeps its layout. Same shape rules as MOE_LAYOUT_PACKED. The
 * layer then computes with the weights code * scale (for FP8, the e4m3 value of the code times the
 * scale; for int4, code * group multiplier * row scale): the codes enter the matrix cores exactly
 * (as bf16) and each output column's fp32 sum is multiplied by its row's scale.
 *
 * Expert outputs (moe_config.expert_out): the per-assignment outputs out[p, :] that the down
 * projection writes and moe_combine weights and sums ("27. Mixture of experts", section "Dispatch",
 * grouped steps 3-4). MOE_EXPERT_OUT_F32 (0): fp32 rows [rows, D]. MOE_EXPERT_OUT_F16S (1): each
 * row is D fp16 values followed by D / 16 int8 exponents, padded to a multiple of 16 bytes:
 *   row stride S = round_up(2 D + D / 16, 16) bytes; value of column c = fp16[c] * 2^exp[c / 16];
 *   exp of a 16-column group = clamp(floor(log2 m) - 14, -128, 127) for the group's largest |v| = m
 *   (0 when m = 0), so every scaled value is below 2^15 (at most 2^15 once rounded) and in range;
 *   fp16[c] = v * 2^-exp rounded to nearest, ties to even (the only rounding: 2^-11 relative,
 *   against 2^-8 for a bf16 output). Non-finite outputs are not supported (inputs are finite).
 * It halves the bytes the down projection writes and moe_combine reads. bf16 layers with D % 16 == 0
 * and weight_layout MOE_LAYOUT_ROWS or MOE_LAYOUT_PACKED only (else MOE_ERR_UNSUPPORTED). An
 * expert-output buffer sized [rows, D] fp32 holds either form (S <= 4 D).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, negative or zero size, k > E, ...      */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not implemented: dtype, alignment, E > 512, ...       */
  MOE_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than moe_workspace_bytes()   */
  MOE_ERR_HIP = -4          /* a kernel launch failed                                           */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_PACKED = 1, MOE_LAYOUT_Q8 = 2, MOE_LAYOUT_Q4 = 3, MOE_LAYOUT_F8 = 4
} moe_weight_layout;

typedef enum { MOE_EXPERT_OUT_F32 = 0, MOE_EXPERT_OUT_F16S = 1 } moe_expert_out;

/* Shape and options of one MoE layer. Refuses, never defaults: every field must be set
 * (the config-ingestion lesson of "27. Mixture of experts", section "Qwen3-MoE", Note). */
typedef struct {
  int64_t n_tokens;       /* N  >= 0: tokens, flattened over batch and sequence               */
  int64_t hidden;         /* D  >= 1: model width (bf16: multiple of 8; fp32: multiple of 4)  */
  int64_t n_experts;      /* E  in [1, 512]                                                   */
  int64_t top_k;          /* k  in [1, E]                                                     */
  int64_t inter;          /* I  >= 1: expert inner width (same alignment as D)                */
  int64_t shared_inter;   /* I_s >= 0: shared expert inner width, 0 = no shared expert        */
  int32_t norm_topk_prob; /* 1: divide kept weights by their sum; 0: keep the probabilities   */
  int32_t dtype;          /* moe_dtype of x and all weights                                   */
  int32_t out_dtype;      /* moe_dtype of y                                                   */
  int32_t weight_layout;  /* moe_weight_layout of the weights (see "Packed weights" and
                             "Quantised experts" above)                                       */
  int32_t expert_out;     /* moe_expert_out: form of the expert outputs (see "Expert outputs") */
} moe_config;

/* Human-readable name of a status code. Never NULL. */
const char* moe_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of device workspace moe_forward needs for this configuration (also enough for
 * moe_permute and moe_router_stats). Host only; no GPU needed. Returns MOE_ERR_INVALID_ARG/UNSUPPORTED for a bad
 * configuration, else writes *bytes. */
int moe_workspace_bytes(const moe_config* cfg, size_t* bytes);

/* Router: logits = x W_r^T (fp32 accumulation, logits never rounded), p = softmax over all E in
 * fp32, the k largest p in descending order with equal p going to the lower expert index, then
 * w = p_sel / sum(p_sel) when norm_topk_prob ("27. Mixture of experts", section "The router",
 * steps 1-3, TopKRouter and the parity note).
 *   x [N, D], w_router [E, D]                      (dtype)
 *   w_shared_gate [D] or NULL                      (dtype) shared-expert gate vector w_s
 *   logits [N, E] fp32 or NULL                     optional copy of the router logits
 *   weights [N, k] fp32, experts [N, k] int32      required outputs
 *   shared_scale [N] fp32 or NULL                  sigmoid(w_s . x); required iff w_shared_gate
 *   ws, ws_bytes: optional workspace (256-byte aligned, at least moe_workspace_bytes()). With it,
 *     few-token batches split the D contraction over more workgroups (partial logits summed in a
 *     fixed order); with ws == NULL the router runs in one pass. The two give the same selection
 *     rule but may differ in the last bits of the fp32 logits. */
int moe_route(const moe_config* cfg, const void* x, const void* w_router, const void* w_shared_gate,
              float* logits, float* weights, int32_t* experts, float* shared_scale, void* ws, size_t ws_bytes,
              void* stream);

/* Sigmoid-score router ("27. Mixture of experts", section "The router", the note on other routers;
 * "Qwen3-VL + MoE: train to deploy", section "How the router and experts learn", the item on balancing without a loss): logits as moe_route
 * (fp32, never rounded), s = sigmoid(logits) in fp32, the k experts with the largest s + bias
 * (descending, equal keys to the lower index); the bias only picks, so
 * weights = s of the picked experts, divided by their sum when norm_topk_prob.
 *   bias [E] fp32 on device, or NULL (zeros); other arguments as moe_route (no shared gate). */
int moe_route_sigmoid(const moe_config* cfg, const void* x, const void* w_router, const float* bias, float* logits,
                      float* weights, int32_t* experts, void* ws, size_t ws_bytes, void* stream);

/* Selection-bias nudge after a step ("Qwen3-VL + MoE: train to deploy", section "Balancing without
 * a loss"): bias[e] -= gamma * sign(counts[e] - N k / E), in place, gamma >= 0. counts [E] int32
 * (e.g. moe_permute's), bias [E] fp32, both on device. */
int moe_router_bias_update(const moe_config* cfg, const int32_t* counts, float* bias, float gamma, void* stream);

/* Grouping by expert: the N*k assignments a = n*k + j are sorted by expert id, stably (ties keep
 * assignment order), with no atomics on ranks, so the result is deterministic ("27. Mixture of
 * experts", section "Dispatch", grouped dispatch steps 1-2; stretch exercise 2 for the row-offset
 * prefix sum).
 *   experts [N, k] int32 in [0, E)                 an id outside [0, E) is dropped: not counted,
 *                                                  given no row, slot_pos = -1 (moe_combine then
 *                                                  skips it, as a capacity drop)
 *   counts [E], offsets [E+1] int32                rows of expert e are [offsets[e], offsets[e+1])
 *   token_of [N*k] int32                           token each sorted row came from
 *   slot_pos [N*k] int32                           sorted row of assignment a (inverse permutation)
 *   x [N, D] and x_perm [N*k, D] (dtype)           optional pair: x_perm[p] = x[token_of[p]]
 *   ws, ws_bytes                                   workspace, at least moe_workspace_bytes() */
int moe_permute(const moe_config* cfg, const int32_t* experts, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* token_of, int32_t* slot_pos, void* x_perm, void* ws,
                size_t ws_bytes, void* stream);

/* moe_permute with a capacity limit ("Qwen3-VL + MoE: train to deploy", section "How the router and experts learn", the item on capacity limits):
 * each expert keeps its first `capacity` (>= 0) assignments in assignment order a = n*k + j; the
 * rest are dropped (their token passes through unchanged). counts/offsets cover the kept rows
 * (offsets[E] = rows kept), token_of and x_perm hold the kept rows only, and slot_pos[a] = -1 for
 * a dropped assignment, which moe_combine then skips. */
int moe_permute_capped(const moe_config* cfg, int64_t capacity, const int32_t* experts, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* token_of, int32_t* slot_pos, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU experts ("27. Mixture of experts", section "Dispatch", Experts.expert and grouped
 * step 3: one launch runs every group's matmuls on its contiguous rows). For group g and each
 * row p in [offsets[g], offsets[g+1]):
 *   h[p, i]   = silu(sum_d X[p, d] G[g, i, d]) * (sum_d X[p, d] G[g, I + i, d])  (moe_expert_gate_up)
 *   out[p, :] = sum_i h[p, i] Dn[g, :, i]                                        (moe_expert_down)
 * where X[p] = x[row_index[p]] if row_index is non-NULL, else x[p] (x holds max_rows rows).
 * cfg gives D (hidden) and dtype; n_tokens, n_experts, top_k and inter of cfg are not used here.
 *   n_groups G >= 1, inter I >= 1 (the width of these experts: cfg.inter or cfg.shared_inter)
 *   max_rows: host-known upper bound of offsets[G] (e.g. N*k); sizes the launch and buffers
 *   offsets [G+1] int32 on device, offsets[0] == 0 and non-decreasing, or NULL for one group of
 *     max_rows rows
 *   gate_up [G, 2I, D], down [G, D, I] (dtype)
 *   h [max_rows, I] (dtype; bf16 when dtype is bf16, the matrix-core input), out: max_rows expert-
 *   output rows in the form cfg.expert_out selects ([max_rows, D] fp32, or rows of S bytes)
 * Accumulation is fp32; with bf16 the SwiGLU product is rounded to bf16 once (the second GEMM's
 * input). Rows at or past offsets[G] are left untouched. */
int moe_expert_gate_up(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows,
                       const void* x, const int32_t* row_index, const int32_t* offsets,
                       const void* gate_up, void* h, void* stream);
int moe_expert_down(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows,
                    const int32_t* offsets, const void* h, const void* down, float* out, void* stream);
/* Both of the above in order. */
int moe_expert_ffn(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows,
                   const void* x, const int32_t* row_index, const int32_t* offsets,
                   const void* gate_up, const void* down, void* h, float* out, void* stream);

/* Packs a row-major bf16 matrix stack src [G, R, K] (R % 16 == 0, K % 32 == 0) into dst, the
 * layout of MOE_LAYOUT_PACKED: block (g, rb, kb) of rows rb*16 .. +15 and columns kb*32 .. +31 is
 * 1 KB at byte offset ((g * R/16 + rb) * K/32 + kb) * 1024, holding at 16-byte slot l the eight
 * values of row rb*16 + l % 16, columns kb*32 + 8 (l / 16) .. + 7. dst has src's size and must
 * not overlap it. Use it on w_router (G = 1, R = E, K = D), gate_up (R = 2I, K = D), down (R = D,
 * K = I) and the shared pair.
 * cfg gives dtype (must be bf16); its other fields are not used. */
int moe_pack_weights(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, const void* src,
                     void* dst, void* stream);

/* Weight-only quantisation of a row-major bf16 stack src [G, R, K] into dst, once at model load:
 * int8 or FP8 (cfg.weight_layout MOE_LAYOUT_Q8 / MOE_LAYOUT_F8; R % 16 == 0, K % 32 == 0) or int4
 * (MOE_LAYOUT_Q4; R % 16 == 0, K % 128 == 0); cfg gives dtype (must be bf16) and weight_layout, its
 * other fields are not used. The pages give bit widths, not a quantiser. Rules, per output row r
 * (every division an IEEE fp32 division, every rounding to nearest with ties to even):
 *   int8: m = max |w| over the row, scale = m / 127, code = clamp(rint(w / scale), -127, 127).
 *   FP8: scale = m / 448, code = the OCP e4m3 byte (1 sign, 4 exponent bits with bias 7, 3
 *     mantissa bits, subnormals below 2^-6) nearest to clamp(w / scale, -448, 448), the sign of zero
 *     kept.
 *   int4 (a scale per 32 columns, as the row scale times an integer): s = m / 224 (the row scale);
 *     for each group q of columns 32 q .. 32 q + 31, mult = min(ceil(max |w over q| / (7 s)), 32)
 *     with 7 s an fp32 product, step = s * mult (fp32), code = clamp(rint(w / step), -7, 7); the
 *     weight is code * mult * s, and code * mult (|.| <= 224) is exact in bf16.
 *   An all-zero row has scale 0 and codes 0 (int4: multipliers 0); an all-zero int4 group has
 *   multiplier 0 and codes 0.
 * dst layout (moe_quantized_bytes() bytes, 16-byte aligned, not overlapping src): codes, then the
 * scales fp32 [G, R] (int4: the row scales s).
 *   int8 / FP8 codes, G R K bytes in the block order of moe_pack_weights: block (g, rb, kb) of rows
 *     rb*16 .. +15 and columns kb*32 .. +31 takes 512 bytes at ((g * R/16 + rb) * K/32 + kb) * 512;
 *     its slot l (8 bytes, l = 0..63) holds the codes of row rb*16 + l % 16, columns
 *     kb*32 + 8 (l / 16) + i, i = 0..7, in byte i (two's complement, or the e4m3 byte).
 *   int4 codes, in super-blocks of 16 rows x 128 columns: super-block (g, rb, kq) of rows rb*16 ..
 *     +15 and columns kq*128 .. +127 takes 1088 bytes at ((g * R/16 + rb) * K/128 + kq) * 1088.
 *     Its first 1024 bytes are 64 slots of 16 bytes; slot l holds row rb*16 + l % 16, and its bytes
 *     4 t .. 4 t + 3 (t = 0..3) the codes of columns (4 kq + t) * 32 + 8 (l / 16) + i, i = 0..7, code
 *     i as the 4-bit value code + 8 in byte i % 4, the low nibble for i < 4 and the high nibble for
 *     i >= 4. The last 64 bytes are the multipliers: byte 1024 + 4 r + t for row rb*16 + r and
 *     columns (4 kq + t) * 32 .. + 31.
 * moe_quantized_bytes: G R K + 4 G R bytes for int8 / FP8, 1088 G (R / 16) (K / 128) + 4 G R for
 * int4. */
int moe_quantized_bytes(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, size_t* bytes);
int moe_quantize_weights(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, const void* src,
                         void* dst, void* stream);

/* Backward pass of the block ("Qwen3-VL + MoE: train to deploy", section "What a mixture-of-experts
 * layer is": the router and the experts are trained end to end through the gated sum). Given the
 * output gradient dy, writes the gradients of L = sum(dy * y) with respect to x and every weight:
 *   router   w = p_sel / S (S = sum of p_sel) when norm_topk_prob, else p_sel; the top-k choice is
 *            piecewise constant, so unselected probabilities get no gradient:
 *            dw[n, j] = dy[n] . expert_{e_j}(x[n]),
 *            dp_sel = (dw - sum_j dw_j w_j) / S (or dw), dlogits = p (dp - sum_e dp_e p_e),
 *            dW_r = dlogits^T x, dx += dlogits W_r
 *   experts  with a = x G_e^T, b = x U_e^T, h = silu(a) b and the row's gradient w dy:
 *            dh = w dy Dn_e, da = dh b silu'(a), db = dh silu(a),
 *            dDn_e = sum (w dy)^T h, dG_e = sum da^T x, dU_e = sum db^T x, dx += da G_e + db U_e
 *   shared   the same with all N tokens, row weight g = sigmoid(w_s . x) (1 without w_s), and for
 *            the gate dz = (dy . shared(x)) g (1 - g): dw_s = sum dz x, dx += dz w_s
 * The forward's routing, grouping and pre-activations are recomputed from x (nothing is kept from a
 * moe_forward call). bf16 layers: matrix-core inputs are bf16 (h, w dy, da, db and dlogits rounded
 * once), accumulation fp32. fp32 layers: every intermediate stays fp32 (FMA weight-gradient kernel).
 * The sums over an expert's rows run in row order, deterministic.
 *   cfg: dtype bf16 or fp32, weight_layout MOE_LAYOUT_ROWS (else MOE_ERR_UNSUPPORTED); expert_out
 *     does not matter here (the backward's intermediates are its own, fp32 rows)
 *   x [N, D], w_router [E, D], gate_up [E, 2I, D], down [E, D, I], dy [N, D]   (cfg.dtype, row-major)
 *   shared_gate_up [2I_s, D], shared_down [D, I_s], w_shared_gate [D] (cfg.dtype): as moe_forward
 *     (required iff shared_inter > 0; w_shared_gate may be NULL: ungated)
 *   dx [N, D], dw_router [E, D], dgate_up [E, 2I, D], ddown [E, D, I]       (fp32, overwritten;
 *     an expert that received no token gets zeros)
 *   dshared_gate_up [2I_s, D], dshared_down [D, I_s] (fp32; iff shared_inter > 0),
 *   dw_shared_gate [D] (fp32; iff w_shared_gate)
 *   ws, ws_bytes: at least moe_backward_workspace_bytes() bytes, 256-byte aligned
 * All tensors 16-byte aligned. */
int moe_backward_workspace_bytes(const moe_config* cfg, size_t* bytes);
int moe_backward(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up, const void* down,
                 const void* shared_gate_up, const void* shared_down, const void* w_shared_gate, const void* dy,
                 float* dx, float* dw_router, float* dgate_up, float* ddown, float* dshared_gate_up,
                 float* dshared_down, float* dw_shared_gate, void* ws, size_t ws_bytes, void* stream);

/* Router load statistics and the Switch-style balance loss ("Qwen3-VL + MoE: train to deploy",
 * section "How the router and experts learn", the item on an auxiliary balance loss, its N read as the number of experts):
 *   f[e] = counts[e] / (N k)                        fraction of the assignments routed to e
 *   P[e] = (1/N) sum_n softmax(logits[n])[e]         mean router probability (fp32 softmax)
 *   loss = E * sum_e f[e] P[e]                        1 for perfectly even routing; the caller
 *                                                     applies its coefficient
 *   logits [N, E] fp32 (moe_route's optional output), counts [E] int32 (moe_permute's)
 *   f [E], P [E], loss [1] fp32 on device
 *   ws, ws_bytes: workspace of at least moe_workspace_bytes(cfg) bytes
 * Per-block partial sums in token order, then fixed-order fp64 sums: deterministic.
 * N = 0 writes zeros. */
int moe_router_stats(const moe_config* cfg, const float* logits, const int32_t* counts, float* f, float* P,
                     float* loss, void* ws, size_t ws_bytes, void* stream);

/* Weighted unpermute ("27. Mixture of experts", section "Dispatch", grouped step 4, and the
 * shared-expert equation): y[n] = sum_{j<k} w[n,j] * out_perm[slot_pos[n*k+j]]
 *                                  (+ shared_scale[n] * shared_out[n]),
 * summed in fp32 in slot order j = 0..k-1, then the shared term, rounded once to out_dtype.
 * A gather per token (no atomics): deterministic.
 *   out_perm: N*k expert-output rows in the form cfg.expert_out selects ([N*k, D] fp32 or rows of
 *     S bytes, see "Expert outputs"), weights [N, k] fp32, slot_pos [N*k] int32 (-1: a dropped pair,
 *     skipped)
 *   shared_out: N rows in the same form, or NULL; shared_scale [N] fp32 or NULL (NULL with
 *     shared_out: scale 1)
 *   y [N, D] (out_dtype) */
int moe_combine(const moe_config* cfg, const float* out_perm, const float* weights,
                const int32_t* slot_pos, const float* shared_out, const float* shared_scale, void* y,
                void* stream);

/* The whole block ("27. Mixture of experts", section "The shared expert", SparseMoeBlock.forward:
 * router, then the experts on their routed rows (section "Dispatch", the grouped form), then the
 * weighted sum back into each token plus the gated shared term): moe_route (with ws) -> moe_permute -> moe_expert_ffn over the
 * routed groups (rows gathered straight from x) -> [shared expert as one more group over all N rows]
 * -> moe_combine. y has x's shape [N, D].
 *   shared_gate_up, shared_down: required iff cfg.shared_inter > 0; w_shared_gate may be NULL
 *     (ungated shared expert, scale 1)
 *   y [N, D] (out_dtype); weights_out [N, k] fp32 / experts_out [N, k] int32: optional copies
 *   ws, ws_bytes: workspace of at least moe_workspace_bytes(cfg) bytes, 256-byte aligned */
int moe_forward(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up,
                const void* down, const void* shared_gate_up, const void* shared_down,
                const void* w_shared_gate, void* y, float* weights_out, int32_t* experts_out,
                void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward with the same arguments minus the workspace.
 * It calls no hipMalloc / hipFree (nor any allocating routine) and runs the kernels of moe_forward
 * (results bitwise equal) on a scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device it runs on, from that device's first call until the process ends.
 *   Limit: moe_workspace_bytes(cfg) must not exceed MOE_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. the
 *     512-token, 60-expert layer of the Keras port, or decode batches of a few hundred tokens at
 *     D = 2048, k = 8); a larger layer returns MOE_ERR_WORKSPACE before anything is enqueued.
 *   Every call on one device shares that device's scratch, which keeps the last call's contents
 *     (nothing in it needs clearing: each call writes what it reads). Calls that overlap on one
 *     device (different streams, or threads without ordering) race on it: order them.
 *   The device is the current HIP device; stream must belong to it. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up,
                        const void* down, const void* shared_gate_up, const void* shared_down,
                        const void* w_shared_gate, void* y, float* weights_out, int32_t* experts_out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
