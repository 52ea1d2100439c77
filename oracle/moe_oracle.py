"""CPU oracle for the sparse Mixture-of-Experts MLP block (Qwen3-MoE / Qwen3-VL-MoE).

TEST INFRASTRUCTURE ONLY. This module is imported by the tests, by the package's smoke check and
by the CPU-baseline leg of the benchmark. The product path never imports, calls or falls back to it.
It shares no code with the HIP path: plain NumPy, float64 unless a page fixes the precision.

Page names used in citations:
  [MoE-ch27]  "27. Mixture of experts" (inference.shantanugoel.com/27-moe)
  [VL-MoE-src] the Qwen3-VL-MoE source walk-through (agent.csdn.net article on qwen3_vl_moe)
  [VL-post]   "Qwen3-VL + MoE: train to deploy" (gopikrishnatummala.com)
  [Keras]     "Qwen3-VL-MoE" Keras port docs (imvision12.github.io/ZeroModels/qwen3_vl_moe)
  [30B-cfg]   Qwen3-VL-30B-A3B MoE architecture explainer (adg.csdn.net)

Every function is pinned by tests in tests/test_oracle.py against the pages' worked examples,
closed forms, special cases and brute force, except where its docstring says "parity unpinned".
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------------------------
# Router: [MoE-ch27] section "The router" (steps 1-3 and the TopKRouter description);
#         [VL-MoE-src] routing section of Qwen3VLMoeTextSparseMoeBlock.forward.
# --------------------------------------------------------------------------------------------

def router_logits(x, w_router):
    """logits[n, e] = sum_d x[n, d] * W_r[e, d]: one linear layer, no bias ([MoE-ch27] "The router").

    Computed in float64 from the stored values, so for bf16 or fp32 inputs it is exact up to
    float64 summation rounding."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def softmax(logits, dtype=np.float32):
    """Softmax over all experts, max-subtracted. The page fixes FP32 for this step ([MoE-ch27],
    "The router", step 1, and the parity note after the example), so the default takes the
    float64 logits to float32 and does exp, sum and divide in float32. ``dtype=np.float64``
    gives the same definition at higher precision (used to cross-check)."""
    lg = np.asarray(logits).astype(dtype)
    m = lg.max(axis=-1, keepdims=True)
    ex = np.exp(lg - m)
    return ex / ex.sum(axis=-1, keepdims=True)


def select_top_k(probs, k):
    """The k largest probabilities per token, in descending order; equal probabilities go to the
    lower expert index ([MoE-ch27] "The router" step 2; ties broken by index per the parity note).

    A stable sort of -p keeps equal keys in index order, which is exactly that rule."""
    order = np.argsort(-probs, axis=-1, kind="stable")
    experts = order[..., :k]
    return experts.astype(np.int64), np.take_along_axis(probs, experts, axis=-1)


def route(x, w_router, k, norm_topk_prob=True, prob_dtype=np.float32):
    """x[N,D] -> (logits[N,E] f64, probs[N,E], weights[N,k], experts[N,k]).

    Steps of [MoE-ch27] "The router": linear scores, FP32 softmax over all E, top-k, then divide the
    kept weights by their sum when norm_topk_prob is set (step 3; also [VL-MoE-src], the
    renormalisation step, which always applies it; [Keras] lists it as a flag)."""
    logits = router_logits(x, w_router)
    probs = softmax(logits, prob_dtype)
    experts, weights = select_top_k(probs, k)
    if norm_topk_prob:
        weights = weights / weights.sum(axis=-1, keepdims=True)
    return logits, probs, weights, experts


def k_gap(probs, k):
    """Per token, p_(k) - p_(k+1) of the sorted probabilities (inf when k == E). Used to find
    tokens whose selection is decided by rounding (a near tie across the top-k boundary)."""
    srt = -np.sort(-np.asarray(probs, np.float64), axis=-1)
    if k >= srt.shape[-1]:
        return np.full(srt.shape[:-1], np.inf)
    return srt[..., k - 1] - srt[..., k]


# --------------------------------------------------------------------------------------------
# Experts: [MoE-ch27] section "Dispatch" (Experts: stacked gate_up_proj [E, 2I, D] with gate rows
# first, down_proj [E, D, I]; expert(e, x) = down(silu(gate) * up)); [VL-MoE-src] expert section.
# --------------------------------------------------------------------------------------------

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu(v, gate_up, down):
    """One SwiGLU expert on rows v[m, D]: gate = first I rows of gate_up, up = last I rows,
    out = (silu(v G^T) * (v U^T)) Dn^T, all in float64 ([MoE-ch27] "Dispatch", Experts.expert)."""
    v = np.asarray(v, np.float64)
    gu = np.asarray(gate_up, np.float64)
    dn = np.asarray(down, np.float64)
    inter = dn.shape[1]
    g = v @ gu[:inter].T
    u = v @ gu[inter:].T
    return (silu(g) * u) @ dn.T


# --------------------------------------------------------------------------------------------
# Dispatch: [MoE-ch27] section "Dispatch: getting tokens to their experts", grouped form steps 1-4.
# --------------------------------------------------------------------------------------------

def permute(experts, n_experts):
    """Sort the N*k assignments a = n*k + j by expert, stably ([MoE-ch27] "Dispatch", grouped step 1).

    Returns counts[E] (bincount), offsets[E+1] (exclusive prefix sum; offsets[e] is where expert e's
    rows start), order[A] (assignment id at each sorted position), token_of[A] = order // k
    (step 2: which token row each sorted position reads) and slot_pos[A], the inverse of order
    (sorted position of assignment a)."""
    experts = np.asarray(experts)
    k = experts.shape[-1]
    flat = experts.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    slot_pos = np.empty_like(order)
    slot_pos[order] = np.arange(flat.size)
    return counts, offsets, order, order // k, slot_pos


def grouped_expert_ffn(x_rows, offsets, gate_up, down):
    """Run group g's SwiGLU expert on its contiguous slice rows[offsets[g]:offsets[g+1]]
    ([MoE-ch27] "Dispatch", grouped step 3). Empty groups are skipped. Returns out_perm[rows, D]."""
    x_rows = np.asarray(x_rows, np.float64)
    out = np.zeros_like(x_rows)                     # expert outputs have the model width D
    for g in range(len(offsets) - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            out[a:b] = swiglu(x_rows[a:b], gate_up[g], down[g])
    return out


def combine(out_perm, weights, slot_pos, shared_out=None, shared_scale=None):
    """Unpermute: y[n] = sum_j w[n, j] * out_perm[slot_pos[n*k + j]] (+ shared_scale[n] * shared_out[n]).

    This is [MoE-ch27] "Dispatch" grouped step 4 (multiply by the routing weight, then add each
    token's k contributions back into its row), written as a gather over the token's own slots
    instead of index_add_; the sum is the same."""
    w = np.asarray(weights, np.float64)
    n, k = w.shape
    rows = np.asarray(out_perm, np.float64)[np.asarray(slot_pos).reshape(n, k)]   # [N, k, D]
    y = np.einsum("nk,nkd->nd", w, rows)
    if shared_out is not None:
        s = np.ones(n) if shared_scale is None else np.asarray(shared_scale, np.float64)
        y = y + s[:, None] * np.asarray(shared_out, np.float64)
    return y


def shared_expert(x, shared_gate_up, shared_down, w_shared_gate=None):
    """(scale[N], out[N,D]): the always-on shared SwiGLU expert and its gate sigmoid(w_s . x)
    ([MoE-ch27] "The shared expert", its equation and SparseMoeBlock). Without w_s the scale is 1
    (an ungated shared expert, the DeepSeekMoE form named in [VL-post])."""
    x = np.asarray(x, np.float64)
    out = swiglu(x, shared_gate_up, shared_down)
    if w_shared_gate is None:
        return np.ones(x.shape[0]), out
    return sigmoid(x @ np.asarray(w_shared_gate, np.float64)), out


# --------------------------------------------------------------------------------------------
# The whole block, in three written forms that must agree.
# --------------------------------------------------------------------------------------------

def forward_grouped(x, w_router, gate_up, down, k, norm_topk_prob=True,
                    shared_gate_up=None, shared_down=None, w_shared_gate=None, routing=None):
    """The block as [MoE-ch27] SparseMoeBlock.forward with grouped dispatch: route, sort by expert,
    run each expert on its slice, weight, unpermute, then add the gated shared expert.

    ``routing=(weights, experts)`` replaces the router's choice (used to force the oracle's choice
    on the GPU path where a near tie makes the selection a matter of rounding).
    Returns (y[N,D] float64, dict of intermediates)."""
    x = np.asarray(x, np.float64)
    E = np.asarray(w_router).shape[0]
    if routing is None:
        logits, probs, weights, experts = route(x, w_router, k, norm_topk_prob)
    else:
        weights, experts = routing
        logits = probs = None
    counts, offsets, order, token_of, slot_pos = permute(experts, E)
    out_perm = grouped_expert_ffn(x[token_of], offsets, gate_up, down)
    y = combine(out_perm, weights, slot_pos)
    scale = None
    if shared_gate_up is not None:
        scale, s = shared_expert(x, shared_gate_up, shared_down, w_shared_gate)
        y = y + scale[:, None] * s
    return y, dict(logits=logits, probs=probs, weights=weights, experts=experts, counts=counts,
                   offsets=offsets, token_of=token_of, slot_pos=slot_pos, shared_scale=scale)


def forward_loop(x, w_router, gate_up, down, k, norm_topk_prob=True,
                 shared_gate_up=None, shared_down=None, w_shared_gate=None):
    """Loop dispatch ([MoE-ch27] "Dispatch", forward_loop; [VL-MoE-src] training branch): for each
    expert that received tokens, gather them, run it, scatter-add the weighted result."""
    x = np.asarray(x, np.float64)
    _, _, weights, experts = route(x, w_router, k, norm_topk_prob)
    y = np.zeros_like(x)
    for e in np.unique(experts):
        token, slot = np.nonzero(experts == e)
        contrib = swiglu(x[token], gate_up[e], down[e]) * np.asarray(weights, np.float64)[token, slot, None]
        np.add.at(y, token, contrib)
    if shared_gate_up is not None:
        scale, s = shared_expert(x, shared_gate_up, shared_down, w_shared_gate)
        y = y + scale[:, None] * s
    return y


def forward_dense_masked(x, w_router, gate_up, down, k, norm_topk_prob=True,
                         shared_gate_up=None, shared_down=None, w_shared_gate=None):
    """Dense evaluation ([VL-MoE-src] inference branch): every expert on every token, multiplied by a
    dense [N, E] routing matrix that is zero outside each token's top-k (the scatter_ step), summed
    over experts. E/k times the necessary work: tiny inputs only."""
    x = np.asarray(x, np.float64)
    E = np.asarray(w_router).shape[0]
    _, _, weights, experts = route(x, w_router, k, norm_topk_prob)
    dense = np.zeros((x.shape[0], E), np.float64)
    np.put_along_axis(dense, experts, np.asarray(weights, np.float64), axis=1)
    all_out = np.stack([swiglu(x, gate_up[e], down[e]) for e in range(E)])   # [E, N, D]
    y = np.einsum("ne,end->nd", dense, all_out)
    if shared_gate_up is not None:
        scale, s = shared_expert(x, shared_gate_up, shared_down, w_shared_gate)
        y = y + scale[:, None] * s
    return y


# --------------------------------------------------------------------------------------------
# Accounting used by the benchmark.
# --------------------------------------------------------------------------------------------

def moe_parameter_split(hidden, layers, experts, top_k, intermediate, shared_intermediate=0):
    """(stored, active-per-token) expert parameters of the MLP part ([MoE-ch27] closing section,
    moe_parameter_split): per expert 3*h*I; each layer also holds the router's E*h and a shared
    expert's 3*h*I_s."""
    per_expert = 3 * hidden * intermediate
    shared = 3 * hidden * shared_intermediate
    router = experts * hidden
    return (layers * (experts * per_expert + shared + router),
            layers * (top_k * per_expert + shared + router))


def expected_touched_experts(n_experts, top_k, batch):
    """E * (1 - (1 - k/E)^B): distinct experts a batch of B tokens touches when each picks k of E
    roughly uniformly ([MoE-ch27] "The economics of MoE inference")."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** batch)


def switch_aux_loss(probs, experts, n_experts):
    """Switch-Transformer balance statistic E * sum_e f_e * P_e, f_e = fraction of the N*k assignments
    routed to e, P_e = mean router probability of e ([VL-post] "How the router and experts learn" (the auxiliary balance loss item), reading
    its N as the number of experts; [MoE-ch27] "Dispatch", closing paragraph). The caller applies
    the coefficient alpha."""
    probs = np.asarray(probs, np.float64)
    counts = np.bincount(np.asarray(experts).reshape(-1), minlength=n_experts)
    f = counts / counts.sum()
    P = probs.mean(axis=0)
    return float(n_experts * np.sum(f * P)), f, P


# --------------------------------------------------------------------------------------------
# Routing variants: [VL-post] "How the router and experts learn" (the capacity-limit and loss-free balancing items); [MoE-ch27] "The
# router", the note on other routers (a sigmoid score per expert with a learned bias).
# --------------------------------------------------------------------------------------------

def route_sigmoid_bias(x, w_router, k, bias=None, norm_topk_prob=True):
    """Sigmoid-score router. scores = sigmoid(logits) in float32; the k experts with the largest
    scores + bias are picked (descending, equal keys to the lower index); the bias only picks and
    never enters the weights ([VL-post] "How the router and experts learn", loss-free balancing item), so the weights are the picked
    scores, divided by their sum when norm_topk_prob (the same flag as the softmax router).
    Returns (logits f64, scores f32, keys f32, weights, experts)."""
    logits = router_logits(x, w_router)
    lg = logits.astype(np.float32)
    one = np.float32(1.0)
    scores = (one / (one + np.exp(-lg))).astype(np.float32)
    b = np.zeros(scores.shape[-1], np.float32) if bias is None else np.asarray(bias, np.float32)
    keys = (scores + b).astype(np.float32)
    experts = np.argsort(-keys, axis=-1, kind="stable")[..., :k].astype(np.int64)
    weights = np.take_along_axis(scores, experts, axis=-1)
    if norm_topk_prob:
        weights = weights / weights.sum(axis=-1, keepdims=True)
    return logits, scores, keys, weights, experts


def capacity_keep(experts, n_experts, capacity):
    """Capacity limit ([VL-post] "How the router and experts learn", capacity-limit item): every expert has `capacity` slots per batch;
    the assignments a = n*k + j claim them in assignment order and those that overflow are dropped
    (their token passes through the block unchanged: the dropped pair contributes nothing).
    Returns keep[N, k] (bool). A plain loop over the assignments."""
    experts = np.asarray(experts)
    flat = experts.reshape(-1)
    keep = np.zeros(flat.size, bool)
    used = np.zeros(n_experts, np.int64)
    for a, e in enumerate(flat):
        if used[e] < capacity:
            keep[a] = True
            used[e] += 1
    return keep.reshape(experts.shape)


def forward_capacity(x, weights, experts, gate_up, down, keep):
    """y[n] = sum_j keep[n,j] * w[n,j] * expert_{e[n,j]}(x[n]) for a given routing and keep mask
    ([MoE-ch27] "The router" equation with [VL-post] "How the router and experts learn" (capacity-limit item)), expert by expert."""
    x = np.asarray(x, np.float64)
    w = np.asarray(weights, np.float64)
    experts = np.asarray(experts)
    y = np.zeros((x.shape[0], np.asarray(down[0]).shape[0]))
    for e in range(len(gate_up)):
        n_idx, j_idx = np.nonzero((experts == e) & keep)
        if n_idx.size:          # a token picks an expert at most once, so n_idx has no repeats
            y[n_idx] += w[n_idx, j_idx, None] * swiglu(x[n_idx], gate_up[e], down[e])
    return y


def bias_update(bias, counts, n_tokens, top_k, gamma):
    """One step of the selection-bias nudge ([VL-post] "How the router and experts learn", loss-free balancing item: overloaded
    experts get their bias lowered slightly, idle ones raised): b_e - gamma * sign(c_e - N k / E),
    in float32; an expert exactly at the mean load keeps its bias."""
    counts = np.asarray(counts, np.float64)
    mean = n_tokens * top_k / counts.size
    step = np.float32(gamma) * np.sign(counts - mean).astype(np.float32)
    return (np.asarray(bias, np.float32) - step).astype(np.float32)


# --------------------------------------------------------------------------------------------
# Weight-only quantised experts: [Keras] "Lower memory" (checkpoints loaded weight-only quantised,
# int8, computing in bf16); [VL-post] "Why 3B active parameters feel like 30B" (an 8-bit copy of the
# 30B model, decode bound by the weight bytes each step reads); [MoE-ch27] "Dispatch" (experts are
# most of the bytes, 4-bit experts) and stretch exercise 3 (only the experts quantised to 4 bits,
# the router kept in bf16). The pages name the bit widths but not the quantiser, so the plainest
# one is read: symmetric absmax with one float32 scale per output row (per channel), the scheme of
# weight-only int8 in the Keras port's framework.
# --------------------------------------------------------------------------------------------

FP8_MAX = 448.0      # largest finite OCP e4m3 value, 1.75 * 2^8


def fp8_e4m3_value(codes):
    """Values of OCP e4m3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
    is subnormal, m * 2^-9; 0x7f / 0xff are NaN): the format of FP8 weights."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * val)


def fp8_e4m3_encode(v):
    """Nearest OCP e4m3 byte to each float32 value with |v| <= 448, ties to the even mantissa; the
    sign bit follows the sign of v (so -0 gives 0x80). In each binade [2^e, 2^(e+1)) the step is
    2^(e-3); below 2^-6 the subnormal step 2^-9 applies."""
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    assert np.all(a <= FP8_MAX), "encode expects values clamped to the finite range"
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3)
    r = np.rint(a / step) * step                       # exact: a / step is a scaled float
    # r may have rounded up into the next binade (its encoding is then that binade's m = 0)
    er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, er + 7, 0).astype(np.int64)
    mant = np.where(normal, r / 2.0 ** er * 8 - 8, r / 2.0 ** -9).astype(np.int64)
    return ((np.signbit(v).astype(np.int64) << 7) | (exp_field << 3) | mant).astype(np.uint8)


INT4_GROUP = 32          # input columns per int4 group
INT4_MULT_MAX = 32       # largest group multiplier: |code * mult| <= 7 * 32 = 224


def quantize_weights(w, bits):
    """Quantise a [G, R, K] stack (R output rows, K inputs) to signed `bits`-bit codes (8 or 4), or
    to OCP e4m3 bytes for bits == "f8" (see quantize_fp8). Returns (codes int8 [G, R, K], scales
    float32 [G, R], mults): mults is None except for int4 (see quantize_int4_groups).

    int8, for each row r:
      m     = max |w[r, :]|                          (float32, exact for bf16 values)
      scale = m / 127                                (float32 division)
      code  = clamp(rint(w / scale), -127, 127)      (float32 quotient, ties to even; 0 if scale 0)
    so code * scale reconstructs w to within scale / 2."""
    if bits == "f8":
        return (*quantize_fp8(w), None)
    if bits == 4:
        return quantize_int4_groups(w)
    Q = np.float32(2 ** (bits - 1) - 1)
    w32 = np.asarray(w, np.float32)
    m = np.abs(w32).max(axis=-1)
    scales = (m / Q).astype(np.float32)
    nz = scales > 0
    div = np.where(nz, scales, np.float32(1.0))[..., None]
    codes = np.clip(np.rint((w32 / div).astype(np.float32)), -Q, Q)
    codes = np.where(nz[..., None], codes, np.float32(0.0))
    return codes.astype(np.int8), scales, None


def quantize_int4_groups(w):
    """int4 with a scale per group of INT4_GROUP input columns, written as the row's float32 scale
    times a small integer per group ([MoE-ch27] "Stretch exercises", item 3: experts in 4 bits; the
    pages fix no quantiser). For each row r and group q (columns 32 q .. 32 q + 31), in float32:
      s     = max |w[r, :]| / 224                     (224 = 7 * INT4_MULT_MAX)
      mult  = min(ceil(max |w[r, group q]| / (7 * s)), 32)   (0 for an all-zero group)
      step  = s * mult
      code  = clamp(rint(w / step), -7, 7)            (ties to even; 0 where step is 0)
    The weight is code * mult * s: code * mult is an integer of magnitude at most 224, exact in
    bfloat16, so the codes times their group multiplier enter a bf16 product exactly and the row
    scale s still factors out of the row's sum. A group's step is the smallest multiple of s that
    covers its largest |w| in 7 steps. Returns (codes int8 [G, R, K], s float32 [G, R],
    mult uint8 [G, R, K / 32]); K must be a multiple of 32."""
    w32 = np.asarray(w, np.float32)
    K = w32.shape[-1]
    assert K % INT4_GROUP == 0, "int4 groups need K % 32 == 0"
    s = (np.abs(w32).max(axis=-1) / np.float32(7 * INT4_MULT_MAX)).astype(np.float32)
    grp = w32.reshape(*w32.shape[:-1], K // INT4_GROUP, INT4_GROUP)
    gmax = np.abs(grp).max(axis=-1)
    unit = (np.float32(7) * s).astype(np.float32)[..., None]          # 7 s, the span of one multiplier
    safe = np.where(unit > 0, unit, np.float32(1.0))
    mult = np.where(unit > 0, np.ceil((gmax / safe).astype(np.float32)), np.float32(0.0))
    mult = np.minimum(mult, np.float32(INT4_MULT_MAX))
    step = (s[..., None] * mult).astype(np.float32)[..., None]
    div = np.where(step > 0, step, np.float32(1.0))
    codes = np.clip(np.rint((grp / div).astype(np.float32)), -7, 7)
    codes = np.where(step > 0, codes, np.float32(0.0)).reshape(w32.shape)
    return codes.astype(np.int8), s, mult.astype(np.uint8)


def quantize_fp8(w):
    """FP8 weights ([VL-post] "Why 3B active parameters feel like 30B": an FP8 copy of the model;
    read as OCP e4m3 with one float32 scale per output row, like the integer codes):
      m = max |w[r, :]|, scale = m / 448 (float32 division),
      code = e4m3(clamp(w / scale, -448, 448)) (float32 quotient, nearest, ties to even);
    an all-zero row has scale 0 and codes 0. Returns (codes uint8 [G, R, K], scales float32 [G, R])."""
    w32 = np.asarray(w, np.float32)
    m = np.abs(w32).max(axis=-1)
    scales = (m / np.float32(FP8_MAX)).astype(np.float32)
    nz = scales > 0
    div = np.where(nz, scales, np.float32(1.0))[..., None]
    q = np.clip((w32 / div).astype(np.float32), np.float32(-FP8_MAX), np.float32(FP8_MAX))
    codes = fp8_e4m3_encode(q)
    return np.where(nz[..., None], codes, np.uint8(0)), scales


def dequantize_weights(codes, scales, mults=None):
    """The weights the quantised layer computes with: w'[g, r, c] = code[g, r, c] * scale[g, r], in
    float64 (exact: a small integer, or an e4m3 value for uint8 FP8 codes, times a float32); with
    int4 group multipliers, code * mult[g, r, c // 32] * scale[g, r]."""
    codes = np.asarray(codes)
    vals = fp8_e4m3_value(codes) if codes.dtype == np.uint8 else codes.astype(np.float64)
    if mults is not None:
        vals = vals * np.repeat(np.asarray(mults, np.float64), INT4_GROUP, axis=-1)
    return vals * np.asarray(scales, np.float64)[..., None]


# --------------------------------------------------------------------------------------------
# Backward pass of the block ([VL-post] "What a mixture-of-experts layer is": the router and the
# experts are trained end to end through the gated sum). Gradients of L = sum(dy * y) with respect
# to x, W_r, the expert weights and the shared expert, by the chain rule through the forward
# definition; the top-k choice is piecewise constant, so unselected probabilities get no gradient.
# Probabilities are float64 here (the derivative of the exact softmax).
# --------------------------------------------------------------------------------------------

def swiglu_backward(v, gate_up, down, dout):
    """For out = (silu(v G^T) * (v U^T)) Dn^T on rows v[m, D] and an output gradient dout[m, D]:
    returns (dv, dgate_up [2I, D], ddown [D, I], out). silu'(a) = s (1 + a (1 - s)), s = sigmoid(a)."""
    v = np.asarray(v, np.float64)
    gu = np.asarray(gate_up, np.float64)
    dn = np.asarray(down, np.float64)
    inter = dn.shape[1]
    a = v @ gu[:inter].T
    b = v @ gu[inter:].T
    s = sigmoid(a)
    h = a * s * b
    dout = np.asarray(dout, np.float64)
    ddown = dout.T @ h
    dh = dout @ dn
    da = dh * b * (s * (1.0 + a * (1.0 - s)))
    db = dh * a * s
    dgate_up = np.concatenate([da.T @ v, db.T @ v], axis=0)
    dv = da @ gu[:inter] + db @ gu[inter:]
    return dv, dgate_up, ddown, h @ dn.T


def backward(x, w_router, gate_up, down, k, dy, norm_topk_prob=True,
             shared_gate_up=None, shared_down=None, w_shared_gate=None):
    """Gradients of L = sum(dy * y) for the block y = sum_j w_j expert_{e_j}(x) [+ g(x) shared(x)].

    Router: logits = x W_r^T, p = softmax (float64), the top-k by p; w = p_sel / S with S = sum of
    p_sel when norm_topk_prob, so dL/dp_sel_k = (dw_k - sum_j dw_j w_j) / S (else dw_k), with
    dw_j = dy . expert_{e_j}(x); then dlogits = p * (dp - sum_e dp_e p_e).
    Experts: for each expert, the rows routed to it with output gradient w_j dy (swiglu_backward).
    Shared expert: g = sigmoid(w_s . x) (1 if no w_s): ds = g dy, dg = dy . shared(x).
    Returns dict(dx, dw_router, dgate_up, ddown [, dshared_gate_up, dshared_down, dw_shared_gate],
    weights, experts, dweights)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    wr = np.asarray(w_router, np.float64)
    logits, probs, weights, experts = route(x, wr, k, norm_topk_prob, prob_dtype=np.float64)
    N, D = x.shape
    E = wr.shape[0]
    dx = np.zeros_like(x)
    dgu = np.zeros((E,) + np.asarray(gate_up[0]).shape)
    ddn = np.zeros((E,) + np.asarray(down[0]).shape)
    dw = np.zeros(weights.shape)
    for e in range(E):
        n_idx, j_idx = np.nonzero(experts == e)
        if n_idx.size == 0:
            continue
        # a token picks an expert at most once, so n_idx has no repeats
        w_e = weights[n_idx, j_idx][:, None]
        dv, dgu[e], ddn[e], out = swiglu_backward(x[n_idx], gate_up[e], down[e], w_e * dy[n_idx])
        dw[n_idx, j_idx] = np.sum(dy[n_idx] * out, axis=1)
        dx[n_idx] += dv
    psel = np.take_along_axis(probs, experts, axis=-1)
    if norm_topk_prob:
        S = psel.sum(axis=-1, keepdims=True)
        dpsel = (dw - np.sum(dw * weights, axis=-1, keepdims=True)) / S
    else:
        dpsel = dw
    dp = np.zeros_like(probs)
    np.put_along_axis(dp, experts, dpsel, axis=-1)
    dlogits = probs * (dp - np.sum(dp * probs, axis=-1, keepdims=True))
    out = dict(dw_router=dlogits.T @ x, dgate_up=dgu, ddown=ddn, weights=weights, experts=experts,
               dweights=dw, dlogits=dlogits)
    dx += dlogits @ wr
    if shared_gate_up is not None:
        if w_shared_gate is not None:
            ws_ = np.asarray(w_shared_gate, np.float64)
            g = sigmoid(x @ ws_)
        else:
            g = np.ones(N)
        dv, out["dshared_gate_up"], out["dshared_down"], s = swiglu_backward(x, shared_gate_up, shared_down,
                                                                             g[:, None] * dy)
        dx += dv
        if w_shared_gate is not None:
            dz = np.sum(dy * s, axis=1) * g * (1.0 - g)
            out["dw_shared_gate"] = dz @ x
            dx += dz[:, None] * ws_[None, :]
    out["dx"] = dx
    return out
