"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Every workload, the full-size ones included, compares routing, the permutation and the layer
output on every token. Tokens whose oracle k-th/(k+1)-th probability gap is below 1e-6 may be
routed either way; where the GPU chose differently, their output is checked through the oracle's
forced choice (permute -> expert FFN -> combine on the oracle's routing).
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import inputs as I
from parity_util import (GAP, check_f16s_exponents, check_permute_invariants, compare_routing, decode_f16s,
                         encode_f16s, f16s_row_bytes, oracle_layer, rel_err, rms, to_np, y_tolerance)

pytestmark = pytest.mark.gpu

ODD = {
    # non-default, non-power-of-two shapes: ragged token tiles, E not a multiple of 32, tails in K and N
    "odd": I.custom_shape("odd", 37, 40, 7, 3, 24, dtype=I.BF16, seed=11),
    "odd_shared": I.custom_shape("odd_shared", 45, 72, 13, 4, 40, shared_inter=24, seed=12),
    "odd_ungated": I.custom_shape("odd_ungated", 33, 64, 5, 2, 16, shared_inter=8, seed=13, shared_gated=False),
    "odd_f32": I.custom_shape("odd_f32", 29, 36, 6, 2, 20, dtype=I.F32, seed=14),
    "k1": I.custom_shape("k1", 70, 64, 9, 1, 32, seed=15),
    "k_eq_e": I.custom_shape("k_eq_e", 50, 48, 6, 6, 16, seed=16),
    "one_token": I.custom_shape("one_token", 1, 128, 16, 4, 64, seed=17),
    "e1": I.custom_shape("e1", 20, 32, 1, 1, 8, seed=18),
    "many_empty": I.custom_shape("many_empty", 5, 256, 300, 2, 128, seed=19),
    "no_renorm": I.custom_shape("no_renorm", 66, 96, 12, 3, 48, norm_topk_prob=False, seed=20),
    "tiles": I.custom_shape("tiles", 600, 264, 4, 2, 200, seed=21),       # > 256 rows per expert
    "e512": I.custom_shape("e512", 130, 64, 512, 10, 16, shared_inter=16, seed=22),
    # long batch (x-stationary router) with a ragged last token tile and two 128-expert blocks
    "xs_e200": I.custom_shape("xs_e200", 8200, 512, 200, 6, 128, seed=23),
}
SMALL = ["tiny"] + list(ODD)
FULL = ["keras", "decode", "prefill", "fanout"]


def shape_of(name):
    return I.WORKLOADS.get(name) or ODD[name]


@functools.lru_cache(maxsize=2)
def data_of(name):
    d = I.make_inputs(shape_of(name))
    return d, B.to_device(d.store)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_route(name, want_logits=True, with_ws=False):
    d, dev = data_of(name)
    s = d.shape
    cfg = B.config_for(s)
    N, k, E = s.n_tokens, s.top_k, s.n_experts
    w = torch.empty((N, k), dtype=torch.float32, device="cuda")
    e = torch.empty((N, k), dtype=torch.int32, device="cuda")
    lg = torch.empty((N, E), dtype=torch.float32, device="cuda") if want_logits else None
    ss = torch.empty((N,), dtype=torch.float32, device="cuda") if "w_shared_gate" in dev else None
    ws = B.alloc_workspace(cfg) if with_ws else None
    B.moe_route(cfg, dev["x"], dev["w_router"], dev.get("w_shared_gate"), lg, w, e, ss, ws)
    torch.cuda.synchronize()
    return w, e, lg, ss


@pytest.mark.parametrize("with_ws", [False, True], ids=["one_pass", "split_k"])
@pytest.mark.parametrize("name", SMALL + FULL)
def test_route(name, with_ws):
    say(f"[route] {name} ws={with_ws}")
    d, dev = data_of(name)
    s = d.shape
    w, e, lg, ss = run_route(name, with_ws=with_ws)
    logits, probs, w_ref, e_ref = O.route(d.values("x"), d.values("w_router"), s.top_k, s.norm_topk_prob)
    lerr = np.abs(to_np(lg) - logits).max()
    assert lerr <= 5e-5 * max(1.0, np.abs(logits).max()), f"logit error {lerr}"
    same, near = compare_routing(to_np(w).astype(np.float64), to_np(e), w_ref, e_ref, probs, s.top_k)
    say(f"  tokens {s.n_tokens}, near ties {near}, logit err {lerr:.2e}")
    if ss is not None:
        sc, _ = O.shared_expert(d.values("x")[:4], d.values("shared_gate_up"), d.values("shared_down"),
                                d.values("w_shared_gate"))
        z = d.values("x") @ d.values("w_shared_gate")
        np.testing.assert_allclose(to_np(ss), 1.0 / (1.0 + np.exp(-z)), atol=1e-6)
        np.testing.assert_allclose(to_np(ss)[:4], sc, atol=1e-6)


def test_route_exact_ties_go_to_lower_index():
    say("[route] ties")
    s = I.custom_shape("ties", 200, 64, 9, 4, 16, seed=30)
    d = I.make_inputs(s)
    wr = d.store["w_router"]
    wr[5] = wr[1]
    wr[7] = wr[1]
    wr[8] = wr[2]
    dev = B.to_device(d.store)
    cfg = B.config_for(s)
    w = torch.empty((200, 4), dtype=torch.float32, device="cuda")
    e = torch.empty((200, 4), dtype=torch.int32, device="cuda")
    lg = torch.empty((200, 9), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, dev["x"], dev["w_router"], None, lg, w, e, None)
    torch.cuda.synchronize()
    lg, e = to_np(lg), to_np(e)
    assert np.array_equal(lg[:, 1], lg[:, 5]) and np.array_equal(lg[:, 1], lg[:, 7])
    hits = 0
    for n in range(200):
        p = lg[n]
        ref = sorted(range(9), key=lambda j: (-p[j], j))[:4]      # equal logits -> equal probabilities
        assert e[n].tolist() == ref
        hits += 1 in ref and 5 in ref
    assert hits > 0


def _random_experts(N, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)]).astype(np.int32)


def run_permute(cfg, experts_np, x=None):
    N, k = experts_np.shape
    E = cfg.n_experts
    ex = torch.from_numpy(experts_np).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    token_of = torch.empty(max(N * k, 1), dtype=torch.int32, device="cuda")
    slot_pos = torch.empty(max(N * k, 1), dtype=torch.int32, device="cuda")
    x_perm = None if x is None else torch.empty((N * k, cfg.hidden), dtype=x.dtype, device="cuda")
    ws = B.alloc_workspace(cfg)
    B.moe_permute(cfg, ex, x, counts, offsets, token_of, slot_pos, x_perm, ws)
    torch.cuda.synchronize()
    return counts, offsets, token_of, slot_pos, x_perm


# one-workgroup grouping (A <= 8192), chunked grouping with a ragged last chunk, and more chunks than
# the scan holds in registers (17,000 x 8 = 136,000 assignments: 133 chunks of 1,024)
@pytest.mark.parametrize("N,k,E,seed", [(1, 1, 1, 0), (37, 3, 7, 1), (5000, 8, 128, 2), (2049, 10, 512, 3),
                                        (4096, 2, 8, 4), (300, 6, 300, 5), (64, 8, 128, 6), (17000, 8, 128, 9)])
def test_permute_bit_exact(N, k, E, seed):
    say(f"[permute] N={N} k={k} E={E}")
    cfg = B.make_config(N, 64, E, k, 64)
    experts = _random_experts(N, k, E, seed)
    x = torch.randn(N, 64, device="cuda").to(torch.bfloat16)
    counts, offsets, token_of, slot_pos, x_perm = run_permute(cfg, experts, x)
    check_permute_invariants(experts, to_np(counts), to_np(offsets), to_np(token_of), to_np(slot_pos), E, k)
    c_ref, o_ref, _, t_ref, s_ref = O.permute(experts, E)
    assert np.array_equal(to_np(counts), c_ref)
    assert np.array_equal(to_np(offsets), o_ref)
    assert np.array_equal(to_np(token_of), t_ref)
    assert np.array_equal(to_np(slot_pos), s_ref)
    assert torch.equal(x_perm.view(torch.int16), x[torch.from_numpy(t_ref).cuda()].view(torch.int16))


@pytest.mark.parametrize("N,k,E,seed", [(50, 3, 9, 7), (3000, 4, 64, 8)])     # one-workgroup and chunked kernels
def test_permute_out_of_range_ids_are_dropped(N, k, E, seed):
    """Ids outside [0, E) from a caller are dropped pairs: the expected grouping is the oracle's on
    the ids with every bad one sent to an extra expert E past the end (its rows then cut off)."""
    say(f"[permute] bad ids N={N} k={k} E={E}")
    cfg = B.make_config(N, 64, E, k, 64)
    experts = _random_experts(N, k, E, seed)
    rng = np.random.default_rng(seed)
    bad = rng.random(experts.shape) < 0.1
    experts[bad] = rng.choice([-1, -7, E, E + 3, 2 ** 31 - 1, -2 ** 31], size=int(bad.sum()))
    counts, offsets, token_of, slot_pos, _ = run_permute(cfg, experts)
    check_permute_invariants(experts, to_np(counts), to_np(offsets), to_np(token_of), to_np(slot_pos), E, k)
    ex = np.where(bad, E, experts)
    c_ref, o_ref, _, t_ref, s_ref = O.permute(ex, E + 1)
    kept = int(o_ref[E])
    s_ref = np.where(bad.reshape(-1), -1, s_ref)
    assert np.array_equal(to_np(counts), c_ref[:E])
    assert np.array_equal(to_np(offsets), o_ref[:E + 1])
    assert np.array_equal(to_np(token_of)[:kept], t_ref[:kept])
    assert np.array_equal(to_np(slot_pos), s_ref)


def test_permute_skewed_and_zero_tokens():
    say("[permute] skew, N=0")
    # everything on one expert (the c4 head), and the N = 0 no-op that still defines counts/offsets
    cfg = B.make_config(3000, 64, 64, 1, 64)
    experts = np.full((3000, 1), 17, np.int32)
    counts, offsets, token_of, slot_pos, _ = run_permute(cfg, experts)
    assert to_np(counts)[17] == 3000 and to_np(counts).sum() == 3000
    assert np.array_equal(to_np(token_of), np.arange(3000))
    cfg0 = B.make_config(0, 64, 9, 2, 64)
    counts, offsets, _, _, _ = run_permute(cfg0, np.zeros((0, 2), np.int32))
    assert not to_np(counts).any() and not to_np(offsets).any()


def _ffn_case(s, seed, rows_per_group):
    rng = np.random.default_rng(seed)
    G = len(rows_per_group)
    offsets = np.zeros(G + 1, np.int64)
    offsets[1:] = np.cumsum(rows_per_group)
    R = int(offsets[-1])
    d = I.make_inputs(I.custom_shape("ffn", max(R, 1), s.hidden, G, 1, s.inter, dtype=s.dtype, seed=seed))
    return d, offsets, R, rng


@pytest.mark.parametrize("dtype,D,I_,rows", [
    ("bf16", 2048, 768, [300, 0, 5, 257, 1, 64, 513]),
    ("bf16", 40, 24, [3, 0, 40, 1]),
    ("bf16", 264, 200, [7, 256, 1]),
    ("bf16", 128, 1408, [2, 4, 3, 1]),
    ("f32", 36, 20, [9, 0, 70]),
    ("f32", 128, 64, [16, 16, 40, 0, 56]),
])
def test_expert_ffn(dtype, D, I_, rows):
    say(f"[ffn] {dtype} D={D} I={I_} rows={rows}")
    s = I.custom_shape("ffn", 1, D, 1, 1, I_, dtype=dtype)
    d, offsets, R, rng = _ffn_case(s, 40 + D, rows)
    dev = B.to_device(d.store)
    cfg = B.make_config(R, D, len(rows), 1, I_, dtype=dtype)
    tdt = B.torch_dtype(cfg.dtype)
    h = torch.empty((R, I_), dtype=tdt, device="cuda")
    out = torch.full((R, D), float("nan"), dtype=torch.float32, device="cuda")
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    # rows gathered through row_index from a shuffled copy of x, to exercise the gather
    perm = rng.permutation(R)
    x_sh = torch.empty_like(dev["x"][:R])
    x_sh[torch.from_numpy(perm).cuda()] = dev["x"][:R]
    ridx = torch.from_numpy(perm.astype(np.int32)).cuda()
    B.moe_expert_ffn(cfg, len(rows), I_, R, x_sh, ridx, off, dev["gate_up"], dev["down"], h, out)
    torch.cuda.synchronize()
    ref = O.grouped_expert_ffn(d.values("x")[:R], offsets, d.expert_view("gate_up"), d.expert_view("down"))
    got = to_np(out)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= tol, rel_err(got, ref)
    # h against the oracle's SwiGLU product (bf16: one rounding of a float32 value)
    xv = d.values("x")[:R]
    for g in range(len(rows)):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            gu = d.expert_view("gate_up")[g]
            z = xv[a:b] @ gu[:I_].T
            href = O.silu(z) * (xv[a:b] @ gu[I_:].T)
            hb = to_np(h)[a:b]
            lim = (2.0 ** -8 if dtype == "bf16" else 1e-5) * np.abs(href) + 1e-5 * max(1e-3, np.abs(href).max())
            assert np.all(np.abs(hb - href) <= lim)


def test_combine():
    say("[combine]")
    rng = np.random.default_rng(5)
    N, k, E, D = 333, 5, 17, 264
    experts = _random_experts(N, k, E, 6)
    _, _, _, _, slot_pos = O.permute(experts, E)
    out_perm = rng.standard_normal((N * k, D)).astype(np.float32)
    weights = rng.random((N, k)).astype(np.float32)
    shared = rng.standard_normal((N, D)).astype(np.float32)
    scale = rng.random(N).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for out_dtype in ("f32", "bf16"):
        for sh in (False, True):
            cfg = B.make_config(N, D, E, k, 8, dtype="bf16", out_dtype=out_dtype)
            y = torch.empty((N, D), dtype=B.torch_dtype(cfg.out_dtype), device="cuda")
            B.moe_combine(cfg, t(out_perm), t(weights), t(slot_pos.astype(np.int32)), t(shared) if sh else None,
                          t(scale) if sh else None, y)
            torch.cuda.synchronize()
            ref = O.combine(out_perm, weights, slot_pos, shared if sh else None, scale if sh else None)
            got = to_np(y)
            if out_dtype == "f32":
                assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
            else:
                assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("D,I_,rows", [
    (2048, 768, [300, 0, 5, 257, 1, 64, 513]),       # streaming kernel (256 x 256 tiles)
    (128, 1408, [2, 4, 3, 1]),                       # weight-streaming kernel (few rows per group)
    (64, 24, [3, 0, 40, 1]),                         # register-staged kernel (K % 128 != 0)
    (2048, 768, [1, 2, 3, 4, 5, 6, 7, 8]),
])
def test_expert_ffn_f16s(D, I_, rows):
    """Expert outputs in the fp16 form: decoded values against the oracle, the exponent rule, and the
    bytes equal to the form's definition applied to the fp32 outputs of the same products."""
    say(f"[ffn f16s] D={D} I={I_} rows={rows}")
    s = I.custom_shape("ffn", 1, D, 1, 1, I_, dtype="bf16")
    d, offsets, R, rng = _ffn_case(s, 60 + D, rows)
    dev = B.to_device(d.store)
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    outs = {}
    for eo in (B.MOE_EXPERT_OUT_F32, B.MOE_EXPERT_OUT_F16S):
        cfg = B.make_config(R, D, len(rows), 1, I_, expert_out=eo)
        h = torch.empty((R, I_), dtype=torch.bfloat16, device="cuda")
        out = torch.full((R, D), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_expert_ffn(cfg, len(rows), I_, R, dev["x"], None, off, dev["gate_up"], dev["down"], h, out)
        torch.cuda.synchronize()
        outs[eo] = out
    raw = outs[B.MOE_EXPERT_OUT_F16S].view(torch.uint8).cpu().numpy().reshape(-1)
    vals, _ = decode_f16s(raw, R, D)
    check_f16s_exponents(raw, R, D)
    ref = O.grouped_expert_ffn(d.values("x")[:R], offsets, d.expert_view("gate_up"), d.expert_view("down"))
    assert np.isfinite(vals).all()
    assert rel_err(vals, ref) <= 2e-2, rel_err(vals, ref)
    f32 = to_np(outs[B.MOE_EXPERT_OUT_F32])
    assert np.abs(vals - f32).max() <= 2.0 ** -11 * np.abs(f32).max() * 1.0001
    want = encode_f16s(f32).reshape(R, -1)
    got = raw[:R * f16s_row_bytes(D)].reshape(R, -1)
    assert np.array_equal(got[:, :2 * D + D // 16], want[:, :2 * D + D // 16]), "bytes differ from the form's definition"


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_combine_f16s(out_dtype):
    say(f"[combine f16s] {out_dtype}")
    rng = np.random.default_rng(8)
    N, k, E, D = 333, 5, 17, 272
    experts = _random_experts(N, k, E, 6)
    _, _, _, _, slot_pos = O.permute(experts, E)
    slot_pos = slot_pos.copy()
    slot_pos[[3, 40, 41]] = -1                                  # dropped pairs are skipped
    scales = np.exp2(rng.integers(-20, 20, (N * k, 1))).astype(np.float32)
    out_perm = (rng.standard_normal((N * k, D)) * scales).astype(np.float32)
    out_perm[7, :32] = 0.0                                     # all-zero groups
    weights = rng.random((N, k)).astype(np.float32)
    shared = rng.standard_normal((N, D)).astype(np.float32)
    scale = rng.random(N).astype(np.float32)
    enc, enc_sh = encode_f16s(out_perm), encode_f16s(shared)
    ov, _ = decode_f16s(enc, N * k, D)
    sv, _ = decode_f16s(enc_sh, N, D)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for sh in (False, True):
        cfg = B.make_config(N, D, E, k, 8, dtype="bf16", out_dtype=out_dtype, expert_out=B.MOE_EXPERT_OUT_F16S)
        y = torch.empty((N, D), dtype=B.torch_dtype(cfg.out_dtype), device="cuda")
        B.moe_combine(cfg, t(enc), t(weights), t(slot_pos.astype(np.int32)), t(enc_sh) if sh else None,
                      t(scale) if sh else None, y)
        torch.cuda.synchronize()
        kept = (slot_pos >= 0).reshape(N, k)          # the oracle's combine has no dropped pairs:
        ref = O.combine(ov, np.where(kept, weights, 0.0), np.where(slot_pos >= 0, slot_pos, 0),   # weight 0
                        sv if sh else None, scale if sh else None)
        got = to_np(y)
        rowmax = np.abs(ref).max(axis=1, keepdims=True) + 1e-30
        if out_dtype == "f32":
            assert np.all(np.abs(got - ref) <= 1e-5 * rowmax)
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * rowmax)


def sample_tokens(N, near_idx, n_sample, seed=0):
    rng = np.random.default_rng(seed)
    base = rng.choice(N, size=min(n_sample, N), replace=False) if N > n_sample else np.arange(N)
    return np.unique(np.concatenate([base, near_idx]).astype(np.int64))


@functools.lru_cache(maxsize=1)
def oracle_of(name):
    """Oracle routing and layer output of every token (float64), computed once per workload."""
    d, _ = data_of(name)
    s = d.shape
    _, probs, w_ref, e_ref = O.route(d.values("x"), d.values("w_router"), s.top_k, s.norm_topk_prob)
    y_ref, _ = oracle_layer(d)
    return probs, w_ref, e_ref, y_ref


def forward_and_check(name, out_dtype, expert_out=B.MOE_EXPERT_OUT_F32):
    d, dev = data_of(name)
    s = d.shape
    cfg = B.config_for(s, out_dtype, expert_out=expert_out)
    N, k = s.n_tokens, s.top_k
    w = torch.empty((N, k), dtype=torch.float32, device="cuda")
    e = torch.empty((N, k), dtype=torch.int32, device="cuda")
    ws = B.alloc_workspace(cfg)
    y = B.forward(cfg, dev, ws=ws, weights=w, experts=e)
    torch.cuda.synchronize()
    got = to_np(y)
    assert np.isfinite(got).all()
    probs, w_ref, e_ref, y_ref = oracle_of(name)
    same, near = compare_routing(to_np(w).astype(np.float64), to_np(e), w_ref, e_ref, probs, k)
    near_idx = np.nonzero(O.k_gap(probs, k) < GAP)[0]
    tol = y_tolerance(s.dtype, out_dtype, y_ref)        # near-tie tokens the GPU routed differently are
    err = rel_err(got[same], y_ref[same])               # checked through the forced choice
    rms_err = rms(got[same] - y_ref[same]) / rms(y_ref)
    say(f"  {name} out={out_dtype}{' f16s' if expert_out else ''}: tokens checked {same.sum()}/{N}, near ties {near}, "
        f"max|dy|/rms = {err:.3e} (tol {tol:.3e}), rms(dy)/rms = {rms_err:.3e}")
    assert err <= tol
    return d, dev, cfg, y, near_idx, probs, w_ref, e_ref


def forced_choice_check(d, dev, cfg, near_idx, w_ref, e_ref):
    """Run permute -> ffn -> combine on the oracle's routing and compare the near-tie tokens (plus
    a sample of the others)."""
    s = d.shape
    N, k, E = s.n_tokens, s.top_k, s.n_experts
    A = N * k
    wt = torch.from_numpy(np.asarray(w_ref, np.float32)).cuda()
    et = torch.from_numpy(e_ref.astype(np.int32)).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    token_of = torch.empty(A, dtype=torch.int32, device="cuda")
    slot_pos = torch.empty(A, dtype=torch.int32, device="cuda")
    ws = B.alloc_workspace(cfg)
    B.moe_permute(cfg, et, None, counts, offsets, token_of, slot_pos, None, ws)
    h = torch.empty((A, s.inter), dtype=B.torch_dtype(cfg.dtype), device="cuda")
    out = torch.empty((A, s.hidden), dtype=torch.float32, device="cuda")
    B.moe_expert_ffn(cfg, E, s.inter, A, dev["x"], token_of, offsets, dev["gate_up"], dev["down"], h, out)
    sh_out = sh_scale = None
    if s.shared_inter:
        shh = torch.empty((N, s.shared_inter), dtype=B.torch_dtype(cfg.dtype), device="cuda")
        sh_out = torch.empty((N, s.hidden), dtype=torch.float32, device="cuda")
        B.moe_expert_ffn(cfg, 1, s.shared_inter, N, dev["x"], None, None, dev["shared_gate_up"],
                         dev["shared_down"], shh, sh_out)
        if "w_shared_gate" in dev:
            z = d.values("x") @ d.values("w_shared_gate")
            sh_scale = torch.from_numpy((1.0 / (1.0 + np.exp(-z))).astype(np.float32)).cuda()
    y = torch.empty((N, s.hidden), dtype=B.torch_dtype(cfg.out_dtype), device="cuda")
    B.moe_combine(cfg, out, wt, slot_pos, sh_out, sh_scale, y)
    torch.cuda.synchronize()
    check_permute_invariants(e_ref, to_np(counts), to_np(offsets), to_np(token_of), to_np(slot_pos), E, k)
    toks = sample_tokens(N, near_idx, 64, seed=1)
    y_ref, _ = oracle_layer(d, toks, routing=(np.asarray(w_ref)[toks], e_ref[toks]))
    err = rel_err(to_np(y)[toks], y_ref)
    tol = y_tolerance(s.dtype, "f32" if cfg.out_dtype == B.MOE_F32 else "bf16", y_ref)
    say(f"  forced choice on {len(near_idx)} near-tie tokens (+ sample): {err:.3e}")
    assert err <= tol


def f16s_ok(s):
    return s.dtype == I.BF16 and s.hidden % 16 == 0


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(name):
    say(f"[forward] {name}")
    s = shape_of(name)
    out = "f32"
    d, dev, cfg, y, near_idx, probs, w_ref, e_ref = forward_and_check(name, out)
    if len(near_idx):
        forced_choice_check(d, dev, cfg, near_idx, w_ref, e_ref)
    if s.dtype == I.BF16:
        forward_and_check(name, "bf16")
    if f16s_ok(s):                       # expert outputs in the fp16 form
        for o in ("f32", "bf16"):
            d, dev, cfg, y, near_idx, probs, w_ref, e_ref = forward_and_check(name, o, B.MOE_EXPERT_OUT_F16S)
            if len(near_idx):
                forced_choice_check(d, dev, cfg, near_idx, w_ref, e_ref)


@pytest.mark.parametrize("expert_out", [B.MOE_EXPERT_OUT_F32, B.MOE_EXPERT_OUT_F16S], ids=["f32out", "f16s"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", FULL)
def test_forward_full(name, out_dtype, expert_out):
    say(f"[forward] {name} {out_dtype} expert_out={expert_out}")
    d, dev, cfg, y, near_idx, probs, w_ref, e_ref = forward_and_check(name, out_dtype, expert_out)
    if len(near_idx):
        forced_choice_check(d, dev, cfg, near_idx, w_ref, e_ref)


@pytest.mark.parametrize("name,expert_out", [("odd_shared", 0), ("keras", 0), ("fanout", 0), ("fanout", 1),
                                             ("odd_ungated", 1)])
def test_forward_deterministic(name, expert_out):
    say(f"[determinism] {name} expert_out={expert_out}")
    d, dev = data_of(name)
    cfg = B.config_for(d.shape, "f32", expert_out=expert_out)
    ws = B.alloc_workspace(cfg)
    y1 = B.forward(cfg, dev, ws=ws).clone()
    ws.fill_(0x5A)
    y2 = B.forward(cfg, dev, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("name,expert_out", [("tiny", 0), ("decode", 0), ("fanout", 0), ("decode", 1), ("fanout", 1),
                                             ("prefill", 1)])
def test_decomposed_chain_equals_forward(name, expert_out):
    """The ABI chain (route -> permute -> gate_up -> down -> [shared] -> combine) gives the same bits
    as moe_forward: the benchmark times the chain so it can time the expert GEMM on its own."""
    say(f"[chain] {name} expert_out={expert_out}")
    d, dev = data_of(name)
    s = d.shape
    cfg = B.config_for(s, expert_out=expert_out)
    y_fwd = B.forward(cfg, dev)
    from mixture_experts_layer_10_amd.chain import Chain
    ch = Chain(cfg, dev)
    ch.step()
    torch.cuda.synchronize()
    assert torch.equal(ch.y.view(torch.int16 if ch.y.dtype == torch.bfloat16 else torch.int32),
                       y_fwd.view(torch.int16 if y_fwd.dtype == torch.bfloat16 else torch.int32))
