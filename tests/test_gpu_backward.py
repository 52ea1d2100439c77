"""Backward pass (moe_backward) on the GPU against the oracle's chain-rule gradients (fp64,
pinned by finite differences in test_oracle.py), on the same seeded bf16 inputs and a seeded
output gradient dy ~ N(0, 1) rounded to bf16.

Bar (derived from the arithmetic; the pages state none for gradients): the matrix-core inputs
h, w dy, da, db and dlogits are rounded to bf16 once (relative error <= 2^-9 each, two rounded
operands per product) and accumulated in fp32, so each gradient G must satisfy
    ||G - G_ref|| / ||G_ref|| <= 1e-2   (Frobenius, about 4 * 2^-9)
    max|G - G_ref| <= 2e-2 * max|G_ref|;
fp32 layers round nothing but the fp32 sums: 1e-5 and 1e-4 (the forward's fp32 bar).
The forward's max-abs / RMS measure does not suit weight gradients: an entry is a sum over the few
rows routed to one expert of products of heavy-tailed factors, so max|G| / RMS(G) reaches 20-30 and
one bf16 rounding shows as several percent of the RMS (a CPU emulation of these roundings gives the
same figures as the GPU). Tokens with a near tie in the top-k (possible either way) get a zero
output gradient, which removes every gradient term they have; the rest have a unique selection.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import inputs as I
from parity_util import GAP, rel_err
from test_gpu_parity import data_of, say

pytestmark = pytest.mark.gpu

TOLS = {I.BF16: (1e-2, 2e-2), I.F32: (1e-5, 1e-4)}     # (normwise, max / max) per layer dtype

SHAPES = {
    "small": I.custom_shape("bwd_small", 40, 256, 16, 2, 128, seed=51),
    "ragged_e12": I.custom_shape("bwd_e12", 37, 384, 12, 3, 256, seed=52),          # E padded to 16 for W_r^T
    "keras_like": I.custom_shape("bwd_keras", 512, 2048, 60, 4, 1408, seed=53),      # E = 60, wide experts
    "tall": I.custom_shape("bwd_tall", 3000, 512, 8, 2, 256, seed=54),               # long per-expert sums
    # tall groups, I = 200: dh reads Dn in its [D, I] layout with a last column tile of 200 columns
    # (a half-filled 32-byte chunk at the edge); dx (K = 2I = 400) goes through the transposed copy
    "tall_cols200": I.custom_shape("bwd_c200", 2000, 256, 8, 2, 200, seed=59),
    "norm_off": I.custom_shape("bwd_nonorm", 64, 256, 16, 4, 128, norm_topk_prob=False, seed=55),
    "shared_gated": I.custom_shape("bwd_sh", 300, 256, 32, 4, 128, shared_inter=256, seed=56),
    "shared_ungated": I.custom_shape("bwd_sh_u", 130, 384, 16, 2, 128, shared_inter=128, seed=57, shared_gated=False),
    "tiny_f32": I.WORKLOADS["tiny"],
    "odd_f32_shared": I.custom_shape("bwd_f32_sh", 45, 72, 13, 4, 40, shared_inter=24, dtype=I.F32, seed=58),
}


def bf16_dev(a):
    return torch.from_numpy(I.round_to_bf16_bits(np.asarray(a, np.float32)).view(np.int16)).cuda().view(torch.bfloat16)


def dy_dev(a, dtype):
    return bf16_dev(a) if dtype == I.BF16 else torch.from_numpy(np.asarray(a, np.float32)).cuda()


def run_and_compare(d, dev):
    s = d.shape
    dy32 = np.random.default_rng(s.seed + 7).standard_normal((s.n_tokens, s.hidden), dtype=np.float32)
    if s.dtype == I.BF16:
        dy32 = I.bf16_bits_to_f32(I.round_to_bf16_bits(dy32))
    dy_np = dy32.astype(np.float64)
    # tokens whose k-th / (k+1)-th probabilities are closer than GAP may be routed either way; with
    # a zero output gradient every gradient term of such a token vanishes, whatever its routing
    _, probs, _, _ = O.route(d.values("x"), d.values("w_router"), s.top_k, s.norm_topk_prob)
    near = O.k_gap(probs, s.top_k) < GAP
    dy_np[near] = 0.0
    say(f"  near-tie tokens with zero dy: {int(near.sum())}")
    cfg = B.config_for(s)
    g = B.backward(cfg, dev, dy_dev(dy_np, s.dtype))
    torch.cuda.synchronize()
    sh = {}
    if s.shared_inter:
        sh = dict(shared_gate_up=d.values("shared_gate_up"), shared_down=d.values("shared_down"),
                  w_shared_gate=d.values("w_shared_gate"))
    ref = O.backward(d.values("x"), d.values("w_router"), d.expert_view("gate_up"), d.expert_view("down"),
                     s.top_k, dy_np, s.norm_topk_prob, **sh)
    names = ["dx", "dw_router", "dgate_up", "ddown"] + [n for n in ("dshared_gate_up", "dshared_down", "dw_shared_gate")
                                                            if n in g]
    assert ("dw_shared_gate" in g) == ("dw_shared_gate" in ref)
    for name, key in ((n, n) for n in names):
        got = g[name].cpu().numpy().astype(np.float64)
        want = np.asarray(ref[key], np.float64).reshape(got.shape)
        assert np.isfinite(got).all(), name
        diff = got - want
        norm_err = float(np.sqrt(np.sum(diff * diff) / np.sum(want * want)))
        max_err = float(np.abs(diff).max() / np.abs(want).max())
        say(f"  {name}: normwise {norm_err:.3e}, max/max {max_err:.3e}, max/rms {rel_err(got, want):.3e}")
        norm_tol, max_tol = TOLS[s.dtype]
        assert norm_err <= norm_tol and max_err <= max_tol, name
    # experts that received no token get exactly zero gradients
    idle = np.setdiff1d(np.arange(s.n_experts), np.unique(ref["experts"][~near]))
    idle = idle[~np.isin(idle, ref["experts"][near])]
    if idle.size:
        assert not g["dgate_up"][idle].any() and not g["ddown"][idle].any()


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_vs_oracle(name):
    say(f"[backward] {name}")
    d = I.make_inputs(SHAPES[name])
    run_and_compare(d, B.to_device(d.store))


@pytest.mark.parametrize("name", ["decode", "prefill", "fanout"])
def test_backward_full_size(name):
    # prefill: 256-row GEMM tiles and a 16,263-row sum for the hottest expert's weight gradients
    say(f"[backward] {name} (full size)")
    d, dev = data_of(name)
    run_and_compare(d, dev)


def test_backward_deterministic():
    d = I.make_inputs(SHAPES["tall"])
    dev = B.to_device(d.store)
    cfg = B.config_for(d.shape)
    dy = bf16_dev(np.random.default_rng(3).standard_normal((d.shape.n_tokens, d.shape.hidden)))
    a = B.backward(cfg, dev, dy)
    b = B.backward(cfg, dev, dy)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k


@pytest.mark.parametrize("name", ["small", "shared_gated"])
def test_backward_ignores_expert_output_form(name):
    """The backward keeps its own fp32 intermediates: a config whose forward keeps expert outputs in
    the fp16 form gives bitwise the gradients of the fp32 form (the combine of the dx rows reads
    fp32 rows either way)."""
    say(f"[backward] {name}, fp16-form config")
    d = I.make_inputs(SHAPES[name])
    dev = B.to_device(d.store)
    cfg = B.config_for(d.shape)
    dy = bf16_dev(np.random.default_rng(4).standard_normal((d.shape.n_tokens, d.shape.hidden)))
    a = B.backward(cfg, dev, dy)
    b = B.backward(cfg.copy(expert_out=B.MOE_EXPERT_OUT_F16S), dev, dy)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k
