"""Router load statistics and the balance loss (moe_router_stats) on the GPU, against the oracle's
switch_aux_loss ("Qwen3-VL + MoE: train to deploy", section "How the router and experts learn", the item on an auxiliary balance loss) and its
closed forms."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import inputs as I
from parity_util import to_np
from test_gpu_parity import ODD, data_of, say

pytestmark = pytest.mark.gpu


def run_stats(cfg, logits, counts):
    E = cfg.n_experts
    f = torch.full((E,), float("nan"), dtype=torch.float32, device="cuda")
    P = torch.full((E,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_router_stats(cfg, logits, counts, f, P, loss, B.alloc_workspace(cfg))
    torch.cuda.synchronize()
    return to_np(f), to_np(P), float(loss.item())


@pytest.mark.parametrize("name", ["tiny", "odd", "e512", "keras", "decode", "prefill", "fanout"])
def test_router_stats_vs_oracle(name):
    say(f"[stats] {name}")
    d, dev = data_of(name)
    s = d.shape
    cfg = B.config_for(s)
    N, k, E = s.n_tokens, s.top_k, s.n_experts
    lg = torch.empty((N, E), dtype=torch.float32, device="cuda")
    w = torch.empty((N, k), dtype=torch.float32, device="cuda")
    e = torch.empty((N, k), dtype=torch.int32, device="cuda")
    ss = torch.empty((N,), dtype=torch.float32, device="cuda") if "w_shared_gate" in dev else None
    ws = B.alloc_workspace(cfg)
    B.moe_route(cfg, dev["x"], dev["w_router"], dev.get("w_shared_gate"), lg, w, e, ss, ws)
    # f depends on the selection: feed the counts of the oracle's own experts (on the GPU's logits,
    # P is independent of the selection) so no expected value comes from the GPU's routing; the
    # GPU's own grouping must give the same counts up to the near-tie tokens
    _, probs, _, e_ref = O.route(d.values("x"), d.values("w_router"), k, s.norm_topk_prob)
    loss_ref, f_ref, P_ref = O.switch_aux_loss(probs, e_ref, E)
    counts_ref = np.bincount(e_ref.reshape(-1), minlength=E).astype(np.int32)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    token_of = torch.empty(N * k, dtype=torch.int32, device="cuda")
    slot_pos = torch.empty(N * k, dtype=torch.int32, device="cuda")
    B.moe_permute(cfg, e, None, counts, offsets, token_of, slot_pos, None, ws)
    torch.cuda.synchronize()
    near = int((O.k_gap(probs, k) < 1e-6).sum())
    assert np.abs(to_np(counts).astype(np.int64) - counts_ref).sum() <= 2 * near
    f, P, loss = run_stats(cfg, lg, torch.from_numpy(counts_ref).cuda())
    assert np.allclose(f, f_ref, rtol=1e-6, atol=0)
    assert np.allclose(P, P_ref, rtol=1e-5, atol=1e-7), np.abs(P - P_ref).max()
    assert abs(loss - loss_ref) <= 1e-5 * loss_ref, (loss, loss_ref)
    f2, P2, loss2 = run_stats(cfg, lg, torch.from_numpy(counts_ref).cuda())      # deterministic
    assert np.array_equal(f, f2) and np.array_equal(P, P2) and loss == loss2


def test_router_stats_closed_forms():
    say("[stats] closed forms")
    E, k, N = 16, 2, 4096
    cfg = B.make_config(N, 128, E, k, 64)
    # even routing: every probability 1/E and every expert N k / E assignments -> loss 1
    logits = torch.zeros((N, E), dtype=torch.float32, device="cuda")
    counts = torch.full((E,), N * k // E, dtype=torch.int32, device="cuda")
    f, P, loss = run_stats(cfg, logits, counts)
    assert np.allclose(P, 1.0 / E, rtol=1e-6) and np.allclose(f, 1.0 / E, rtol=0)
    assert abs(loss - 1.0) <= 1e-5
    # collapsed router: expert 3 takes every assignment with probability ~1 -> loss ~ E
    cfg1 = B.make_config(N, 128, E, 1, 64)
    logits = torch.full((N, E), -60.0, dtype=torch.float32, device="cuda")
    logits[:, 3] = 60.0
    counts = torch.zeros((E,), dtype=torch.int32, device="cuda")
    counts[3] = N
    f, P, loss = run_stats(cfg1, logits, counts)
    assert f[3] == 1.0 and abs(P[3] - 1.0) <= 1e-6 and abs(loss - E) <= 1e-4
    # no tokens: zeros
    cfg0 = B.make_config(0, 128, E, k, 64)
    f, P, loss = run_stats(cfg0, None, None)
    assert not f.any() and not P.any() and loss == 0.0
