"""The seeded input recipe: shapes, draw order, bf16 rounding and the prefill load skew."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_10_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-3, 65504.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)])
    ours = I.round_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_tiny_recipe_is_deterministic_and_shaped():
    s = I.WORKLOADS["tiny"]
    a, b = I.make_inputs(s), I.make_inputs(s)
    for k in ("x", "w_router", "gate_up", "down"):
        assert np.array_equal(a.store[k], b.store[k])
    assert a.store["x"].dtype == np.float32
    assert a.store["gate_up"].shape == (8, 128, 128)
    assert a.store["down"].shape == (8, 128, 64)
    assert abs(a.store["w_router"].std() - 0.02) < 0.002
    rng = np.random.default_rng(1001)
    assert np.array_equal(a.store["x"], rng.standard_normal((64, 128), dtype=np.float32))


def test_shared_tensors_and_bf16_storage():
    s = I.custom_shape("t", 9, 16, 5, 2, 8, shared_inter=24)
    d = I.make_inputs(s)
    assert d.store["shared_gate_up"].shape == (48, 16)
    assert d.store["shared_down"].shape == (16, 24)
    assert d.store["w_shared_gate"].shape == (16,)
    assert d.store["x"].dtype == np.uint16
    v = d.values("x")
    assert v.dtype == np.float64 and np.array_equal(v, I.bf16_bits_to_f32(d.store["x"]))


@pytest.mark.slow
def test_prefill_skew_realised_load():
    s = I.WORKLOADS["prefill"]
    d = I.make_inputs(s)
    x = d.values("x")
    assert np.all(x[:, 0] == 1.0)
    _, _, _, experts = O.route(x, d.values("w_router"), s.top_k, True)
    counts = np.bincount(experts.reshape(-1), minlength=s.n_experts)
    top = np.sort(counts)[::-1]
    assert counts.sum() == s.n_tokens * s.top_k
    assert top[0] > 0.9 * s.n_tokens                 # the hottest expert sees almost every token
    assert top[:8].sum() > 0.6 * counts.sum()        # heavy head
    assert (counts == 0).sum() >= 3                  # and a few idle experts
