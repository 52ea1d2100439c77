"""Seeded synthetic inputs for the sparse MoE block.

This module only draws and stores numbers. It computes nothing of the MoE method itself
(no router, softmax, selection, expert FFN or combine), so both the CPU oracle and the GPU
path can be fed from it without sharing any of the method's arithmetic.

Workloads (shapes from the pages):
  * ``tiny``     - a small fp32 layer that the oracle finishes instantly.
  * ``keras``    - the Keras Qwen3-VL-MoE defaults (E=60, k=4, expert width 1408, D=2048),
                   "Qwen3-VL-MoE" page, API table of ``Qwen3VLMoeModel``.
  * ``decode``   - Qwen3-VL-30B-A3B MoE layer (E=128, k=8, D=2048, I=768; config.json fields on
                   the "Qwen3-VL-30B-A3B-Instruct MoE architecture" page), 64 tokens, one per sequence.
  * ``prefill``  - the same layer at 16,384 tokens (16 requests of about 900 image tokens + 124 text
                   tokens; roughly 900 tokens per 1280x720 screenshot per the Qwen3-VL train-to-deploy
                   post), with expert load skewed to follow Zipf(s=1.2).
  * ``fanout``   - a Flash-Next-like layer: 512 routed experts, top-10, plus one shared expert
                   ("Mixture of experts" chapter, section "The shared expert").

Recipe (fixed, part of the contract):
  * ``rng = numpy.random.default_rng(1000 + index)`` with index 1..5 in the order above.
  * Draws, in this order: x[N,D] ~ N(0,1); w_router[E,D], gate_up[E,2I,D], down[E,D,I] ~ N(0, 0.02^2);
    then, with a shared expert, shared_gate_up[2I_s,D], shared_down[D,I_s], w_shared_gate[D],
    all ~ N(0, 0.02^2). Normals are drawn in float32.
  * bf16 workloads round every tensor to bfloat16 (round to nearest, ties to even) on the host.
    The oracle upcasts exactly those values; the GPU receives the same bits.
  * The ``prefill`` skew: hidden channel 0 of every token is set to 1.0 and column 0 of the router
    weight to b_e = -1.2 * ln(1 + perm[e]), perm a seeded permutation of the experts drawn after
    all other tensors. The router stays a plain linear map; its logits are those of a router with
    a per-expert bias b, so expected load falls off like rank^-1.2 (Gumbel-top-k reading of a
    Zipf(1.2) load, with Gaussian instead of Gumbel noise) while hot experts are scattered
    over the index range.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class MoeShape:
    name: str
    n_tokens: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int = 0
    norm_topk_prob: bool = True
    dtype: str = BF16
    seed: int = 0
    zipf_s: float = 0.0           # 0 = no skew
    shared_gated: bool = True     # shared expert scaled by sigmoid(w_s . x)

    def as_dict(self):
        return asdict(self)

    @property
    def assignments(self) -> int:
        return self.n_tokens * self.top_k


WORKLOADS = {
    "tiny": MoeShape("tiny", 64, 128, 8, 2, 64, 0, True, F32, 1001),
    "keras": MoeShape("keras", 512, 2048, 60, 4, 1408, 0, True, BF16, 1002),
    "decode": MoeShape("decode", 64, 2048, 128, 8, 768, 0, True, BF16, 1003),
    "prefill": MoeShape("prefill", 16384, 2048, 128, 8, 768, 0, True, BF16, 1004, zipf_s=1.2),
    "fanout": MoeShape("fanout", 8192, 2048, 512, 10, 256, 512, True, BF16, 1005),
}
WORKLOAD_ORDER = ["tiny", "keras", "decode", "prefill", "fanout"]


def custom_shape(name, n_tokens, hidden, n_experts, top_k, inter, shared_inter=0,
                 norm_topk_prob=True, dtype=BF16, seed=7, zipf_s=0.0, shared_gated=True):
    return MoeShape(name, n_tokens, hidden, n_experts, top_k, inter, shared_inter,
                    norm_topk_prob, dtype, seed, zipf_s, shared_gated)


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class MoeInputs:
    """One seeded draw. ``store`` holds what the GPU receives (float32 arrays, or uint16
    bfloat16 bit patterns); ``values(name)`` gives the exact float64 values of the same data."""
    shape: MoeShape
    store: dict = field(default_factory=dict)

    def values(self, name: str) -> Optional[np.ndarray]:
        a = self.store.get(name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def expert_view(self, name: str) -> "ExpertView":
        """Lazy float64 view of a stacked [E, ...] tensor: view[e] converts expert e only."""
        return ExpertView(self.store[name])

    def token_rows(self, idx) -> np.ndarray:
        """Exact float64 values of x for the given token indices only."""
        a = self.store["x"][np.asarray(idx)]
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


class ExpertView:
    def __init__(self, a: np.ndarray):
        self.a = a
        self.shape = a.shape

    def __len__(self):
        return self.a.shape[0]

    def __getitem__(self, e):
        v = self.a[e]
        return bf16_bits_to_f32(v).astype(np.float64) if v.dtype == np.uint16 else v.astype(np.float64)


TENSOR_ORDER = ["x", "w_router", "gate_up", "down", "shared_gate_up", "shared_down", "w_shared_gate"]


def make_inputs(shape: MoeShape) -> MoeInputs:
    s = shape
    rng = np.random.default_rng(s.seed)
    out = {}

    def normal(shp, std):
        a = rng.standard_normal(size=shp, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return a

    out["x"] = normal((s.n_tokens, s.hidden), 1.0)
    out["w_router"] = normal((s.n_experts, s.hidden), 0.02)
    out["gate_up"] = normal((s.n_experts, 2 * s.inter, s.hidden), 0.02)
    out["down"] = normal((s.n_experts, s.hidden, s.inter), 0.02)
    if s.shared_inter > 0:
        out["shared_gate_up"] = normal((2 * s.shared_inter, s.hidden), 0.02)
        out["shared_down"] = normal((s.hidden, s.shared_inter), 0.02)
        w = normal((s.hidden,), 0.02)
        if s.shared_gated:
            out["w_shared_gate"] = w
    if s.zipf_s > 0.0:
        perm = rng.permutation(s.n_experts)
        bias = -s.zipf_s * np.log(1.0 + perm.astype(np.float64))
        out["x"][:, 0] = 1.0
        out["w_router"][:, 0] = bias.astype(np.float32)
    if s.dtype == BF16:
        out = {k: round_to_bf16_bits(v) for k, v in out.items()}
    return MoeInputs(s, out)
