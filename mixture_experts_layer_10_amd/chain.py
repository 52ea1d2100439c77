"""The block with every buffer allocated once, run either as one moe_forward call (step() without
events) or as the chain of C-ABI calls moe_forward is made of (route -> permute -> gate_up -> down
-> [shared gate_up -> down] -> combine; decomposed()), so that the benchmark can put events around
the gate_up launch. Both produce the same bits; moe_forward may merge the routing and grouping of
small batches into fewer launches."""
from __future__ import annotations

import torch

from . import binding as B


class Chain:
    def __init__(self, cfg: B.MoeConfig, dev: dict, device="cuda"):
        self.cfg, self.dev = cfg, dev
        N, k, E, D, I, Is = cfg.n_tokens, cfg.top_k, cfg.n_experts, cfg.hidden, cfg.inter, cfg.shared_inter
        A = N * k
        f32, i32, dt = torch.float32, torch.int32, B.torch_dtype(cfg.dtype)
        e = lambda *shape, dtype=f32: torch.empty(shape, dtype=dtype, device=device)
        self.weights, self.experts = e(N, k), e(N, k, dtype=i32)
        self.gated = Is > 0 and dev.get("w_shared_gate") is not None
        self.shared_scale = e(N) if self.gated else None
        self.counts, self.offsets = e(E, dtype=i32), e(E + 1, dtype=i32)
        self.token_of, self.slot_pos = e(A, dtype=i32), e(A, dtype=i32)
        self.h, self.out = e(A, I, dtype=dt), e(A, D)
        self.sh_h = e(N, Is, dtype=dt) if Is else None
        self.sh_out = e(N, D) if Is else None
        self.y = e(N, D, dtype=B.torch_dtype(cfg.out_dtype))
        self.ws = B.alloc_workspace(cfg, device)
        self.A = A

    def step(self, gate_up_events=None):
        """One pass of the block: moe_forward, or the decomposed chain when gate_up events are given."""
        if gate_up_events is not None:
            return self.decomposed(gate_up_events)
        c, d = self.cfg, self.dev
        B.moe_forward(c, d["x"], d["w_router"], d["gate_up"], d["down"], d.get("shared_gate_up"), d.get("shared_down"),
                      d.get("w_shared_gate") if self.gated else None, self.y, self.weights, self.experts, self.ws)
        return self.y

    def decomposed(self, gate_up_events=None):
        c, d = self.cfg, self.dev
        B.moe_route(c, d["x"], d["w_router"], d.get("w_shared_gate") if self.gated else None, None,
                    self.weights, self.experts, self.shared_scale, self.ws)
        B.moe_permute(c, self.experts, None, self.counts, self.offsets, self.token_of, self.slot_pos, None, self.ws)
        if gate_up_events:
            gate_up_events[0].record()
        B.moe_expert_gate_up(c, c.n_experts, c.inter, self.A, d["x"], self.token_of, self.offsets, d["gate_up"], self.h)
        if gate_up_events:
            gate_up_events[1].record()
        B.moe_expert_down(c, c.n_experts, c.inter, self.A, self.offsets, self.h, d["down"], self.out)
        if c.shared_inter:
            B.moe_expert_gate_up(c, 1, c.shared_inter, c.n_tokens, d["x"], None, None, d["shared_gate_up"], self.sh_h)
            B.moe_expert_down(c, 1, c.shared_inter, c.n_tokens, None, self.sh_h, d["shared_down"], self.sh_out)
        B.moe_combine(c, self.out, self.weights, self.slot_pos, self.sh_out, self.shared_scale, self.y)
        return self.y
