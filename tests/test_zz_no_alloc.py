"""moe_forward_noalloc (the entry point for callers that cannot allocate) against moe_forward through
the C ABI: same kernels, so outputs, routing weights and expert ids are bitwise equal. Two calls in a
row on the library's scratch, the second with fewer tokens, then a layer too large for the scratch."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _both(cfg, dev, n):
    """moe_forward (caller workspace) and moe_forward_noalloc on the first n tokens."""
    c = cfg.copy(n_tokens=n)
    x = dev["x"][:n].contiguous()
    outs = []
    for fn in ("ws", "noalloc"):
        y = torch.full((n, c.hidden), float("nan"), dtype=B.torch_dtype(c.out_dtype), device="cuda")
        w = torch.full((n, c.top_k), float("nan"), dtype=torch.float32, device="cuda")
        e = torch.full((n, c.top_k), -5, dtype=torch.int32, device="cuda")
        args = (c, x, dev["w_router"], dev["gate_up"], dev["down"], dev.get("shared_gate_up"), dev.get("shared_down"),
                dev.get("w_shared_gate"), y, w, e)
        if fn == "ws":
            B.moe_forward(*args, B.alloc_workspace(c))
        else:
            B.moe_forward_noalloc(*args)
        outs.append((y, w, e))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name,out_dtype,layout", [
    ("decode", "f32", "packed"),          # the decode layer as the benchmark runs it
    ("decode", "bf16", "rows"),
    ("keras", "f32", "rows"),             # E = 60: row layout only
    ("e512", "f32", "rows"),              # 512 experts, gated shared expert
])
def test_noalloc_equals_forward(name, out_dtype, layout):
    s = I.WORKLOADS.get(name) or I.custom_shape("e512", 130, 64, 512, 10, 16, shared_inter=16, seed=22)
    print(f"[noalloc] {name} out={out_dtype} {layout}", flush=True)
    d = I.make_inputs(s)
    dev = B.to_device(d.store)
    cfg = B.config_for(s, out_dtype, packed=layout == "packed")
    if layout == "packed":
        dev = B.pack_device_weights(cfg, dev)
    assert B.moe_workspace_bytes(cfg) <= B.NOALLOC_SCRATCH_BYTES
    # the full batch, then a smaller one on the scratch the first call left behind
    for n in (s.n_tokens, max(1, s.n_tokens // 3 - 4)):
        (y0, w0, e0), (y1, w1, e1) = _both(cfg, dev, n)
        assert torch.isfinite(y1.float()).all()
        assert torch.equal(_bits(y0), _bits(y1)), f"y differs at n={n}"
        assert torch.equal(_bits(w0), _bits(w1)) and torch.equal(e0, e1), f"routing differs at n={n}"


def test_noalloc_refuses_a_layer_above_the_scratch():
    cfg = B.make_config(16384, 2048, 128, 8, 768)
    x = torch.zeros((8, 8), device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_noalloc(cfg, x, x, x, x, None, None, None, x, None, None)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
