"""Tile list of the streaming grouped GEMM (gate_up + down) under group-size mixes that exercise its
ordering: every count of live 32-row blocks in a group's last m-tile (sizes at and around the
multiples of 32 and 256, empty groups), and the largest group count the boundary accepts. The list
only changes which workgroup computes a tile and when, so the result must equal the oracle's
grouped FFN to the bf16 bar, and the packed and row layouts must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import inputs as I
from parity_util import rel_err, to_np
from test_gpu_packed import _ffn
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

CLASS_SIZES = [0, 1, 31, 32, 33, 64, 95, 96, 128, 160, 192, 223, 224, 225, 255, 256, 257, 288, 480, 511, 512,
               513, 700, 767, 768, 1000, 2100, 0, 37]


@pytest.mark.parametrize("case", ["classes", "max_groups"])
def test_tile_order_ffn(case):
    D, I_ = 384, 256                              # down: a full and a half-empty 256-column tile
    if case == "classes":
        rows = CLASS_SIZES
    else:
        rows = list(np.random.default_rng(11).integers(0, 700, 512))   # 512 groups, the maximum
    G = len(rows)
    offsets = np.zeros(G + 1, np.int64)
    offsets[1:] = np.cumsum(rows)
    R = int(offsets[-1])
    assert R > 64 * G                             # tall groups: the streaming kernel, not weight streaming
    say(f"[tile order] {case}: G={G} rows={R}")
    d = I.make_inputs(I.custom_shape("tile_order", R, D, G, 1, I_, seed=600 + G))
    dev = B.to_device(d.store)
    cfg_rows = B.make_config(R, D, min(G, 512), 1, I_)
    cfg_pack = B.make_config(R, D, 16, 1, I_, packed=True)
    pdev = {}
    for name, (r_, c_) in {"gate_up": (2 * I_, D), "down": (D, I_)}.items():
        pdev[name] = torch.empty_like(dev[name])
        B.moe_pack_weights(cfg_pack, G, r_, c_, dev[name], pdev[name])
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    perm = np.random.default_rng(5).permutation(R)
    ridx = torch.from_numpy(perm.astype(np.int32)).cuda()
    h0, o0 = _ffn(cfg_rows, G, I_, R, dev["x"], ridx, off, dev["gate_up"], dev["down"])
    h1, o1 = _ffn(cfg_pack, G, I_, R, dev["x"], ridx, off, pdev["gate_up"], pdev["down"])
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
    got = to_np(o1)
    assert np.isfinite(got).all()                 # every row written (outputs start as NaN)
    ref = O.grouped_expert_ffn(d.values("x")[perm], offsets, d.expert_view("gate_up"), d.expert_view("down"))
    err = rel_err(got, ref)
    say(f"  max|d out|/rms = {err:.3e}")
    assert err <= 2e-2
