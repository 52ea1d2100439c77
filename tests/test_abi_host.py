"""C ABI checks that need no GPU: the library loads, exports every symbol the header declares,
sizes workspaces on the host, and refuses bad arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_10_amd import binding as B
from mixture_experts_layer_10_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        BUILD.build()
    return B.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_symbols_all_exported(lib):
    names = header_functions()
    assert len(names) == 20
    assert sorted(B.EXPORTED) == names
    for n in names:
        assert getattr(lib, n) is not None


def test_config_struct_layout_matches_header():
    assert ctypes.sizeof(B.MoeConfig) == 6 * 8 + 5 * 4 + 4       # five int32 fields, padded to 8 bytes


def test_status_strings(lib):
    assert B.status_string(0) == "MOE_OK"
    assert B.status_string(-3) == "MOE_ERR_WORKSPACE"
    assert B.status_string(99) == "MOE_ERR_UNKNOWN"


def test_workspace_bytes_host_only(lib):
    c = B.make_config(16384, 2048, 128, 8, 768)
    n = B.moe_workspace_bytes(c)
    A = 16384 * 8
    assert n >= A * 2048 * 4 + A * 768 * 2            # fp32 expert outputs + bf16 h
    assert n < A * 2048 * 4 * 1.3
    # fp16 expert outputs: rows of 2 D value bytes + D / 16 exponent bytes instead of 4 D
    f = B.moe_workspace_bytes(c.copy(expert_out=B.MOE_EXPERT_OUT_F16S))
    assert n - f == A * (2048 * 4 - (2 * 2048 + 2048 // 16))
    c5 = B.make_config(8192, 2048, 512, 10, 256, shared_inter=512)
    assert B.moe_workspace_bytes(c5) > B.moe_workspace_bytes(c5.copy(shared_inter=0))


@pytest.mark.parametrize("field,value,status", [
    ("n_tokens", -1, B.MOE_ERR_INVALID_ARG),
    ("hidden", 0, B.MOE_ERR_INVALID_ARG),
    ("n_experts", 0, B.MOE_ERR_INVALID_ARG),
    ("top_k", 0, B.MOE_ERR_INVALID_ARG),
    ("top_k", 9, B.MOE_ERR_INVALID_ARG),
    ("inter", 0, B.MOE_ERR_INVALID_ARG),
    ("shared_inter", -8, B.MOE_ERR_INVALID_ARG),
    ("norm_topk_prob", 2, B.MOE_ERR_INVALID_ARG),
    ("weight_layout", 5, B.MOE_ERR_INVALID_ARG),
    ("weight_layout", 4, B.MOE_ERR_UNSUPPORTED),      # FP8: the packed shape rules
    ("weight_layout", -1, B.MOE_ERR_INVALID_ARG),
    ("weight_layout", 2, B.MOE_ERR_UNSUPPORTED),      # quantised: the packed shape rules
    ("weight_layout", 1, B.MOE_ERR_UNSUPPORTED),      # packed needs widths that are multiples of 128
    ("dtype", 7, B.MOE_ERR_UNSUPPORTED),
    ("out_dtype", 3, B.MOE_ERR_UNSUPPORTED),
    ("hidden", 36, B.MOE_ERR_UNSUPPORTED),             # bf16 rows must be 16-byte vectors
    ("inter", 12, B.MOE_ERR_UNSUPPORTED),
    ("n_experts", 513, B.MOE_ERR_UNSUPPORTED),
    ("expert_out", 2, B.MOE_ERR_INVALID_ARG),
    ("expert_out", -1, B.MOE_ERR_INVALID_ARG),
])
def test_config_validation(lib, field, value, status):
    c = B.make_config(64, 128, 8, 2, 64).copy(**{field: value})
    with pytest.raises(B.MoeError) as ei:
        B.moe_workspace_bytes(c)
    assert ei.value.status == status
    assert field.split("_")[0] in B.last_error() or B.last_error()


def test_f16s_expert_out_rules(lib):
    ok = B.make_config(64, 256, 16, 2, 128, expert_out=B.MOE_EXPERT_OUT_F16S)
    assert B.moe_workspace_bytes(ok) > 0 and B.f16s_supported(ok)
    assert B.moe_workspace_bytes(ok.copy(weight_layout=B.MOE_LAYOUT_PACKED)) > 0
    for bad in (B.make_config(64, 256, 16, 2, 128, dtype="f32", expert_out=1),      # fp32 layers
                B.make_config(64, 40, 16, 2, 128, expert_out=1),                    # D % 16 != 0
                B.make_config(64, 256, 16, 2, 128, layout=B.MOE_LAYOUT_Q8, expert_out=1)):
        assert not B.f16s_supported(bad)
        with pytest.raises(B.MoeError) as ei:
            B.moe_workspace_bytes(bad)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "fp16 expert outputs" in str(ei.value)
    # expert-output buffers are 16-byte vectors: a misaligned out is refused before any launch
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_down(ok, 16, 128, 128, FAKE, FAKE, FAKE, FAKE + 8, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "aligned" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_combine(ok, FAKE + 4, FAKE, FAKE, None, None, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_packed_layout_rules(lib):
    ok = B.make_config(64, 256, 16, 2, 128, shared_inter=384, packed=True)
    assert B.moe_workspace_bytes(ok) > 0 and B.packable(ok)
    for bad in (B.make_config(64, 256, 16, 2, 128, dtype="f32", packed=True),
                B.make_config(64, 256, 16, 2, 128, shared_inter=64, packed=True),
                B.make_config(64, 200, 16, 2, 128, packed=True)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_workspace_bytes(bad)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "packed" in str(ei.value)
    # any E: the experts are packed, the router only when E % 16 == 0 (else it keeps its rows)
    e60 = B.make_config(64, 256, 60, 2, 128, packed=True)
    assert B.moe_workspace_bytes(e60) > 0 and B.packable(e60) and not B.router_packed(e60) and B.router_packed(ok)
    # the standalone expert entry points check the width they are given
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_ffn(ok, 8, 96, 128, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_pack_refuses_before_launch(lib):
    c = B.make_config(64, 256, 8, 2, 128)
    cases = [
        (dict(cfg=B.make_config(64, 256, 8, 2, 128, dtype="f32")), B.MOE_ERR_UNSUPPORTED),
        (dict(rows=24), B.MOE_ERR_UNSUPPORTED),
        (dict(cols=48), B.MOE_ERR_UNSUPPORTED),
        (dict(rows=-16), B.MOE_ERR_INVALID_ARG),
        (dict(src=None), B.MOE_ERR_INVALID_ARG),
        (dict(dst=FAKE + 1024), B.MOE_ERR_INVALID_ARG),          # overlaps src
        (dict(dst=FAKE * 4 + 8), B.MOE_ERR_UNSUPPORTED),         # not 16-byte aligned
    ]
    for kw, status in cases:
        a = dict(cfg=c, n_groups=2, rows=32, cols=64, src=FAKE, dst=FAKE * 4)
        a.update(kw)
        with pytest.raises(B.MoeError) as ei:
            B.moe_pack_weights(a["cfg"], a["n_groups"], a["rows"], a["cols"], a["src"], a["dst"], stream=0)
        assert ei.value.status == status, (kw, str(ei.value))
    B.moe_pack_weights(c, 0, 32, 64, None, None, stream=0)       # nothing to pack: no-op


@pytest.mark.parametrize("layout,bits", [(B.MOE_LAYOUT_Q8, 8), (B.MOE_LAYOUT_Q4, 4), (B.MOE_LAYOUT_F8, 8)])
def test_quantized_bytes_and_layout_rules(lib, layout, bits):
    c = B.make_config(64, 256, 16, 2, 128, shared_inter=384, layout=layout)
    assert B.moe_workspace_bytes(c) > 0
    G, R, K = 16, 256, 2048
    codes = G * (R // 16) * (K // 128) * 1088 if bits == 4 else G * R * K * bits // 8   # int4: 64 multiplier bytes per 1 KB
    assert B.moe_quantized_bytes(c, G, R, K) == codes + G * R * 4
    if bits == 4:                                            # int4 super-blocks are 128 columns wide
        with pytest.raises(B.MoeError) as ei:
            B.moe_quantized_bytes(c, G, R, 96)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "128" in str(ei.value)
    # the quantised layouts follow the packed shape rules
    assert B.moe_workspace_bytes(B.make_config(64, 256, 8, 2, 128, layout=layout)) > 0   # router in rows
    for bad in (B.make_config(64, 256, 16, 2, 128, dtype="f32", layout=layout),
                B.make_config(64, 256, 16, 2, 96, layout=layout)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_workspace_bytes(bad)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:
        B.moe_workspace_bytes(c.copy(weight_layout=5))
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


def test_quantize_refuses_before_launch(lib):
    q8 = B.make_config(64, 256, 16, 2, 128, layout=B.MOE_LAYOUT_Q8)
    cases = [
        (dict(cfg=B.make_config(64, 256, 16, 2, 128, packed=True)), B.MOE_ERR_INVALID_ARG),   # not quantised
        (dict(cols=48), B.MOE_ERR_UNSUPPORTED),                  # columns come in blocks of 32
        (dict(rows=24), B.MOE_ERR_UNSUPPORTED),
        (dict(rows=-16), B.MOE_ERR_INVALID_ARG),
        (dict(src=None), B.MOE_ERR_INVALID_ARG),
        (dict(dst=FAKE + 1024), B.MOE_ERR_INVALID_ARG),          # overlaps src
        (dict(dst=FAKE * 4 + 8), B.MOE_ERR_UNSUPPORTED),         # not 16-byte aligned
    ]
    for kw, status in cases:
        a = dict(cfg=q8, n_groups=2, rows=32, cols=256, src=FAKE, dst=FAKE * 4)
        a.update(kw)
        with pytest.raises(B.MoeError) as ei:
            B.moe_quantize_weights(a["cfg"], a["n_groups"], a["rows"], a["cols"], a["src"], a["dst"], stream=0)
        assert ei.value.status == status, (kw, str(ei.value))
    with pytest.raises(B.MoeError) as ei:
        B.moe_quantized_bytes(q8, 2, 32, 200)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    B.moe_quantize_weights(q8, 0, 32, 256, None, None, stream=0)  # nothing to quantise: no-op
    # expert weights must be 16-byte aligned (every weight load is 16 bytes wide)
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_gate_up(q8, 2, 128, 64, FAKE, None, FAKE, FAKE + 4, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "aligned" in str(ei.value)


def test_backward_rules_and_workspace(lib):
    c = B.make_config(64, 256, 12, 2, 128)
    n = B.moe_backward_workspace_bytes(c)
    assert n > 64 * 2 * 2 * 128 * 4                               # at least the recomputed pre-activations
    assert B.moe_backward_workspace_bytes(c.copy(shared_inter=128)) > n
    assert B.moe_backward_workspace_bytes(c.copy(dtype=B.MOE_F32, out_dtype=B.MOE_F32)) > n   # fp32 intermediates
    for bad, what in ((B.make_config(64, 256, 16, 2, 128, packed=True), "row-layout"),):
        with pytest.raises(B.MoeError) as ei:
            B.moe_backward_workspace_bytes(bad)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED and what in str(ei.value)
    args = [FAKE] * 4 + [None] * 3 + [FAKE] + [FAKE * 2] * 4 + [None] * 3
    with pytest.raises(B.MoeError) as ei:                          # no workspace
        B.moe_backward(c, *args, None, 0, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    no_dy = list(args)
    no_dy[7] = None
    with pytest.raises(B.MoeError) as ei:
        B.moe_backward(c, *no_dy, FAKE * 4, n, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    cs = c.copy(shared_inter=128)
    with pytest.raises(B.MoeError) as ei:                          # shared expert without its gradients
        B.moe_backward(cs, *args[:4], FAKE, FAKE, None, *args[7:], FAKE * 4, 1 << 40, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    B.moe_backward(c.copy(n_tokens=0), *args, None, 0, stream=0)  # no tokens: no-op


def test_router_stats_refuses_before_launch(lib):
    c = B.make_config(300, 128, 8, 2, 64)
    with pytest.raises(B.MoeError) as ei:                       # no place for the outputs
        B.moe_router_stats(c, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:                       # tokens but no logits
        B.moe_router_stats(c, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:                       # 2 blocks x 8 experts x 4 B needed
        B.moe_router_stats(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert B.moe_workspace_bytes(c) >= 2 * 8 * 4


def test_null_config_and_null_out(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_bytes(ctypes.byref(B.make_config(4, 8, 2, 1, 8)), None) == B.MOE_ERR_INVALID_ARG


FAKE = 1 << 20    # never dereferenced: every call below fails validation on the host first


def test_route_refuses_before_launch(lib):
    c = B.make_config(64, 128, 8, 2, 64)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(c, None, FAKE, None, None, FAKE, FAKE, None, None, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG and "x" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:          # gate without a place for its output
        B.moe_route(c, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(lib):
    c = B.make_config(0, 128, 8, 2, 64)
    B.moe_route(c, None, None, None, None, None, None, None, stream=0)
    B.moe_combine(c, None, None, None, None, None, None, stream=0)
    B.moe_forward(c, None, None, None, None, None, None, None, None, None, None, None, 0, stream=0)
    B.moe_expert_ffn(c, 1, 64, 0, None, None, None, None, None, None, None, stream=0)


def test_forward_workspace_checks(lib):
    c = B.make_config(64, 128, 8, 2, 64)
    need = B.moe_workspace_bytes(c)
    args = (c, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(*args, FAKE, need - 1, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(*args, FAKE + 16, need, stream=0)     # not 256-byte aligned
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoeError) as ei:                    # shared tensors without shared_inter
        B.moe_forward(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    cs = c.copy(shared_inter=32)
    with pytest.raises(B.MoeError) as ei:                    # shared_inter without its tensors
        B.moe_forward(cs, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None, FAKE,
                      B.moe_workspace_bytes(cs), stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


def test_forward_noalloc_refuses_before_launch(lib):
    # the scratch limit is checked on the host: a layer needing more returns MOE_ERR_WORKSPACE
    big = B.make_config(16384, 2048, 128, 8, 768)
    assert B.moe_workspace_bytes(big) > B.NOALLOC_SCRATCH_BYTES
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_noalloc(big, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE and "scratch" in str(ei.value)
    c = B.make_config(64, 128, 8, 2, 64)
    with pytest.raises(B.MoeError) as ei:                    # y missing
        B.moe_forward_noalloc(c, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None, None, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    B.moe_forward_noalloc(c.copy(n_tokens=0), None, None, None, None, None, None, None, None, None, None, stream=0)


def test_permute_and_ffn_argument_checks(lib):
    c = B.make_config(64, 128, 8, 2, 64)
    with pytest.raises(B.MoeError) as ei:
        B.moe_permute(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG        # x without x_perm
    with pytest.raises(B.MoeError) as ei:
        B.moe_permute(c, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_ffn(c, 8, 64, 128, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG        # 8 groups need offsets
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_ffn(c, 8, 60, 128, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED        # inter 60 not a multiple of 8
    with pytest.raises(B.MoeError) as ei:
        B.moe_combine(c, FAKE, FAKE, FAKE, None, FAKE, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG        # scale without shared output
