"""ctypes binding of the C ABI in include/moe.h. Argument marshalling only: every step of the
block runs in the HIP library. Tensors are torch device tensors (PyTorch provides device memory
and streams); each function passes raw pointers and the current torch stream to the C call of
the same name and raises MoeError on a non-zero status.

The library is loaded from mixture_experts_layer_10_amd/_lib/libmoe_mi355x.so. If it is missing,
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same library (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(PKG, "_lib", "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROWS, MOE_LAYOUT_PACKED, MOE_LAYOUT_Q8, MOE_LAYOUT_Q4, MOE_LAYOUT_F8 = 0, 1, 2, 3, 4
MOE_EXPERT_OUT_F32, MOE_EXPERT_OUT_F16S = 0, 1

# Every symbol include/moe.h declares.
EXPORTED = ["moe_status_string", "moe_last_error", "moe_workspace_bytes", "moe_route", "moe_permute",
            "moe_expert_gate_up", "moe_expert_down", "moe_expert_ffn", "moe_pack_weights", "moe_router_stats",
            "moe_combine", "moe_forward", "moe_route_sigmoid", "moe_router_bias_update", "moe_permute_capped",
            "moe_quantized_bytes", "moe_quantize_weights", "moe_backward_workspace_bytes", "moe_backward",
            "moe_forward_noalloc"]
NOALLOC_SCRATCH_BYTES = 64 << 20      # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status}): {detail}")


class MoeConfig(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("n_experts", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("inter", ctypes.c_int64), ("shared_inter", ctypes.c_int64),
                ("norm_topk_prob", ctypes.c_int32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("expert_out", ctypes.c_int32)]

    def copy(self, **kw):
        c = MoeConfig()
        for name, _ in self._fields_:
            setattr(c, name, kw.get(name, getattr(self, name)))
        return c


def make_config(n_tokens, hidden, n_experts, top_k, inter, shared_inter=0, norm_topk_prob=True,
                dtype="bf16", out_dtype=None, packed=False, layout=None, expert_out=MOE_EXPERT_OUT_F32) -> MoeConfig:
    """layout: a MOE_LAYOUT_* value; default rows, or packed when ``packed``. expert_out: a
    MOE_EXPERT_OUT_* value (the form of the per-assignment expert outputs)."""
    dt = {"bf16": MOE_BF16, "f32": MOE_F32}
    if layout is None:
        layout = MOE_LAYOUT_PACKED if packed else MOE_LAYOUT_ROWS
    return MoeConfig(n_tokens, hidden, n_experts, top_k, inter, shared_inter, int(bool(norm_topk_prob)),
                     dt[dtype], dt[out_dtype or dtype], layout, expert_out)


def config_for(shape, out_dtype=None, packed=False, layout=None, expert_out=MOE_EXPERT_OUT_F32) -> MoeConfig:
    """MoeConfig for an inputs.MoeShape."""
    return make_config(shape.n_tokens, shape.hidden, shape.n_experts, shape.top_k, shape.inter,
                       shape.shared_inter, shape.norm_topk_prob, shape.dtype, out_dtype, packed, layout, expert_out)


def f16s_supported(cfg: MoeConfig) -> bool:
    """Whether MOE_EXPERT_OUT_F16S applies (bf16, D % 16 == 0, row or packed bf16 weights)."""
    return cfg.dtype == MOE_BF16 and cfg.hidden % 16 == 0 and cfg.weight_layout in (MOE_LAYOUT_ROWS, MOE_LAYOUT_PACKED)


def packable(cfg: MoeConfig) -> bool:
    """Whether the packed weight layout applies (bf16, widths multiples of 128)."""
    return cfg.dtype == MOE_BF16 and cfg.hidden % 128 == 0 and cfg.inter % 128 == 0 and cfg.shared_inter % 128 == 0


def router_packed(cfg: MoeConfig) -> bool:
    """Whether a packed or quantised layout packs the router too (n_experts a multiple of 16)."""
    return cfg.weight_layout != MOE_LAYOUT_ROWS and cfg.n_experts % 16 == 0


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_CFG = ctypes.POINTER(MoeConfig)


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} (run python -m mixture_experts_layer_10_amd.build)")
    lib = ctypes.CDLL(path)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_workspace_bytes": (ctypes.c_int, [_CFG, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_route": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_permute": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_expert_gate_up": (ctypes.c_int, [_CFG, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
        "moe_expert_down": (ctypes.c_int, [_CFG, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
        "moe_expert_ffn": (ctypes.c_int, [_CFG, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
        "moe_pack_weights": (ctypes.c_int, [_CFG, _I64, _I64, _I64, _P, _P, _P]),
        "moe_router_stats": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_route_sigmoid": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_router_bias_update": (ctypes.c_int, [_CFG, _P, _P, ctypes.c_float, _P]),
        "moe_permute_capped": (ctypes.c_int, [_CFG, _I64, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_combine": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P]),
        "moe_quantized_bytes": (ctypes.c_int, [_CFG, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_quantize_weights": (ctypes.c_int, [_CFG, _I64, _I64, _I64, _P, _P, _P]),
        "moe_backward_workspace_bytes": (ctypes.c_int, [_CFG, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_backward": (ctypes.c_int, [_CFG] + [_P] * 16 + [ctypes.c_size_t, _P]),
        "moe_forward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "moe_forward_noalloc": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def last_error() -> str:
    return load().moe_last_error().decode()


def _ptr(t) -> Optional[int]:
    """Raw pointer of a contiguous tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, last_error())


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", load().moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return ws_bytes
    return 0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size()


def moe_route(cfg, x, w_router, w_shared_gate, logits, weights, experts, shared_scale, ws=None, ws_bytes=None,
              stream=None):
    _check("moe_route", load().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(w_shared_gate),
                                         _ptr(logits), _ptr(weights), _ptr(experts), _ptr(shared_scale),
                                         _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)))


def moe_permute(cfg, experts, x, counts, offsets, token_of, slot_pos, x_perm, ws, ws_bytes=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else (0 if ws is None or isinstance(ws, int)
                                                    else ws.numel() * ws.element_size())
    _check("moe_permute", load().moe_permute(ctypes.byref(cfg), _ptr(experts), _ptr(x), _ptr(counts), _ptr(offsets),
                                             _ptr(token_of), _ptr(slot_pos), _ptr(x_perm), _ptr(ws), nbytes,
                                             _stream(stream)))


def moe_expert_gate_up(cfg, n_groups, inter, max_rows, x, row_index, offsets, gate_up, h, stream=None):
    _check("moe_expert_gate_up", load().moe_expert_gate_up(ctypes.byref(cfg), n_groups, inter, max_rows, _ptr(x),
                                                           _ptr(row_index), _ptr(offsets), _ptr(gate_up), _ptr(h),
                                                           _stream(stream)))


def moe_expert_down(cfg, n_groups, inter, max_rows, offsets, h, down, out, stream=None):
    _check("moe_expert_down", load().moe_expert_down(ctypes.byref(cfg), n_groups, inter, max_rows, _ptr(offsets),
                                                     _ptr(h), _ptr(down), _ptr(out), _stream(stream)))


def moe_expert_ffn(cfg, n_groups, inter, max_rows, x, row_index, offsets, gate_up, down, h, out, stream=None):
    _check("moe_expert_ffn", load().moe_expert_ffn(ctypes.byref(cfg), n_groups, inter, max_rows, _ptr(x),
                                                   _ptr(row_index), _ptr(offsets), _ptr(gate_up), _ptr(down),
                                                   _ptr(h), _ptr(out), _stream(stream)))


def moe_pack_weights(cfg, n_groups, rows, cols, src, dst, stream=None):
    _check("moe_pack_weights", load().moe_pack_weights(ctypes.byref(cfg), n_groups, rows, cols, _ptr(src), _ptr(dst),
                                                       _stream(stream)))


def moe_quantized_bytes(cfg, n_groups, rows, cols) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_quantized_bytes", load().moe_quantized_bytes(ctypes.byref(cfg), n_groups, rows, cols, ctypes.byref(n)))
    return n.value


def moe_quantize_weights(cfg, n_groups, rows, cols, src, dst, stream=None):
    _check("moe_quantize_weights", load().moe_quantize_weights(ctypes.byref(cfg), n_groups, rows, cols, _ptr(src),
                                                               _ptr(dst), _stream(stream)))


def moe_backward_workspace_bytes(cfg) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_bytes", load().moe_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def moe_backward(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, dy, dx, dw_router,
                 dgate_up, ddown, dshared_gate_up, dshared_down, dw_shared_gate, ws, ws_bytes=None, stream=None):
    _check("moe_backward", load().moe_backward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(gate_up), _ptr(down),
                                               _ptr(shared_gate_up), _ptr(shared_down), _ptr(w_shared_gate), _ptr(dy),
                                               _ptr(dx), _ptr(dw_router), _ptr(dgate_up), _ptr(ddown),
                                               _ptr(dshared_gate_up), _ptr(dshared_down), _ptr(dw_shared_gate),
                                               _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)))


def backward(cfg: MoeConfig, dev: dict, dy, ws=None, stream=None):
    """Run moe_backward on the tensors of ``dev``; returns the fp32 gradients dx, dw_router, dgate_up,
    ddown (and dshared_gate_up, dshared_down, dw_shared_gate when the shapes have them)."""
    import torch
    x = dev["x"]
    out = {"dx": torch.empty(x.shape, dtype=torch.float32, device=x.device)}
    pairs = [("dw_router", "w_router"), ("dgate_up", "gate_up"), ("ddown", "down")]
    if cfg.shared_inter:
        pairs += [("dshared_gate_up", "shared_gate_up"), ("dshared_down", "shared_down")]
        if dev.get("w_shared_gate") is not None:
            pairs.append(("dw_shared_gate", "w_shared_gate"))
    for name, key in pairs:
        out[name] = torch.empty(dev[key].shape, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_backward_workspace_bytes(cfg), 256), dtype=torch.uint8, device=x.device)
    moe_backward(cfg, x, dev["w_router"], dev["gate_up"], dev["down"], dev.get("shared_gate_up"), dev.get("shared_down"),
                 dev.get("w_shared_gate"), dy, out["dx"], out["dw_router"], out["dgate_up"], out["ddown"],
                 out.get("dshared_gate_up"), out.get("dshared_down"), out.get("dw_shared_gate"), ws, stream=stream)
    return out


def moe_route_sigmoid(cfg, x, w_router, bias, logits, weights, experts, ws=None, ws_bytes=None, stream=None):
    _check("moe_route_sigmoid", load().moe_route_sigmoid(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias),
                                                         _ptr(logits), _ptr(weights), _ptr(experts), _ptr(ws),
                                                         _nbytes(ws, ws_bytes), _stream(stream)))


def moe_router_bias_update(cfg, counts, bias, gamma, stream=None):
    _check("moe_router_bias_update", load().moe_router_bias_update(ctypes.byref(cfg), _ptr(counts), _ptr(bias),
                                                                   float(gamma), _stream(stream)))


def moe_permute_capped(cfg, capacity, experts, x, counts, offsets, token_of, slot_pos, x_perm, ws, ws_bytes=None,
                       stream=None):
    _check("moe_permute_capped", load().moe_permute_capped(ctypes.byref(cfg), int(capacity), _ptr(experts), _ptr(x),
                                                           _ptr(counts), _ptr(offsets), _ptr(token_of), _ptr(slot_pos),
                                                           _ptr(x_perm), _ptr(ws), _nbytes(ws, ws_bytes),
                                                           _stream(stream)))


def moe_router_stats(cfg, logits, counts, f, P, loss, ws, ws_bytes=None, stream=None):
    _check("moe_router_stats", load().moe_router_stats(ctypes.byref(cfg), _ptr(logits), _ptr(counts), _ptr(f), _ptr(P),
                                                       _ptr(loss), _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)))


def moe_combine(cfg, out_perm, weights, slot_pos, shared_out, shared_scale, y, stream=None):
    _check("moe_combine", load().moe_combine(ctypes.byref(cfg), _ptr(out_perm), _ptr(weights), _ptr(slot_pos),
                                             _ptr(shared_out), _ptr(shared_scale), _ptr(y), _stream(stream)))


def moe_forward(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y,
                weights_out, experts_out, ws, ws_bytes=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else (0 if ws is None or isinstance(ws, int)
                                                    else ws.numel() * ws.element_size())
    _check("moe_forward", load().moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(gate_up), _ptr(down),
                                             _ptr(shared_gate_up), _ptr(shared_down), _ptr(w_shared_gate), _ptr(y),
                                             _ptr(weights_out), _ptr(experts_out), _ptr(ws), nbytes,
                                             _stream(stream)))


def moe_forward_noalloc(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y,
                        weights_out, experts_out, stream=None):
    _check("moe_forward_noalloc",
           load().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(gate_up), _ptr(down),
                                      _ptr(shared_gate_up), _ptr(shared_down), _ptr(w_shared_gate), _ptr(y),
                                      _ptr(weights_out), _ptr(experts_out), _stream(stream)))


# ------------------------------------------------------------------------------------------------
# Torch conveniences (allocation only).
# ------------------------------------------------------------------------------------------------

def to_device(store: dict, device="cuda"):
    """Host arrays (float32, or uint16 bfloat16 bits) -> device tensors with the same bits."""
    import torch
    out = {}
    for k, a in store.items():
        if a.dtype == np.uint16:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out


def torch_dtype(code):
    import torch
    return torch.bfloat16 if code == MOE_BF16 else torch.float32


def pack_device_weights(cfg: MoeConfig, dev: dict):
    """A copy of ``dev`` whose weight matrices (gate_up, down, the shared pair and, when E % 16 == 0,
    the router) are in the packed layout, made by moe_pack_weights (a one-time step, like loading
    the model)."""
    import torch
    D, E, I, Is = cfg.hidden, cfg.n_experts, cfg.inter, cfg.shared_inter
    out = dict(dev)
    shapes = {"gate_up": (E, 2 * I, D), "down": (E, D, I)}
    if router_packed(cfg):
        shapes["w_router"] = (1, E, D)
    if Is:
        shapes.update(shared_gate_up=(1, 2 * Is, D), shared_down=(1, D, Is))
    for name, (g, r, c) in shapes.items():
        src = dev[name]
        dst = torch.empty_like(src)
        moe_pack_weights(cfg, g, r, c, src, dst)
        out[name] = dst
    return out


def quantize_device_weights(cfg: MoeConfig, dev: dict):
    """A copy of ``dev`` (row layout) for a quantised ``cfg``: the router packed (bf16) by
    moe_pack_weights when E % 16 == 0, gate_up, down and the shared pair quantised by moe_quantize_weights into uint8
    buffers of moe_quantized_bytes() bytes (a one-time step, like loading the model)."""
    import torch
    D, E, I, Is = cfg.hidden, cfg.n_experts, cfg.inter, cfg.shared_inter
    out = dict(dev)
    if router_packed(cfg):
        dst = torch.empty_like(dev["w_router"])
        moe_pack_weights(cfg, 1, E, D, dev["w_router"], dst)
        out["w_router"] = dst
    shapes = {"gate_up": (E, 2 * I, D), "down": (E, D, I)}
    if Is:
        shapes.update(shared_gate_up=(1, 2 * Is, D), shared_down=(1, D, Is))
    for name, (g, r, c) in shapes.items():
        q = torch.empty(moe_quantized_bytes(cfg, g, r, c), dtype=torch.uint8, device=dev[name].device)
        moe_quantize_weights(cfg, g, r, c, dev[name], q)
        out[name] = q
    return out


def alloc_workspace(cfg: MoeConfig, device="cuda"):
    import torch
    n = moe_workspace_bytes(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def forward(cfg: MoeConfig, dev: dict, ws=None, y=None, weights=None, experts=None, stream=None):
    """Run moe_forward on the tensors of ``dev`` (keys as in inputs.TENSOR_ORDER). Returns y."""
    import torch
    x = dev["x"]
    if y is None:
        y = torch.empty((cfg.n_tokens, cfg.hidden), dtype=torch_dtype(cfg.out_dtype), device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, x.device)
    moe_forward(cfg, x, dev["w_router"], dev["gate_up"], dev["down"], dev.get("shared_gate_up"),
                dev.get("shared_down"), dev.get("w_shared_gate"), y, weights, experts, ws, stream=stream)
    return y
