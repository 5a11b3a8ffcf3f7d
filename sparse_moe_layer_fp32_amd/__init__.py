"""Sparse MoE block forward on one MI355X (gfx950): Python binding of the C ABI.

The block (router with bias, top-k, softmax over the selected logits, FP8
SwiGLU experts with biases, 128x128 block-scaled FP8, MXFP8 or MXFP4 weights,
weighted combine) runs in
HIP kernels of ``libsparse_moe.so``; this module only checks tensors and
passes device pointers and the current HIP stream (see ``include/moe.h``).
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_moe.so")

PATHS = {"auto": 0, "prefill": 1, "decode": 2}
ROUTINGS = {"topk_softmax": 0, "softmax_topk": 4}   # MOE_ROUTE_SOFTMAX_ALL
GATE_BF16 = 8                                       # MOE_GATE_BF16
FORMATS = {"block128": 0, "mx": 16, "mxfp4": 48}    # MOE_FORMAT_MX, MOE_FORMAT_MXFP4
MX_FORMATS = ("mx", "mxfp4")


def flags_of(path="auto", routing="topk_softmax", gate_bf16=False, fmt="block128") -> int:
    """The C ABI's `flags` word: GEMM path, gate-weight rule, bf16 gate weights,
    weight format."""
    return PATHS[path] | ROUTINGS[routing] | (GATE_BF16 if gate_bf16 else 0) | FORMATS[fmt]


BLOCK = 128
MX_BLOCK = 32
MAX_EXPERTS = 256
MAX_TOPK = 8

SYMBOLS = ("moe_workspace_bytes", "moe_forward", "moe_forward_ex", "moe_forward_mx",
           "moe_forward_stages", "moe_forward_debug", "moe_forward_noalloc", "moe_status_string",
           "attn_sink_prefill", "attn_sink_decode_workspace_bytes", "attn_sink_decode")
STAGES = {"router": 0, "scan": 1, "place": 2, "gateup": 3, "down": 4, "combine": 5}


class MoeError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, U, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    L.moe_workspace_bytes.restype = S
    L.moe_workspace_bytes.argtypes = [I, I, I, I, I]
    fwd = [P, P, P, I, P, P, P, P, P, P, P, I, I, I, I, P, S]
    L.moe_forward.restype = I
    L.moe_forward.argtypes = fwd + [P]
    L.moe_forward_ex.restype = I
    L.moe_forward_ex.argtypes = fwd + [U, P]
    L.moe_forward_mx.restype = I
    L.moe_forward_mx.argtypes = fwd + [U, P]
    L.moe_forward_stages.restype = I
    L.moe_forward_stages.argtypes = fwd + [U, I, I, P]
    L.moe_forward_debug.restype = I
    L.moe_forward_debug.argtypes = fwd + [U, P] + [P] * 10
    L.moe_forward_noalloc.restype = I
    L.moe_forward_noalloc.argtypes = fwd[:15] + [U, P]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [I]
    F = ctypes.c_float
    L.attn_sink_prefill.restype = I
    L.attn_sink_prefill.argtypes = [P, P, P, P, P, I, I, I, I, F, P]
    L.attn_sink_decode_workspace_bytes.restype = S
    L.attn_sink_decode_workspace_bytes.argtypes = [I, I, I]
    L.attn_sink_decode.restype = I
    L.attn_sink_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P, S, P]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise MoeError(status, status_string(status))


def workspace_bytes(T: int, d: int, f: int, E: int, k: int) -> int:
    return int(lib().moe_workspace_bytes(T, d, f, E, k))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name, shape, nbytes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.element_size() != nbytes:
        raise TypeError(f"{name} has {t.element_size()}-byte elements, expected {nbytes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device, stream, *tensors):
    """Raw handle of ``stream`` (default: the current stream).  Tensors allocated
    here on the current stream are recorded on a different target stream so
    the caching allocator does not reuse them before that stream is done."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    if stream is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(s)
    return ctypes.c_void_p(s.cuda_stream)


def scale_shapes(d, f, E, fmt="block128"):
    """(shape, element bytes) of S_gateup and S_down for a weight format."""
    if fmt in MX_FORMATS:
        return ((E, d // MX_BLOCK, 2 * f), 1), ((E, f // MX_BLOCK, d), 1)
    if fmt == "block128":
        return ((E, d // BLOCK, 2 * f // BLOCK), 4), ((E, f // BLOCK, d // BLOCK), 4)
    raise ValueError(f"unknown weight format {fmt!r}")


def _args(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down, b_down,
          out, workspace, fmt="block128", need_workspace=True):
    T, d = x.shape
    E = W_router.shape[1]
    f = W_down.shape[1] * (2 if fmt == "mxfp4" else 1)
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    _expect(x, "x", (T, d), 2, dev)
    _expect(W_router, "W_router", (d, E), 4, dev)
    _expect(b_router, "b_router", (E,), 4, dev)
    (sg_shape, sg_bytes), (sd_shape, sd_bytes) = scale_shapes(d, f, E, fmt)
    kp = 2 if fmt == "mxfp4" else 1                  # K rows per stored byte row
    _expect(W_gateup, "W_gateup", (E, d // kp, 2 * f), 1, dev)
    _expect(S_gateup, "S_gateup", sg_shape, sg_bytes, dev)
    _expect(b_gateup, "b_gateup", (E, 2 * f), 2, dev)
    _expect(W_down, "W_down", (E, f // kp, d), 1, dev)
    _expect(S_down, "S_down", sd_shape, sd_bytes, dev)
    _expect(b_down, "b_down", (E, d), 2, dev)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", (T, d), 2, dev)
    if need_workspace and workspace is None:
        workspace = torch.empty(max(workspace_bytes(T, d, f, E, k), 1), dtype=torch.uint8, device=dev)
    args = [_ptr(x), _ptr(W_router), _ptr(b_router), int(k), _ptr(W_gateup), _ptr(S_gateup),
            _ptr(b_gateup), _ptr(W_down), _ptr(S_down), _ptr(b_down), _ptr(out), T, d, f, E,
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()]
    return args, out, workspace, (T, d, f, E)


def forward(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down, b_down,
            out=None, workspace=None, path="auto", stream=None, routing="topk_softmax",
            gate_bf16=False, fmt="block128"):
    """bf16 [T, d] output of the block; every argument is a device tensor laid
    out as ``include/moe.h`` states (bf16 tensors may be any 2-byte dtype,
    e4m3 and E8M0 tensors any 1-byte dtype).  ``fmt="mx"`` takes MXFP8
    weights (E8M0 scales per 32 K rows) and ``fmt="mxfp4"`` MXFP4 weights (two
    E2M1 codes per byte along K) through ``moe_forward_mx``."""
    args, out, ws, _ = _args(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down,
                             S_down, b_down, out, workspace, fmt)
    entry = lib().moe_forward_mx if fmt in MX_FORMATS else lib().moe_forward_ex
    _check(entry(*args, flags_of(path, routing, gate_bf16, fmt), _stream(x.device, stream, ws, out)))
    return out


SCRATCH_BYTES = 64 << 20   # MOE_SCRATCH_BYTES


def forward_noalloc(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down, b_down,
                    out, path="auto", stream=None, routing="topk_softmax", gate_bf16=False,
                    fmt="block128"):
    """``forward`` through ``moe_forward_noalloc``: the library's static device
    scratch is the workspace, and the caller passes ``out`` (nothing is
    allocated here or in the library).  Raises MoeError (status -8) when the
    sizes need more than ``SCRATCH_BYTES`` of workspace."""
    if out is None:
        raise ValueError("forward_noalloc writes into a caller-provided `out`")
    args, out, _, _ = _args(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down,
                            S_down, b_down, out, None, fmt, need_workspace=False)
    _check(lib().moe_forward_noalloc(*args[:15], flags_of(path, routing, gate_bf16, fmt),
                                     _stream(x.device, stream, out)))
    return out


def forward_stages(first, last, x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down,
                   S_down, b_down, out, workspace, path="auto", stream=None, routing="topk_softmax",
                   gate_bf16=False, fmt="block128"):
    """Stages ``first``..``last`` (names of ``STAGES`` or ints) of ``forward`` on a
    caller-kept workspace; all stages must run in order on that workspace."""
    first = STAGES.get(first, first)
    last = STAGES.get(last, last)
    args, out, ws, _ = _args(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down,
                             S_down, b_down, out, workspace, fmt)
    _check(lib().moe_forward_stages(*args, flags_of(path, routing, gate_bf16, fmt), int(first), int(last),
                                    _stream(x.device, stream, ws, out)))
    return out


def forward_debug(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down, b_down,
                  path="auto", stream=None, routing="topk_softmax", gate_bf16=False,
                  fmt="block128"):
    """``forward`` plus the intermediates (routing, permutation, quantised
    activations and h, per-row expert outputs) as a dict of device tensors.
    MX: xs / hs are E8M0 codes [T, d/32] / [T*k, f/32]."""
    T, d = x.shape
    E, f = W_router.shape[1], W_down.shape[1] * (2 if fmt == "mxfp4" else 1)
    R = T * k
    dev = x.device
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    dbg = dict(topk_idx=torch.empty((T, k), dtype=i32, device=dev),
               topk_w=torch.empty((T, k), dtype=f32, device=dev),
               offsets=torch.empty(E + 1, dtype=i32, device=dev),
               row_token=torch.empty(R, dtype=i32, device=dev),
               row_of=torch.empty((T, k), dtype=i32, device=dev),
               xq=torch.empty((T, d), dtype=u8, device=dev),
               xs=(torch.empty((T, d // MX_BLOCK), dtype=u8, device=dev) if fmt in MX_FORMATS
                   else torch.empty((T, d // BLOCK), dtype=f32, device=dev)),
               hq=torch.empty((R, f), dtype=u8, device=dev),
               hs=(torch.empty((R, f // MX_BLOCK), dtype=u8, device=dev) if fmt in MX_FORMATS
                   else torch.empty((R, f // BLOCK), dtype=f32, device=dev)),
               y=torch.empty((R, d), dtype=f32, device=dev))
    args, out, ws, _ = _args(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down,
                             S_down, b_down, None, None, fmt)
    order = ["topk_idx", "topk_w", "offsets", "row_token", "row_of", "xq", "xs", "hq", "hs", "y"]
    _check(lib().moe_forward_debug(*args, flags_of(path, routing, gate_bf16, fmt),
                                   _stream(dev, stream, ws, out, *dbg.values()),
                                   *[_ptr(dbg[n]) for n in order]))
    dbg["out"] = out
    return dbg


def device_inputs(inp: dict, device="cuda"):
    """Host arrays of ``inputs.make_inputs`` -> device tensors in the C-ABI dtypes
    (the weight-format name under "fmt")."""
    import numpy as np

    def t(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to(device)

    fmt = inp.get("format", "block128")
    sdt = torch.uint8 if fmt in MX_FORMATS else torch.float32
    return dict(
        x=t(inp["x"], torch.bfloat16), W_router=t(inp["W_router"], torch.float32),
        b_router=t(inp["b_router"], torch.float32), k=int(inp["k"]),
        W_gateup=t(inp["W_gateup"], torch.uint8), S_gateup=t(inp["S_gateup"], sdt),
        b_gateup=t(inp["b_gateup"], torch.bfloat16), W_down=t(inp["W_down"], torch.uint8),
        S_down=t(inp["S_down"], sdt), b_down=t(inp["b_down"], torch.bfloat16), fmt=fmt)


class MoeBlock:
    """Device-resident layer parameters plus a reusable workspace."""

    def __init__(self, params: dict):
        self.p = {k: v for k, v in params.items() if k not in ("x", "fmt")}
        self.fmt = params.get("fmt", "block128")
        self._ws = None

    def workspace(self, T):
        p = self.p
        f = p["W_down"].shape[1] * (2 if self.fmt == "mxfp4" else 1)
        need = workspace_bytes(T, p["W_router"].shape[0], f, p["W_router"].shape[1], p["k"])
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=p["W_router"].device)
        return self._ws

    def __call__(self, x, out=None, path="auto", stream=None, routing="topk_softmax", gate_bf16=False):
        p = self.p
        return forward(x, p["W_router"], p["b_router"], p["k"], p["W_gateup"], p["S_gateup"],
                       p["b_gateup"], p["W_down"], p["S_down"], p["b_down"], out=out,
                       workspace=self.workspace(x.shape[0]), path=path, stream=stream,
                       routing=routing, gate_bf16=gate_bf16, fmt=self.fmt)


# ----------------------------------------------------------------------------- attention with sinks
def attn_prefill(q, k, v, sinks, sm_scale=None, out=None, stream=None):
    """Causal GQA attention with per-head sinks over one sequence
    (``include/attention.h``): q [S, Hq, D], k and v [S, Hkv, D] (2-byte
    dtypes, bf16 bits), sinks [Hq] fp32 -> out [S, Hq, D] bf16."""
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _expect(q, "q", (S, Hq, D), 2, dev)
    _expect(k, "k", (S, Hkv, D), 2, dev)
    _expect(v, "v", (S, Hkv, D), 2, dev)
    _expect(sinks, "sinks", (Hq,), 4, dev)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", (S, Hq, D), 2, dev)
    scale = float(1.0 / D ** 0.5 if sm_scale is None else sm_scale)
    _check(lib().attn_sink_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), S, Hq, Hkv, D,
                                   scale, _stream(dev, stream, out)))
    return out


def attn_decode_workspace_bytes(B, Hq, Lmax) -> int:
    return int(lib().attn_sink_decode_workspace_bytes(B, Hq, Lmax))


def attn_decode(q, k_cache, v_cache, kv_len, sinks, sm_scale=None, out=None, workspace=None,
                stream=None):
    """One query per sequence over an HND KV cache: q [B, Hq, D], caches
    [B, Hkv, Lmax, D], kv_len [B] int32, sinks [Hq] fp32 -> out [B, Hq, D] bf16."""
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    _expect(q, "q", (B, Hq, D), 2, dev)
    _expect(k_cache, "k_cache", (B, Hkv, Lmax, D), 2, dev)
    _expect(v_cache, "v_cache", (B, Hkv, Lmax, D), 2, dev)
    _expect(kv_len, "kv_len", (B,), 4, dev)
    _expect(sinks, "sinks", (Hq,), 4, dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", (B, Hq, D), 2, dev)
    need = attn_decode_workspace_bytes(B, Hq, Lmax)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    scale = float(1.0 / D ** 0.5 if sm_scale is None else sm_scale)
    _check(lib().attn_sink_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(sinks),
                                  _ptr(out), B, Hq, Hkv, D, Lmax, scale, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(dev, stream, out, workspace)))
    return out


def attn_device_inputs(inp: dict, device="cuda"):
    """Host arrays of ``inputs.make_attn_prefill`` / ``make_attn_decode`` -> device tensors."""
    import numpy as np

    def t(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to(device)

    d = dict(q=t(inp["q"], torch.bfloat16), k=t(inp["k"], torch.bfloat16), v=t(inp["v"], torch.bfloat16),
             sinks=t(inp["sinks"], torch.float32), sm_scale=inp["sm_scale"])
    if "kv_len" in inp:
        d["kv_len"] = t(inp["kv_len"], torch.int32)
    return d
