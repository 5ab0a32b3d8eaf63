"""Thin ctypes binding of libmoe_layer_03_amd.so on torch tensors.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions carry the C names; each takes a ``Shape`` and torch
tensors on the GPU, passes their data pointers and the current HIP stream,
and raises ``MoeError`` on a non-zero status.  Output tensors the caller
does not pass are allocated with torch (device memory only).

The library must be built (``moe_layer_03_amd.build``); loading fails loudly
otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

from . import build as _build

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_F32 = 0
MOE_BF16 = 1
MOE_F16 = 2
MOE_MXFP8 = 3

MOE_GEMM_GATE_UP = 0
MOE_GEMM_DOWN = 1
MOE_EPI_NONE = 0
MOE_EPI_SWIGLU = 1

EXPORTED = [
    "moe_dispatch_workspace_bytes", "moe_route_workspace_bytes", "moe_route_screen_layout",
    "moe_layer_workspace_bytes",
    "moe_packed_weight_bytes",
    "moe_pack_weights", "moe_route", "moe_route_from_logits", "moe_dispatch", "moe_grouped_gemm",
    "moe_combine", "moe_layer", "moe_status_string", "moe_last_hip_error",
    "moe_probe_mfma_bf16_flops", "moe_probe_mfma_bf16", "moe_layer_noalloc",
    "moe_packed_weight_bytes_mxfp8", "moe_pack_weights_mxfp8", "moe_quantize_mxfp8", "moe_grouped_gemm_mxfp8",
    "moe_layer_workspace_bytes_mxfp8", "moe_layer_mxfp8",
]

MOE_LAYER_NOALLOC_MAX_WS_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status}, hip error {hip_error})")
        self.status = status
        self.hip_error = hip_error


class _CShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "E", "K", "I", "e_begin", "e_end")]


class _CScreenInfo(ctypes.Structure):
    _fields_ = [("slices", ctypes.c_int32), ("part_offset", ctypes.c_size_t), ("nx_offset", ctypes.c_size_t),
                ("nw_offset", ctypes.c_size_t), ("bytes", ctypes.c_size_t)]


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    H: int
    E: int
    K: int
    I: int
    e_begin: int
    e_end: int

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    @property
    def cap(self) -> int:
        return self.T * min(self.K, self.E_loc)

    def c(self) -> _CShape:
        return _CShape(self.T, self.H, self.E, self.K, self.I, self.e_begin, self.e_end)

    @staticmethod
    def of(wl) -> "Shape":
        return Shape(wl.T, wl.H, wl.E, wl.K, wl.I, wl.e_begin, wl.e_end)


_lib = None
_P = ctypes.c_void_p
_S = ctypes.POINTER(_CShape)


def lib_path() -> str:
    """The in-tree library, or the file named by MOE_LAYER_03_AMD_LIB."""
    return os.environ.get("MOE_LAYER_03_AMD_LIB") or _build.LIB


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m moe_layer_03_amd.build` "
                          "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    sz = ctypes.c_size_t
    i32 = ctypes.c_int
    sigs = {
        "moe_dispatch_workspace_bytes": (sz, [_S]),
        "moe_route_workspace_bytes": (sz, [_S]),
        "moe_route_screen_layout": (i32, [_S, i32, i32, ctypes.POINTER(_CScreenInfo)]),
        "moe_layer_workspace_bytes": (sz, [_S]),
        "moe_packed_weight_bytes": (sz, [_S]),
        "moe_pack_weights": (i32, [_S, _P, _P, _P, i32, _P, _P]),
        "moe_route": (i32, [_S, _P, i32, _P, i32, _P, _P, _P, _P, _P, sz, _P]),
        "moe_route_from_logits": (i32, [_S, _P, _P, _P, _P]),
        "moe_dispatch": (i32, [_S, _P, _P, i32, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "moe_grouped_gemm": (i32, [_S, _P, i32, _P, _P, _P, i32, i32, _P, i32, _P]),
        "moe_combine": (i32, [_S, _P, i32, _P, _P, _P, _P]),
        "moe_layer": (i32, [_S, _P, i32, _P, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_last_hip_error": (ctypes.c_int32, []),
        "moe_layer_noalloc": (i32, [_S, _P, i32, _P, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "moe_packed_weight_bytes_mxfp8": (sz, [_S]),
        "moe_pack_weights_mxfp8": (i32, [_S, _P, _P, _P, i32, _P, _P]),
        "moe_quantize_mxfp8": (i32, [ctypes.c_int64, ctypes.c_int32, _P, i32, _P, _P, _P]),
        "moe_grouped_gemm_mxfp8": (i32, [_S, _P, _P, _P, _P, _P, i32, i32, _P, i32, _P, _P]),
        "moe_layer_workspace_bytes_mxfp8": (sz, [_S]),
        "moe_layer_mxfp8": (i32, [_S, _P, i32, _P, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "moe_probe_mfma_bf16_flops": (ctypes.c_int64, [i32, i32]),
        "moe_probe_mfma_bf16": (i32, [i32, i32, _P, _P]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        lib = load()
        raise MoeError(fn, status, int(lib.moe_last_hip_error()), lib.moe_status_string(status).decode())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.float16:
        return MOE_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, numel=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr() or None


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def operand_dtype(x_dtype: torch.dtype) -> torch.dtype:
    """GEMM operand type of a layer whose inputs have dtype x_dtype."""
    return torch.bfloat16 if x_dtype == torch.bfloat16 else torch.float16


def _empty(n, dtype, device):
    return torch.empty(n, dtype=dtype, device=device)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def moe_dispatch_workspace_bytes(s: Shape) -> int:
    return int(load().moe_dispatch_workspace_bytes(ctypes.byref(s.c())))


def moe_route_workspace_bytes(s: Shape) -> int:
    return int(load().moe_route_workspace_bytes(ctypes.byref(s.c())))


def moe_route_screen_layout(s: Shape, x_dtype: int = MOE_BF16, w_dtype: int = MOE_BF16) -> dict:
    """Offsets of the screened router's estimates in its workspace (see the C header)."""
    info = _CScreenInfo()
    st = load().moe_route_screen_layout(ctypes.byref(s.c()), x_dtype, w_dtype, ctypes.byref(info))
    _check("moe_route_screen_layout", st)
    return dict(slices=int(info.slices), part_offset=int(info.part_offset), nx_offset=int(info.nx_offset),
                nw_offset=int(info.nw_offset), bytes=int(info.bytes))


def moe_layer_workspace_bytes(s: Shape) -> int:
    return int(load().moe_layer_workspace_bytes(ctypes.byref(s.c())))


def moe_packed_weight_bytes(s: Shape) -> int:
    return int(load().moe_packed_weight_bytes(ctypes.byref(s.c())))


def moe_pack_weights(s: Shape, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                     packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack [E_loc,H,I], [E_loc,H,I], [E_loc,I,H] weights (fp32 or bf16) into the GEMM layout."""
    n = s.E_loc * s.H * s.I
    dt = w_gate.dtype
    need = moe_packed_weight_bytes(s)
    if packed is None:
        packed = _empty(need, torch.uint8, w_gate.device)
    if packed.dtype != torch.uint8 or packed.numel() < need:
        raise ValueError(f"packed must be a uint8 buffer of at least {need} bytes")
    st = load().moe_pack_weights(ctypes.byref(s.c()), _ptr(w_gate, dt, n, "w_gate"), _ptr(w_up, dt, n, "w_up"),
                                 _ptr(w_down, dt, n, "w_down"), _dt(w_gate), _ptr(packed, torch.uint8, None, "packed"),
                                 _stream(stream))
    _check("moe_pack_weights", st)
    return packed


def moe_route(s: Shape, x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor] = None,
              topk_idx=None, topk_w=None, logits=None, want_logits=False, ws=None, screened=True, stream=None):
    """Returns (topk_idx int32 [T,K], topk_w fp32 [T,K], logits fp32 [T,E] or None).

    ``screened=False`` passes no workspace, so (without logits requested) the
    library takes its per-token form; with the default it passes a workspace of
    ``moe_route_workspace_bytes`` and the library screens large bf16 batches or
    tiles small ones when the shape allows it (the outputs are the same)."""
    dev = x.device
    if topk_idx is None:
        topk_idx = _empty((s.T, s.K), torch.int32, dev)
    if topk_w is None:
        topk_w = _empty((s.T, s.K), torch.float32, dev)
    if logits is None and want_logits:
        logits = _empty((s.T, s.E), torch.float32, dev)
    if not screened:
        ws = None
    elif ws is None:
        need = moe_route_workspace_bytes(s)
        ws = _empty(need, torch.uint8, dev) if need > 0 else None
    st = load().moe_route(ctypes.byref(s.c()), _ptr(x, None, s.T * s.H, "x"), _dt(x),
                          _ptr(w_router, None, s.H * s.E, "w_router"), _dt(w_router),
                          _ptr(bias, torch.float32, s.E, "bias"), _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                          _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"),
                          _ptr(logits, torch.float32, s.T * s.E, "logits"),
                          _ptr(ws, torch.uint8, None, "ws"), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_route", st)
    return topk_idx, topk_w, logits


def moe_route_from_logits(s: Shape, logits: torch.Tensor, topk_idx=None, topk_w=None, stream=None):
    dev = logits.device
    if topk_idx is None:
        topk_idx = _empty((s.T, s.K), torch.int32, dev)
    if topk_w is None:
        topk_w = _empty((s.T, s.K), torch.float32, dev)
    st = load().moe_route_from_logits(ctypes.byref(s.c()), _ptr(logits, torch.float32, s.T * s.E, "logits"),
                                      _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                                      _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"), _stream(stream))
    _check("moe_route_from_logits", st)
    return topk_idx, topk_w


def moe_dispatch(s: Shape, topk_idx: torch.Tensor, x: Optional[torch.Tensor] = None, *, counts=None, offsets=None,
                 row_token=None, row_slot=None, slot_row=None, x_packed=None, ws=None, stream=None):
    """Returns dict(counts, offsets, row_token, row_slot, slot_row, x_packed)."""
    dev = topk_idx.device
    cap = s.cap
    counts = _empty(s.E_loc, torch.int32, dev) if counts is None else counts
    offsets = _empty(s.E_loc + 1, torch.int32, dev) if offsets is None else offsets
    row_token = _empty(cap, torch.int32, dev) if row_token is None else row_token
    row_slot = _empty(cap, torch.int32, dev) if row_slot is None else row_slot
    slot_row = _empty((s.T, s.K), torch.int32, dev) if slot_row is None else slot_row
    if x is not None and x_packed is None:
        x_packed = _empty((cap, s.H), operand_dtype(x.dtype), dev)
    need = moe_dispatch_workspace_bytes(s)
    if ws is None:
        ws = _empty(max(need, 16), torch.uint8, dev)
    st = load().moe_dispatch(ctypes.byref(s.c()), _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                             _ptr(x, None, s.T * s.H, "x"), _dt(x) if x is not None else MOE_BF16,
                             _ptr(counts, torch.int32, s.E_loc, "counts"),
                             _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                             _ptr(row_token, torch.int32, cap, "row_token"),
                             _ptr(row_slot, torch.int32, cap, "row_slot"),
                             _ptr(slot_row, torch.int32, s.T * s.K, "slot_row"),
                             _ptr(x_packed, operand_dtype(x.dtype) if x is not None else None, cap * s.H,
                                  "x_packed"),
                             _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_dispatch", st)
    return dict(counts=counts, offsets=offsets, row_token=row_token, row_slot=row_slot, slot_row=slot_row,
                x_packed=x_packed)


def moe_grouped_gemm(s: Shape, a: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor, which: int,
                     epilogue: int = MOE_EPI_NONE, c=None, c_dtype=torch.float16, a_rows=None,
                     stream=None) -> torch.Tensor:
    """a: bf16/fp16 packed rows [cap, Kd], or the unpacked input with a_rows [cap] int32 (row gather)."""
    cap = s.cap
    kd = s.H if which == MOE_GEMM_GATE_UP else s.I
    if which == MOE_GEMM_GATE_UP:
        nc = s.I if epilogue == MOE_EPI_SWIGLU else 2 * s.I
    else:
        nc = s.H
    if c is None:
        c = _empty((cap, nc), c_dtype, a.device)
    if a_rows is None and a.numel() != cap * kd:
        raise ValueError(f"a must have {cap * kd} elements without a_rows")
    if a.numel() % kd:
        raise ValueError("a rows must have the reduction length")
    st = load().moe_grouped_gemm(ctypes.byref(s.c()), _ptr(a, None, None, "a"), _dt(a),
                                 _ptr(a_rows, torch.int32, cap, "a_rows"),
                                 _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                                 _ptr(packed, torch.uint8, None, "packed"), which, epilogue,
                                 _ptr(c, None, cap * nc, "c"), _dt(c), _stream(stream))
    _check("moe_grouped_gemm", st)
    return c


def moe_combine(s: Shape, y_packed: torch.Tensor, slot_row: torch.Tensor, topk_w: torch.Tensor, out=None,
                stream=None) -> torch.Tensor:
    if out is None:
        out = _empty((s.T, s.H), torch.float32, y_packed.device)
    st = load().moe_combine(ctypes.byref(s.c()), _ptr(y_packed, None, s.cap * s.H, "y_packed"), _dt(y_packed),
                            _ptr(slot_row, torch.int32, s.T * s.K, "slot_row"),
                            _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"),
                            _ptr(out, torch.float32, s.T * s.H, "out"), _stream(stream))
    _check("moe_combine", st)
    return out


def moe_layer(s: Shape, x: torch.Tensor, w_router: torch.Tensor, packed: torch.Tensor,
              bias: Optional[torch.Tensor] = None, out=None, ws=None, *, topk_idx=None, topk_w=None, counts=None,
              offsets=None, row_token=None, row_slot=None, slot_row=None, stream=None) -> torch.Tensor:
    """The fused layer share; optional routing/dispatch outputs are written when given."""
    if out is None:
        out = _empty((s.T, s.H), torch.float32, x.device)
    if ws is None:
        ws = _empty(max(moe_layer_workspace_bytes(s), 16), torch.uint8, x.device)
    cap = s.cap
    st = load().moe_layer(ctypes.byref(s.c()), _ptr(x, None, s.T * s.H, "x"), _dt(x),
                          _ptr(w_router, None, s.H * s.E, "w_router"), _dt(w_router),
                          _ptr(bias, torch.float32, s.E, "bias"), _ptr(packed, torch.uint8, None, "packed"),
                          _ptr(out, torch.float32, s.T * s.H, "out"),
                          _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                          _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"),
                          _ptr(counts, torch.int32, s.E_loc, "counts"),
                          _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                          _ptr(row_token, torch.int32, cap, "row_token"), _ptr(row_slot, torch.int32, cap, "row_slot"),
                          _ptr(slot_row, torch.int32, s.T * s.K, "slot_row"),
                          _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_layer", st)
    return out


def moe_layer_noalloc(s: Shape, x: torch.Tensor, w_router: torch.Tensor, packed: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, out=None, *, topk_idx=None, topk_w=None, counts=None,
                      offsets=None, row_token=None, row_slot=None, slot_row=None, stream=None) -> torch.Tensor:
    """moe_layer with the library's static per-GPU workspace (the C call allocates nothing)."""
    if out is None:
        out = _empty((s.T, s.H), torch.float32, x.device)
    cap = s.cap
    st = load().moe_layer_noalloc(ctypes.byref(s.c()), _ptr(x, None, s.T * s.H, "x"), _dt(x),
                                  _ptr(w_router, None, s.H * s.E, "w_router"), _dt(w_router),
                                  _ptr(bias, torch.float32, s.E, "bias"), _ptr(packed, torch.uint8, None, "packed"),
                                  _ptr(out, torch.float32, s.T * s.H, "out"),
                                  _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                                  _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"),
                                  _ptr(counts, torch.int32, s.E_loc, "counts"),
                                  _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                                  _ptr(row_token, torch.int32, cap, "row_token"),
                                  _ptr(row_slot, torch.int32, cap, "row_slot"),
                                  _ptr(slot_row, torch.int32, s.T * s.K, "slot_row"), _stream(stream))
    _check("moe_layer_noalloc", st)
    return out


def moe_probe_mfma_bf16(blocks: int, iters: int, sink: torch.Tensor, stream=None) -> int:
    """Launch the MFMA rate probe; returns the FLOPs of the launch (measurement helper)."""
    if sink.numel() < blocks * 512:
        raise ValueError("sink needs blocks * 512 floats")
    st = load().moe_probe_mfma_bf16(blocks, iters, _ptr(sink, torch.float32, None, "sink"), _stream(stream))
    _check("moe_probe_mfma_bf16", st)
    return int(load().moe_probe_mfma_bf16_flops(blocks, iters))


# ---------------------------------------------------------------------------
# MXFP8 (OCP microscaling, E4M3 codes + E8M0 scale per 32 along K)
# ---------------------------------------------------------------------------

def moe_packed_weight_bytes_mxfp8(s: Shape) -> int:
    return int(load().moe_packed_weight_bytes_mxfp8(ctypes.byref(s.c())))


def moe_pack_weights_mxfp8(s: Shape, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                           packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n = s.E_loc * s.H * s.I
    dt = w_gate.dtype
    need = moe_packed_weight_bytes_mxfp8(s)
    if need == 0:
        raise MoeError("moe_packed_weight_bytes_mxfp8", MOE_ERR_UNSUPPORTED, 0, "shape not supported for MXFP8")
    if packed is None:
        packed = _empty(need, torch.uint8, w_gate.device)
    st = load().moe_pack_weights_mxfp8(ctypes.byref(s.c()), _ptr(w_gate, dt, n, "w_gate"), _ptr(w_up, dt, n, "w_up"),
                                       _ptr(w_down, dt, n, "w_down"), _dt(w_gate),
                                       _ptr(packed, torch.uint8, None, "packed"), _stream(stream))
    _check("moe_pack_weights_mxfp8", st)
    return packed


def moe_quantize_mxfp8(x: torch.Tensor, codes=None, scales=None, stream=None):
    """x [rows, K] bf16/fp32 -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    rows, K = x.shape
    if codes is None:
        codes = _empty((rows, K), torch.uint8, x.device)
    if scales is None:
        scales = _empty((rows, K // 32), torch.uint8, x.device)
    st = load().moe_quantize_mxfp8(rows, K, _ptr(x, None, rows * K, "x"), _dt(x),
                                   _ptr(codes, torch.uint8, rows * K, "codes"),
                                   _ptr(scales, torch.uint8, rows * (K // 32), "scales"), _stream(stream))
    _check("moe_quantize_mxfp8", st)
    return codes, scales


def moe_grouped_gemm_mxfp8(s: Shape, a: torch.Tensor, a_scales: torch.Tensor, offsets: torch.Tensor,
                           packed: torch.Tensor, which: int, epilogue: int = MOE_EPI_NONE, c=None,
                           c_dtype=torch.float16, c_scales=None, a_rows=None, stream=None):
    """MXFP8 grouped GEMM.  c_dtype torch.uint8 means MXFP8 output (SwiGLU only):
    returns (codes [cap, I], scales [cap, I/32]); otherwise returns c."""
    cap = s.cap
    kd = s.H if which == MOE_GEMM_GATE_UP else s.I
    if which == MOE_GEMM_GATE_UP:
        nc = s.I if epilogue == MOE_EPI_SWIGLU else 2 * s.I
    else:
        nc = s.H
    mx_out = c_dtype == torch.uint8
    if c is None:
        c = _empty((cap, nc), c_dtype, a.device)
    if mx_out and c_scales is None:
        c_scales = _empty((cap, nc // 32), torch.uint8, a.device)
    if a.numel() % kd or a_scales.numel() * 32 != a.numel():
        raise ValueError("a [rows, K] codes with a_scales [rows, K/32]")
    st = load().moe_grouped_gemm_mxfp8(ctypes.byref(s.c()), _ptr(a, torch.uint8, None, "a"),
                                       _ptr(a_scales, torch.uint8, None, "a_scales"),
                                       _ptr(a_rows, torch.int32, cap, "a_rows"),
                                       _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                                       _ptr(packed, torch.uint8, None, "packed"), which, epilogue,
                                       _ptr(c, None, cap * nc, "c"), MOE_MXFP8 if mx_out else _dt(c),
                                       _ptr(c_scales, torch.uint8, None, "c_scales") if mx_out else None,
                                       _stream(stream))
    _check("moe_grouped_gemm_mxfp8", st)
    return (c, c_scales) if mx_out else c


def moe_layer_workspace_bytes_mxfp8(s: Shape) -> int:
    return int(load().moe_layer_workspace_bytes_mxfp8(ctypes.byref(s.c())))


def moe_layer_mxfp8(s: Shape, x: torch.Tensor, w_router: torch.Tensor, packed: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, out=None, ws=None, *, topk_idx=None, topk_w=None,
                    counts=None, offsets=None, row_token=None, row_slot=None, slot_row=None,
                    stream=None) -> torch.Tensor:
    """The layer share with MXFP8 expert GEMMs (packed from moe_pack_weights_mxfp8)."""
    if out is None:
        out = _empty((s.T, s.H), torch.float32, x.device)
    if ws is None:
        ws = _empty(max(moe_layer_workspace_bytes_mxfp8(s), 16), torch.uint8, x.device)
    cap = s.cap
    st = load().moe_layer_mxfp8(ctypes.byref(s.c()), _ptr(x, None, s.T * s.H, "x"), _dt(x),
                                _ptr(w_router, None, s.H * s.E, "w_router"), _dt(w_router),
                                _ptr(bias, torch.float32, s.E, "bias"), _ptr(packed, torch.uint8, None, "packed"),
                                _ptr(out, torch.float32, s.T * s.H, "out"),
                                _ptr(topk_idx, torch.int32, s.T * s.K, "topk_idx"),
                                _ptr(topk_w, torch.float32, s.T * s.K, "topk_w"),
                                _ptr(counts, torch.int32, s.E_loc, "counts"),
                                _ptr(offsets, torch.int32, s.E_loc + 1, "offsets"),
                                _ptr(row_token, torch.int32, cap, "row_token"),
                                _ptr(row_slot, torch.int32, cap, "row_slot"),
                                _ptr(slot_row, torch.int32, s.T * s.K, "slot_row"),
                                _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_layer_mxfp8", st)
    return out
