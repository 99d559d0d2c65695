"""ctypes binding of libfp4moe.so (the C ABI in include/fp4moe.h).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  torch provides device memory and the current HIP stream.  There is
no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4moe.so")

FMT = {"nvfp4": 0, "mxfp4": 1, "mxfp8": 2, "fp8_block": 3, "fp8_row": 4, "none": 5}
RULE = {"rtn": 0, "4over6": 1, "sweep": 2}
TS_DYNAMIC, TS_STATIC = 0, 1
DT_BF16, DT_F32 = 0, 1
STATUS = {0: "FP4_OK", -1: "FP4_ERR_INVALID_ARG", -2: "FP4_ERR_SHAPE",
          -3: "FP4_ERR_UNSUPPORTED", -4: "FP4_ERR_WORKSPACE", -5: "FP4_ERR_HIP"}

EXPORTED = ["fp4_quantize", "fp4_quantize_hessian", "fp4_dequantize", "fp4_block_error", "moe_fp4_workspace_layout",
            "moe_fp4_workspace_size", "moe_fp4_forward", "moe_fp4_forward_profiled",
            "moe_fp4_route", "moe_fp4_tile_weights", "moe_fp4_forward_noalloc", "fp4_status_string",
            "fp4_last_error"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # FP4_NOALLOC_SCRATCH_BYTES
STAGES = ["permute", "x_quant", "gate_up", "h_quant", "down", "shared", "combine"]


class Fp4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class LayerStruct(ctypes.Structure):
    _fields_ = [
        ("w_fmt", ctypes.c_int32), ("a_fmt", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w13_scale_2", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("w2_scale_2", ctypes.c_void_p),
        ("input_scale", ctypes.c_void_p), ("inter_scale", ctypes.c_void_p),
        ("shared_inter", ctypes.c_int32),
        ("ws13", ctypes.c_void_p), ("ws13_scale", ctypes.c_void_p),
        ("ws2", ctypes.c_void_p), ("ws2_scale", ctypes.c_void_p),
        ("shared_gate", ctypes.c_void_p),
        ("w13_tiled", ctypes.c_void_p), ("w13_scale_tiled", ctypes.c_void_p),
        ("w2_tiled", ctypes.c_void_p), ("w2_scale_tiled", ctypes.c_void_p),
    ]


class WsLayoutStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total", "error_flag", "counts", "offsets", "pair_of_row", "row_of_pair",
        "x_tensor_scale", "h_tensor_scale", "h", "hq_codes", "hq_scales", "o")]


_lib = None


def lib():
    """Load libfp4moe.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run "
                              "`python -m block_scaled_fp4_nvfp4_amd.build` first")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.fp4_quantize.argtypes = [i32, i32, i32, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
        L.fp4_quantize.restype = i32
        L.fp4_quantize_hessian.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.fp4_quantize_hessian.restype = i32
        L.fp4_dequantize.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp, i32, vp]
        L.fp4_dequantize.restype = i32
        L.fp4_block_error.argtypes = [i32, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
        L.fp4_block_error.restype = i32
        L.moe_fp4_workspace_layout.argtypes = [ctypes.POINTER(LayerStruct), i64, ctypes.POINTER(WsLayoutStruct)]
        L.moe_fp4_workspace_layout.restype = i32
        L.moe_fp4_workspace_size.argtypes = [ctypes.POINTER(LayerStruct), i64, ctypes.POINTER(sz)]
        L.moe_fp4_workspace_size.restype = i32
        L.moe_fp4_forward.argtypes = [ctypes.POINTER(LayerStruct), vp, i64, vp, vp, vp, vp, sz, vp]
        L.moe_fp4_forward.restype = i32
        L.moe_fp4_forward_profiled.argtypes = [ctypes.POINTER(LayerStruct), vp, i64, vp, vp, vp, vp, sz, vp,
                                               ctypes.POINTER(vp), i32]
        L.moe_fp4_forward_profiled.restype = i32
        L.moe_fp4_forward_noalloc.argtypes = [ctypes.POINTER(LayerStruct), vp, i64, vp, vp, vp, vp]
        L.moe_fp4_forward_noalloc.restype = i32
        L.moe_fp4_route.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        L.moe_fp4_route.restype = i32
        L.moe_fp4_tile_weights.argtypes = [i32, vp, vp, i64, i64, i64, vp, vp, vp]
        L.moe_fp4_tile_weights.restype = i32
        L.fp4_status_string.argtypes = [i32]
        L.fp4_status_string.restype = ctypes.c_char_p
        L.fp4_last_error.argtypes = []
        L.fp4_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise Fp4Error(status, lib().fp4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dims(x: torch.Tensor):
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape
    raise ValueError("expected [rows, cols] or [batch, rows, cols]")


def quantize(x: torch.Tensor, fmt: str, rule: str = "4over6",
             tensor_scale: Optional[torch.Tensor] = None, want_m4: bool = False):
    """fp4_quantize.  x: contiguous bf16/f32 device tensor [rows, cols] or
    [batch, rows, cols].  Returns dict(codes, scales, tensor_scale, m4)."""
    assert x.is_cuda and x.is_contiguous()
    b, r, c = (int(v) for v in _dims(x))
    dev = x.device
    f = FMT[fmt]
    lead = x.shape[:-1]
    if fmt in ("nvfp4", "mxfp4"):
        codes = torch.empty(*lead, c // 2, dtype=torch.uint8, device=dev)
    else:
        codes = torch.empty(*lead, c, dtype=torch.uint8, device=dev)
    bs = {"nvfp4": 16, "mxfp4": 32, "mxfp8": 32}.get(fmt)
    if bs is not None:
        scales = torch.empty(*lead, max(c // bs, 0), dtype=torch.uint8, device=dev)
    elif fmt == "fp8_row":
        scales = torch.empty(*lead, c // 128, dtype=torch.float32, device=dev)
    else:
        scales = torch.empty(*x.shape[:-2], r // 128, c // 128, dtype=torch.float32, device=dev)
    ts_mode = TS_DYNAMIC
    ts = None
    if fmt == "nvfp4":
        if tensor_scale is None:
            ts = torch.empty(b, dtype=torch.float32, device=dev)
        else:
            ts = tensor_scale.to(device=dev, dtype=torch.float32).reshape(b).contiguous()
            ts_mode = TS_STATIC
    m4 = None
    if want_m4 and bs is not None and fmt != "mxfp8":
        m4 = torch.empty(*lead, c // bs, dtype=torch.uint8, device=dev)
    _check(lib().fp4_quantize(f, RULE[rule], ts_mode, _ptr(x), _dtype_code(x), b, r, c,
                              _ptr(codes), _ptr(scales), _ptr(ts), _ptr(m4), _stream()))
    return {"codes": codes, "scales": scales, "tensor_scale": ts, "m4": m4}


def quantize_hessian(x: torch.Tensor, hessian: torch.Tensor, calib_rows: torch.Tensor,
                     want_choice: bool = False):
    """fp4_quantize_hessian.  x: contiguous bf16/f32 device tensor [E, rows,
    cols] (or [rows, cols] for one expert); hessian: f32 [E, cols/16, 16, 16];
    calib_rows: int32 [E].  Returns dict(codes, scales, tensor_scale, choice)
    in the NVFP4 layout of quantize()."""
    assert x.is_cuda and x.is_contiguous()
    b, r, c = (int(v) for v in _dims(x))
    dev = x.device
    hessian = hessian.to(device=dev, dtype=torch.float32).contiguous()
    calib_rows = calib_rows.to(device=dev, dtype=torch.int32).contiguous()
    assert hessian.numel() == b * (c // 16) * 256 and calib_rows.numel() == b
    lead = x.shape[:-1]
    codes = torch.empty(*lead, c // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(*lead, c // 16, dtype=torch.uint8, device=dev)
    ts = torch.empty(b, dtype=torch.float32, device=dev)
    choice = torch.empty(*lead, c // 16, dtype=torch.uint8, device=dev) if want_choice else None
    _check(lib().fp4_quantize_hessian(_ptr(x), _dtype_code(x), b, r, c, _ptr(hessian), _ptr(calib_rows),
                                      _ptr(codes), _ptr(scales), _ptr(ts), _ptr(choice), _stream()))
    return {"codes": codes, "scales": scales, "tensor_scale": ts, "choice": choice}


def route(logits: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None):
    """moe_fp4_route.  logits: contiguous f32 device tensor [T, E]; bias: f32
    [E] or None.  Returns (topk_ids int32 [T, k], topk_weights f32 [T, k])."""
    assert logits.is_cuda and logits.is_contiguous() and logits.dtype == torch.float32 and logits.dim() == 2
    T, E = (int(v) for v in logits.shape)
    if bias is not None:
        bias = bias.to(device=logits.device, dtype=torch.float32).contiguous()
        assert bias.numel() == E
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _check(lib().moe_fp4_route(_ptr(logits), _ptr(bias), T, E, k, _ptr(ids), _ptr(w), _stream()))
    return ids, w


def block_error(x: torch.Tensor, q: dict, fmt: str) -> torch.Tensor:
    """fp4_block_error: f32 squared error of every block of x's quantization
    q (a record from quantize(), NVFP4 or MXFP4), shape x.shape[:-1] +
    (cols / block,)."""
    bs = 16 if fmt == "nvfp4" else 32
    b, r, c = (int(v) for v in _dims(x))
    err = torch.empty(*x.shape[:-1], x.shape[-1] // bs, dtype=torch.float32, device=x.device)
    _check(lib().fp4_block_error(FMT[fmt], _ptr(x), _dtype_code(x), b, r, c, _ptr(q["codes"]), _ptr(q["scales"]),
                                 _ptr(q.get("tensor_scale")), _ptr(err), _stream()))
    return err


def tile_weights(codes: torch.Tensor, scales: Optional[torch.Tensor], fmt: str = "mxfp4"):
    """moe_fp4_tile_weights.  NVFP4 / MXFP4: codes uint8 [E, rows, cols/2],
    scales [E, rows, cols/16] (E4M3) / [E, rows, cols/32] (UE8M0); block FP8
    ("fp8_block"): codes uint8 [E, rows, cols], scales unused.  Contiguous
    device tensors.  Returns the tiled (codes, scales) for MoELayer.w13_tiled /
    w13_scale_tiled (or w2_tiled / w2_scale_tiled); scales None for block FP8."""
    assert codes.is_cuda and codes.is_contiguous() and codes.dim() == 3
    E, rows, width = (int(v) for v in codes.shape)
    fp4 = fmt in ("nvfp4", "mxfp4")
    cols = 2 * width if fp4 else width
    tc = torch.empty_like(codes)
    ts = torch.empty_like(scales) if fp4 else None
    _check(lib().moe_fp4_tile_weights(FMT[fmt], _ptr(codes), _ptr(scales) if fp4 else None, E, rows, cols,
                                      _ptr(tc), _ptr(ts), _stream()))
    return tc, ts


def dequantize(q: dict, fmt: str, shape, out_dtype=torch.float32) -> torch.Tensor:
    """fp4_dequantize of a record produced by quantize(); shape = x's shape."""
    codes = q["codes"]
    out = torch.empty(*shape, dtype=out_dtype, device=codes.device)
    b, r, c = (int(v) for v in _dims(out))
    _check(lib().fp4_dequantize(FMT[fmt], _ptr(codes), _ptr(q["scales"]), _ptr(q.get("tensor_scale")),
                                b, r, c, _ptr(out), _dtype_code(out), _stream()))
    return out


@dataclasses.dataclass
class MoELayer:
    """Device tensors of one routed-expert layer (see moe_fp4_layer)."""
    w_fmt: str
    a_fmt: str
    num_experts: int
    hidden: int
    inter: int
    top_k: int
    w13: torch.Tensor
    w13_scale: torch.Tensor
    w2: torch.Tensor
    w2_scale: torch.Tensor
    w13_scale_2: Optional[torch.Tensor] = None
    w2_scale_2: Optional[torch.Tensor] = None
    input_scale: Optional[torch.Tensor] = None
    inter_scale: Optional[torch.Tensor] = None
    shared_inter: int = 0
    ws13: Optional[torch.Tensor] = None
    ws13_scale: Optional[torch.Tensor] = None
    ws2: Optional[torch.Tensor] = None
    ws2_scale: Optional[torch.Tensor] = None
    shared_gate: Optional[torch.Tensor] = None
    w13_tiled: Optional[torch.Tensor] = None
    w13_scale_tiled: Optional[torch.Tensor] = None
    w2_tiled: Optional[torch.Tensor] = None
    w2_scale_tiled: Optional[torch.Tensor] = None

    def struct(self) -> LayerStruct:
        p = lambda t: None if t is None else t.data_ptr()
        return LayerStruct(
            FMT[self.w_fmt], FMT[self.a_fmt], self.num_experts, self.hidden, self.inter, self.top_k,
            p(self.w13), p(self.w13_scale), p(self.w13_scale_2),
            p(self.w2), p(self.w2_scale), p(self.w2_scale_2),
            p(self.input_scale), p(self.inter_scale), self.shared_inter,
            p(self.ws13), p(self.ws13_scale), p(self.ws2), p(self.ws2_scale), p(self.shared_gate),
            p(self.w13_tiled), p(self.w13_scale_tiled), p(self.w2_tiled), p(self.w2_scale_tiled))


def workspace_layout(layer: MoELayer, tokens: int) -> dict:
    s = layer.struct()
    out = WsLayoutStruct()
    _check(lib().moe_fp4_workspace_layout(ctypes.byref(s), tokens, ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in WsLayoutStruct._fields_}


def workspace_size(layer: MoELayer, tokens: int) -> int:
    s = layer.struct()
    n = ctypes.c_size_t()
    _check(lib().moe_fp4_workspace_size(ctypes.byref(s), tokens, ctypes.byref(n)))
    return n.value


def moe_forward(layer: MoELayer, x: torch.Tensor, topk_ids: torch.Tensor,
                topk_weights: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_fp4_forward: x bf16 [T, H], topk_ids int32 [T, k], topk_weights f32 [T, k] -> y f32 [T, H]."""
    T = int(x.shape[0])
    if y is None:
        y = torch.empty(T, layer.hidden, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(layer, T), 1), dtype=torch.uint8, device=x.device)
    s = layer.struct()
    _check(lib().moe_fp4_forward(ctypes.byref(s), _ptr(x), T, _ptr(topk_ids), _ptr(topk_weights),
                                 _ptr(y), _ptr(workspace), workspace.numel(), _stream()))
    return y


def moe_forward_noalloc(layer: MoELayer, x: torch.Tensor, topk_ids: torch.Tensor,
                        topk_weights: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_fp4_forward_noalloc: moe_forward with the library's per-device
    scratch as the workspace (nothing allocated by the call; y is allocated
    here only when not given)."""
    T = int(x.shape[0])
    if y is None:
        y = torch.empty(T, layer.hidden, dtype=torch.float32, device=x.device)
    s = layer.struct()
    _check(lib().moe_fp4_forward_noalloc(ctypes.byref(s), _ptr(x), T, _ptr(topk_ids), _ptr(topk_weights),
                                         _ptr(y), _stream()))
    return y


_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_runtime():
    """The HIP runtime torch already loaded (for events without a system fence)."""
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            return ctypes.CDLL(name)
        except OSError:
            continue
    return None


class StageTimer:
    """Eight HIP events recorded by moe_fp4_forward_profiled at the stage
    boundaries; durations() gives milliseconds per stage of the last call.

    The events are created with hipEventDisableSystemFence when the HIP
    runtime library can be loaded: a default event's system-scope release
    writes back the L2 at every record, which adds several microseconds to
    each stage of a short (decode) layer."""

    def __init__(self):
        self._hip = _hip_runtime()
        self._raw = None
        if self._hip is not None:
            evs = []
            for _ in range(8):
                ev = ctypes.c_void_p()
                if self._hip.hipEventCreateWithFlags(ctypes.byref(ev), _HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                    evs = None
                    break
                evs.append(ev.value)
            self._raw = evs
        if self._raw is not None:
            self._arr = (ctypes.c_void_p * 8)(*self._raw)
        else:
            self.events = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
            for e in self.events:  # create the underlying hipEvent_t
                e.record()
            torch.cuda.synchronize()
            self._arr = (ctypes.c_void_p * 8)(*[e.cuda_event for e in self.events])

    def durations(self) -> dict:
        if self._raw is None:
            return {name: self.events[i].elapsed_time(self.events[i + 1]) for i, name in enumerate(STAGES)}
        out = {}
        for i, name in enumerate(STAGES):
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self._raw[i]),
                                             ctypes.c_void_p(self._raw[i + 1])) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def __del__(self):
        if getattr(self, "_raw", None) and self._hip is not None:
            for ev in self._raw:
                self._hip.hipEventDestroy(ctypes.c_void_p(ev))


def moe_forward_profiled(layer: MoELayer, x: torch.Tensor, topk_ids: torch.Tensor,
                         topk_weights: torch.Tensor, workspace: torch.Tensor, y: torch.Tensor,
                         timer: StageTimer) -> torch.Tensor:
    T = int(x.shape[0])
    s = layer.struct()
    _check(lib().moe_fp4_forward_profiled(ctypes.byref(s), _ptr(x), T, _ptr(topk_ids), _ptr(topk_weights),
                                          _ptr(y), _ptr(workspace), workspace.numel(), _stream(),
                                          timer._arr, 8))
    return y


def status_string(status: int) -> str:
    return lib().fp4_status_string(status).decode()
