"""ctypes binding of libmoe.so: one Python function per C entry point, same names.

Argument marshalling only: tensors are checked for dtype, shape (every row-indexed buffer
against the row capacity it is used with), contiguity and device, and passed as raw device
pointers together with torch's current HIP stream; outputs that the caller
does not pass are allocated with torch (memory plumbing). Every step of the computation runs
in the library's HIP kernels. There is no CPU fallback: if libmoe.so is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_WS_PERMUTE, MOE_WS_SITU_GLU_FWD, MOE_WS_SITU_GLU_BWD, MOE_WS_DOWN_COMBINE, MOE_WS_EXPERT_BWD = 1, 2, 3, 4, 5
MOE_BWD_DA, MOE_BWD_DW_DOWN, MOE_BWD_DW_GU, MOE_BWD_DX, MOE_BWD_DP, MOE_BWD_ALL = 1, 2, 4, 8, 16, 31

_lock = threading.Lock()
_lib = None


class MoEError(RuntimeError):
    """A libmoe.so call returned a non-OK status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_hip_error": (_I, []),
    "moe_version": (_I, []),
    "moe_route_topk": (_I, [_P, _I64, _I, _I, _P, _P, _P]),
    "moe_permute": (_I, [_P, _P, _I64, _I, _I, _I, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_unpermute": (_I, [_P, _P, _P, _I64, _I, _I, _P, _P]),
    "moe_grouped_gemm_gate_up": (_I, [_P, _I64, _P, _P, _I, _I64, _I, _I, _P, _F, _F, _P, _P,
                                      _P]),
    "situ_glu_fwd": (_I, [_P, _I64, _I, _F, _F, _P, _P, _SZ, _P]),
    "situ_glu_bwd": (_I, [_P, _P, _I64, _I, _F, _F, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_down_combine": (_I, [_P, _P, _P, _P, _I64, _I, _I, _I64, _I, _I, _P, _P,
                                           _P, _SZ, _P]),
    "moe_expert_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I64, _I, _I, _P, _P, _F,
                            _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_router_bwd": (_I, [_P, _P, _I64, _I, _P, _P]),
    "moe_grouped_gemm_down_combine_noalloc": (_I, [_P, _P, _P, _P, _I64, _I, _I, _I64, _I, _I,
                                                   _P, _P, _P]),
    "moe_expert_bwd_stages": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I64, _I,
                                   _I, _P, _P, _F, _F, _P, _P, _P, _P, _P, _SZ, _I, _P]),
    "moe_grouped_gemm_gate_up_mx": (_I, [_P, _I64, _P, _P, _I, _I64, _I, _I, _P, _F, _F, _P, _P,
                                         _P, _P]),
    "moe_expert_bwd_mx": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I64, _I, _I, _P,
                               _P, _F, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp8_quantize": (_I, [_P, _I64, _I, _P, _P, _P]),
    "moe_mxfp8_dequantize": (_I, [_P, _P, _I64, _I, _P, _P]),
    "moe_mxfp4_quantize": (_I, [_P, _I64, _I, _P, _P, _P]),
    "moe_mxfp4_dequantize": (_I, [_P, _P, _I64, _I, _P, _P]),
    "moe_grouped_gemm_gate_up_w4a8": (_I, [_P, _P, _I64, _P, _P, _I, _I64, _I, _I, _P, _P, _F,
                                           _F, _P, _P, _P]),
    "moe_grouped_gemm_down_combine_w4a8": (_I, [_P, _P, _P, _P, _P, _I64, _I, _I, _I64, _I, _I,
                                                _P, _P, _P, _P, _SZ, _P]),
    "moe_workspace_size": (_I, [_I, _I64, _I, _I, _I, _I, _I64, ctypes.POINTER(_SZ)]),
    "moe_workspace_size_passes": (_I, [_I, _I64, _I, _I, _I, _I, _I64, _I,
                                       ctypes.POINTER(_SZ)]),
}


def header_functions(path: str = HEADER_PATH) -> list:
    """Names of the functions include/moe.h declares (parsed from the header text)."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def load():
    """Load libmoe.so once (raises OSError with a clear message when it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise OSError(f"{LIB_PATH} is not built; run sparse_moe_expert_top_amd.build.build()")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        lib = load()
        msg = lib.moe_status_string(status).decode()
        if status == 6:
            msg += f" (hipError {lib.moe_last_hip_error()})"
        raise MoEError(fn, status, msg)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    """Device pointer of a tensor argument. Evaluated only when a call's arguments are built,
    after every dtype and shape check of that call, so the device check comes last."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"every tensor argument must be a GPU tensor (got {t.device})")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None):
    """Type, dtype, exact shape (when given) and contiguity; the device is checked by _ptr."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _need_rows(t, name, dtype, min_rows, cols=None):
    """A row-indexed buffer: at least `min_rows` rows (of `cols` columns when given; a 1-D
    buffer when cols is None), so every row the library may touch lies inside it."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if cols is None:
        if t.dim() != 1 or t.shape[0] < min_rows:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected ({min_rows},) or longer")
    elif t.dim() != 2 or t.shape[1] != cols or t.shape[0] < min_rows:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected (>= {min_rows}, {cols})")
    return _need(t, name, dtype)


def _need_ws(ws, name="ws"):
    return _need(ws, name, torch.uint8)


def _need_perm(perm, T, k, E_loc, R_cap):
    """Metadata from moe_permute for T tokens, k slots, E_loc experts and capacity R_cap."""
    _need(perm["offsets"], "offsets", torch.int32, (E_loc + 1,))
    _need_rows(perm["row_token"], "row_token", torch.int32, R_cap)
    _need_rows(perm["row_gate"], "row_gate", torch.float32, R_cap)
    _need(perm["slot_row"], "slot_row", torch.int32, (T, k))


def workspace_size(which: int, T=0, E_loc=1, k=1, d=64, H=64, R_cap=0) -> int:
    out = _SZ(0)
    _check("moe_workspace_size", load().moe_workspace_size(which, T, E_loc, k, d, H, R_cap,
                                                           ctypes.byref(out)))
    return int(out.value)


def workspace_size_passes(which: int, passes: int, T=0, E_loc=1, k=1, d=64, H=64,
                          R_cap=0) -> int:
    out = _SZ(0)
    _check("moe_workspace_size_passes", load().moe_workspace_size_passes(
        which, T, E_loc, k, d, H, R_cap, passes, ctypes.byref(out)))
    return int(out.value)


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- entry points
def moe_route_topk(logits, k, topk_idx=None, gates=None, stream=None):
    T, E = logits.shape
    _need(logits, "logits", torch.float32)
    dev = logits.device
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    gates = torch.empty((T, k), dtype=torch.float32, device=dev) if gates is None else gates
    _need(topk_idx, "topk_idx", torch.int32, (T, k))
    _need(gates, "gates", torch.float32, (T, k))
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx),
                                                   _ptr(gates), _stream(stream)))
    return topk_idx, gates


def moe_permute(topk_idx, gates, e_lo, E_loc, R_cap, out=None, ws=None, stream=None):
    """Returns dict(offsets, row_token, row_gate, slot_row, status)."""
    T, k = topk_idx.shape
    _need(topk_idx, "topk_idx", torch.int32)
    _need(gates, "gates", torch.float32, (T, k))
    dev = topk_idx.device
    if out is None:
        out = dict(offsets=torch.empty(E_loc + 1, dtype=torch.int32, device=dev),
                   row_token=torch.empty(max(R_cap, 1), dtype=torch.int32, device=dev),
                   row_gate=torch.empty(max(R_cap, 1), dtype=torch.float32, device=dev),
                   slot_row=torch.empty((T, k), dtype=torch.int32, device=dev),
                   status=torch.empty(1, dtype=torch.int32, device=dev))
    _need_perm(out, T, k, E_loc, R_cap)
    _need(out["status"], "status", torch.int32, (1,))
    need = workspace_size(MOE_WS_PERMUTE, T=T, E_loc=E_loc)
    ws = _ws(need, dev) if ws is None else _need_ws(ws)
    _check("moe_permute", load().moe_permute(
        _ptr(topk_idx), _ptr(gates), T, k, e_lo, E_loc, R_cap, _ptr(out["offsets"]),
        _ptr(out["row_token"]), _ptr(out["row_gate"]), _ptr(out["slot_row"]), _ptr(out["status"]),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_unpermute(rows, slot_row, row_weight=None, out=None, stream=None):
    """Every slot_row entry must be -1 or a row of `rows` (checked by the caller)."""
    T, k = slot_row.shape
    n = rows.shape[1]
    _need(rows, "rows", torch.bfloat16)
    _need(slot_row, "slot_row", torch.int32)
    if row_weight is not None:
        _need(row_weight, "row_weight", torch.float32)
    out = torch.empty((T, n), dtype=torch.bfloat16, device=rows.device) if out is None else out
    _need(out, "out", torch.bfloat16, (T, n))
    _check("moe_unpermute", load().moe_unpermute(_ptr(rows), _ptr(slot_row), _ptr(row_weight), T,
                                                 k, n, _ptr(out), _stream(stream)))
    return out


def moe_grouped_gemm_gate_up(x, row_token, offsets, w_gu, R_cap, beta=4.0, linear_beta=25.0,
                             h=None, a=None, stream=None):
    E_loc, H2, d = w_gu.shape
    H = H2 // 2
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, d))
    _need(w_gu, "w_gu", torch.bfloat16)
    _need_rows(row_token, "row_token", torch.int32, R_cap)
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    dev = x.device
    h = torch.empty((R_cap, 2 * H), dtype=torch.bfloat16, device=dev) if h is None else h
    a = torch.empty((R_cap, H), dtype=torch.bfloat16, device=dev) if a is None else a
    _need_rows(h, "h", torch.bfloat16, R_cap, 2 * H)
    _need_rows(a, "a", torch.bfloat16, R_cap, H)
    _check("moe_grouped_gemm_gate_up", load().moe_grouped_gemm_gate_up(
        _ptr(x), T, _ptr(row_token), _ptr(offsets), E_loc, R_cap, d, H, _ptr(w_gu), beta,
        linear_beta, _ptr(h), _ptr(a), _stream(stream)))
    return h, a


def situ_glu_fwd(h, beta=4.0, linear_beta=25.0, a=None, stream=None):
    R, H2 = h.shape
    H = H2 // 2
    _need(h, "h", torch.bfloat16)
    a = torch.empty((R, H), dtype=torch.bfloat16, device=h.device) if a is None else a
    _need(a, "a", torch.bfloat16, (R, H))
    _check("situ_glu_fwd", load().situ_glu_fwd(_ptr(h), R, H, beta, linear_beta, _ptr(a), None,
                                               0, _stream(stream)))
    return a


def situ_glu_bwd(h, da, beta=4.0, linear_beta=25.0, dh=None, stream=None):
    R, H2 = h.shape
    H = H2 // 2
    _need(h, "h", torch.bfloat16)
    _need(da, "da", torch.bfloat16, (R, H))
    dh = torch.empty_like(h) if dh is None else dh
    _need(dh, "dh", torch.bfloat16, (R, 2 * H))
    _check("situ_glu_bwd", load().situ_glu_bwd(_ptr(h), _ptr(da), R, H, beta, linear_beta,
                                               _ptr(dh), None, 0, _stream(stream)))
    return dh


def moe_grouped_gemm_down_combine(a, offsets, row_gate, slot_row, w_down, R_cap, y=None,
                                  ws=None, stream=None):
    """ws: uint8 workspace; None allocates the one-pass size. Any size from
    workspace_size_passes(MOE_WS_DOWN_COMBINE, d // 256, ...) up works (more column passes
    when smaller)."""
    E_loc, d, H = w_down.shape
    T, k = slot_row.shape
    _need_rows(a, "a", torch.bfloat16, R_cap, H)
    _need(w_down, "w_down", torch.bfloat16)
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    _need_rows(row_gate, "row_gate", torch.float32, R_cap)
    _need(slot_row, "slot_row", torch.int32)
    dev = a.device
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, (T, d))
    need = workspace_size(MOE_WS_DOWN_COMBINE, T=T, E_loc=E_loc, k=k, d=d, H=H, R_cap=R_cap)
    ws = _ws(need, dev) if ws is None else _need_ws(ws)
    _check("moe_grouped_gemm_down_combine", load().moe_grouped_gemm_down_combine(
        _ptr(a), _ptr(offsets), _ptr(row_gate), _ptr(slot_row), T, k, E_loc, R_cap, H, d,
        _ptr(w_down), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_grouped_gemm_down_combine_noalloc(a, offsets, row_gate, slot_row, w_down, R_cap,
                                          y=None, stream=None):
    """moe_grouped_gemm_down_combine without a workspace: the fp32 rows live in the library's
    static per-device scratch (R_cap at most 65536 for d >= 256). Calls that overlap on one GPU
    race on that scratch."""
    E_loc, d, H = w_down.shape
    T, k = slot_row.shape
    _need_rows(a, "a", torch.bfloat16, R_cap, H)
    _need(w_down, "w_down", torch.bfloat16)
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    _need_rows(row_gate, "row_gate", torch.float32, R_cap)
    _need(slot_row, "slot_row", torch.int32)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=a.device) if y is None else y
    _need(y, "y", torch.bfloat16, (T, d))
    _check("moe_grouped_gemm_down_combine_noalloc", load().moe_grouped_gemm_down_combine_noalloc(
        _ptr(a), _ptr(offsets), _ptr(row_gate), _ptr(slot_row), T, k, E_loc, R_cap, H, d,
        _ptr(w_down), _ptr(y), _stream(stream)))
    return y


def moe_expert_bwd(dy, x, h, perm, w_gu, w_down, R_cap, beta=4.0, linear_beta=25.0,
                   dx=None, dw_gu=None, dw_down=None, dp=None, ws=None, stream=None):
    """perm: dict with offsets, row_token, row_gate, slot_row (from moe_permute).
    ws: uint8 workspace; None allocates the one-pass size. Any size from
    workspace_size_passes(MOE_WS_EXPERT_BWD, d // 256, ...) up works (more dX column passes
    when smaller)."""
    E_loc, H2, d = w_gu.shape
    H = H2 // 2
    T, k = perm["slot_row"].shape
    _need(dy, "dy", torch.bfloat16, (T, d))
    _need(x, "x", torch.bfloat16, (T, d))
    _need_rows(h, "h", torch.bfloat16, R_cap, 2 * H)
    _need_perm(perm, T, k, E_loc, R_cap)
    _need(w_gu, "w_gu", torch.bfloat16)
    _need(w_down, "w_down", torch.bfloat16, (E_loc, d, H))
    dev = dy.device
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if dx is None else dx
    dw_gu = torch.empty((E_loc, 2 * H, d), dtype=torch.float32, device=dev) if dw_gu is None else dw_gu
    dw_down = torch.empty((E_loc, d, H), dtype=torch.float32, device=dev) if dw_down is None else dw_down
    dp = torch.empty((T, k), dtype=torch.float32, device=dev) if dp is None else dp
    _need(dx, "dx", torch.bfloat16, (T, d))
    _need(dw_gu, "dw_gu", torch.float32, (E_loc, 2 * H, d))
    _need(dw_down, "dw_down", torch.float32, (E_loc, d, H))
    _need(dp, "dp", torch.float32, (T, k))
    need = workspace_size(MOE_WS_EXPERT_BWD, T=T, E_loc=E_loc, k=k, d=d, H=H, R_cap=R_cap)
    ws = _ws(need, dev) if ws is None else _need_ws(ws)
    _check("moe_expert_bwd", load().moe_expert_bwd(
        _ptr(dy), _ptr(x), _ptr(h), _ptr(perm["row_token"]), _ptr(perm["row_gate"]),
        _ptr(perm["slot_row"]), _ptr(perm["offsets"]), T, k, E_loc, R_cap, d, H, _ptr(w_gu),
        _ptr(w_down), beta, linear_beta, _ptr(dx), _ptr(dw_gu), _ptr(dw_down), _ptr(dp),
        _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dw_gu, dw_down, dp


def moe_grouped_gemm_gate_up_mx(x, row_token, offsets, w_gu, R_cap, beta=4.0,
                                linear_beta=25.0, h_codes=None, h_scales=None, a=None,
                                stream=None):
    """moe_grouped_gemm_gate_up storing the saved h as MXFP8 (codes, scale bytes)."""
    E_loc, H2, d = w_gu.shape
    H = H2 // 2
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, d))
    _need(w_gu, "w_gu", torch.bfloat16)
    _need_rows(row_token, "row_token", torch.int32, R_cap)
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    dev = x.device
    h_codes = torch.empty((R_cap, 2 * H), dtype=torch.uint8, device=dev) if h_codes is None else h_codes
    h_scales = (torch.empty((R_cap, 2 * H // 32), dtype=torch.uint8, device=dev)
                if h_scales is None else h_scales)
    a = torch.empty((R_cap, H), dtype=torch.bfloat16, device=dev) if a is None else a
    _need_rows(h_codes, "h_codes", torch.uint8, R_cap, 2 * H)
    _need_rows(h_scales, "h_scales", torch.uint8, R_cap, 2 * H // 32)
    _need_rows(a, "a", torch.bfloat16, R_cap, H)
    _check("moe_grouped_gemm_gate_up_mx", load().moe_grouped_gemm_gate_up_mx(
        _ptr(x), T, _ptr(row_token), _ptr(offsets), E_loc, R_cap, d, H, _ptr(w_gu), beta,
        linear_beta, _ptr(h_codes), _ptr(h_scales), _ptr(a), _stream(stream)))
    return h_codes, h_scales, a


def moe_expert_bwd_mx(dy, x, h_codes, h_scales, perm, w_gu, w_down, R_cap, beta=4.0,
                      linear_beta=25.0, dx=None, dw_gu=None, dw_down=None, dp=None, ws=None,
                      stream=None):
    """moe_expert_bwd reading the saved h from MXFP8 codes and scale bytes."""
    E_loc, H2, d = w_gu.shape
    H = H2 // 2
    T, k = perm["slot_row"].shape
    _need(dy, "dy", torch.bfloat16, (T, d))
    _need(x, "x", torch.bfloat16, (T, d))
    _need_rows(h_codes, "h_codes", torch.uint8, R_cap, 2 * H)
    _need_rows(h_scales, "h_scales", torch.uint8, R_cap, 2 * H // 32)
    _need_perm(perm, T, k, E_loc, R_cap)
    _need(w_gu, "w_gu", torch.bfloat16)
    _need(w_down, "w_down", torch.bfloat16, (E_loc, d, H))
    dev = dy.device
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if dx is None else dx
    dw_gu = torch.empty((E_loc, 2 * H, d), dtype=torch.float32, device=dev) if dw_gu is None else dw_gu
    dw_down = torch.empty((E_loc, d, H), dtype=torch.float32, device=dev) if dw_down is None else dw_down
    dp = torch.empty((T, k), dtype=torch.float32, device=dev) if dp is None else dp
    _need(dx, "dx", torch.bfloat16, (T, d))
    _need(dw_gu, "dw_gu", torch.float32, (E_loc, 2 * H, d))
    _need(dw_down, "dw_down", torch.float32, (E_loc, d, H))
    _need(dp, "dp", torch.float32, (T, k))
    need = workspace_size(MOE_WS_EXPERT_BWD, T=T, E_loc=E_loc, k=k, d=d, H=H, R_cap=R_cap)
    ws = _ws(need, dev) if ws is None else _need_ws(ws)
    _check("moe_expert_bwd_mx", load().moe_expert_bwd_mx(
        _ptr(dy), _ptr(x), _ptr(h_codes), _ptr(h_scales), _ptr(perm["row_token"]),
        _ptr(perm["row_gate"]), _ptr(perm["slot_row"]), _ptr(perm["offsets"]), T, k, E_loc,
        R_cap, d, H, _ptr(w_gu), _ptr(w_down), beta, linear_beta, _ptr(dx), _ptr(dw_gu),
        _ptr(dw_down), _ptr(dp), _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dw_gu, dw_down, dp


def moe_expert_bwd_stages(dy, x, perm, w_gu, w_down, R_cap, stages, dx, dw_gu, dw_down, dp, ws,
                          h=None, h_codes=None, h_scales=None, beta=4.0, linear_beta=25.0,
                          stream=None):
    """The backward stages in the bit mask `stages` (MOE_BWD_*), in their fixed order. The
    saved h is bf16 `h` or MXFP8 `h_codes` + `h_scales`. Outputs and ws are required: calls
    over one backward share them (ws carries what MOE_BWD_DA writes to the later stages)."""
    E_loc, H2, d = w_gu.shape
    H = H2 // 2
    T, k = perm["slot_row"].shape
    _need(dy, "dy", torch.bfloat16, (T, d))
    _need(x, "x", torch.bfloat16, (T, d))
    if h is not None:
        _need_rows(h, "h", torch.bfloat16, R_cap, 2 * H)
    else:
        _need_rows(h_codes, "h_codes", torch.uint8, R_cap, 2 * H)
        _need_rows(h_scales, "h_scales", torch.uint8, R_cap, 2 * H // 32)
    _need_perm(perm, T, k, E_loc, R_cap)
    _need(w_gu, "w_gu", torch.bfloat16)
    _need(w_down, "w_down", torch.bfloat16, (E_loc, d, H))
    _need(dx, "dx", torch.bfloat16, (T, d))
    _need(dw_gu, "dw_gu", torch.float32, (E_loc, 2 * H, d))
    _need(dw_down, "dw_down", torch.float32, (E_loc, d, H))
    _need(dp, "dp", torch.float32, (T, k))
    _need_ws(ws)
    _check("moe_expert_bwd_stages", load().moe_expert_bwd_stages(
        _ptr(dy), _ptr(x), _ptr(h), _ptr(h_codes), _ptr(h_scales), _ptr(perm["row_token"]),
        _ptr(perm["row_gate"]), _ptr(perm["slot_row"]), _ptr(perm["offsets"]), T, k, E_loc,
        R_cap, d, H, _ptr(w_gu), _ptr(w_down), beta, linear_beta, _ptr(dx), _ptr(dw_gu),
        _ptr(dw_down), _ptr(dp), _ptr(ws), ws.numel(), int(stages), _stream(stream)))
    return dx, dw_gu, dw_down, dp


def moe_mxfp8_quantize(v, codes=None, scales=None, stream=None):
    """bf16 [rows, n] -> (codes uint8 [rows, n], scale bytes uint8 [rows, n/32])."""
    rows, n = v.shape
    _need(v, "v", torch.bfloat16)
    codes = torch.empty((rows, n), dtype=torch.uint8, device=v.device) if codes is None else codes
    scales = (torch.empty((rows, n // 32), dtype=torch.uint8, device=v.device)
              if scales is None else scales)
    _need(codes, "codes", torch.uint8, (rows, n))
    _need(scales, "scales", torch.uint8, (rows, n // 32))
    _check("moe_mxfp8_quantize", load().moe_mxfp8_quantize(_ptr(v), rows, n, _ptr(codes),
                                                           _ptr(scales), _stream(stream)))
    return codes, scales


def moe_mxfp8_dequantize(codes, scales, out=None, stream=None):
    """(codes, scale bytes) -> bf16 [rows, n]."""
    rows, n = codes.shape
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8, (rows, n // 32))
    out = torch.empty((rows, n), dtype=torch.bfloat16, device=codes.device) if out is None else out
    _need(out, "out", torch.bfloat16, (rows, n))
    _check("moe_mxfp8_dequantize", load().moe_mxfp8_dequantize(_ptr(codes), _ptr(scales), rows,
                                                               n, _ptr(out), _stream(stream)))
    return out


def moe_mxfp4_quantize(v, codes=None, scales=None, stream=None):
    """bf16 [rows, n] -> (packed E2M1 codes uint8 [rows, n/2], scale bytes uint8 [rows, n/32])."""
    rows, n = v.shape
    _need(v, "v", torch.bfloat16)
    codes = (torch.empty((rows, n // 2), dtype=torch.uint8, device=v.device)
             if codes is None else codes)
    scales = (torch.empty((rows, n // 32), dtype=torch.uint8, device=v.device)
              if scales is None else scales)
    _need(codes, "codes", torch.uint8, (rows, n // 2))
    _need(scales, "scales", torch.uint8, (rows, n // 32))
    _check("moe_mxfp4_quantize", load().moe_mxfp4_quantize(_ptr(v), rows, n, _ptr(codes),
                                                           _ptr(scales), _stream(stream)))
    return codes, scales


def moe_mxfp4_dequantize(codes, scales, out=None, stream=None):
    """(packed codes [rows, n/2], scale bytes [rows, n/32]) -> bf16 [rows, n]."""
    rows, half = codes.shape
    n = 2 * half
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8, (rows, n // 32))
    out = torch.empty((rows, n), dtype=torch.bfloat16, device=codes.device) if out is None else out
    _need(out, "out", torch.bfloat16, (rows, n))
    _check("moe_mxfp4_dequantize", load().moe_mxfp4_dequantize(_ptr(codes), _ptr(scales), rows,
                                                               n, _ptr(out), _stream(stream)))
    return out


def moe_grouped_gemm_gate_up_w4a8(x_codes, x_scales, row_token, offsets, w_gu_codes,
                                  w_gu_scales, R_cap, beta=4.0, linear_beta=25.0, a_codes=None,
                                  a_scales=None, stream=None):
    """W4A8 gate/up + SiTU-GLU: MXFP8 x [T, d] (+ scales), MXFP4 w_gu [E_loc, 2H, d/2]
    (+ scales [E_loc, 2H, d/32]) -> a as MXFP8 (codes [R_cap, H], scales [R_cap, H/32])."""
    T, d = x_codes.shape
    E_loc, H2, _ = w_gu_codes.shape
    H = H2 // 2
    _need(x_codes, "x_codes", torch.uint8, (T, d))
    _need(x_scales, "x_scales", torch.uint8, (T, d // 32))
    _need(w_gu_codes, "w_gu_codes", torch.uint8, (E_loc, 2 * H, d // 2))
    _need(w_gu_scales, "w_gu_scales", torch.uint8, (E_loc, 2 * H, d // 32))
    _need_rows(row_token, "row_token", torch.int32, R_cap)
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    dev = x_codes.device
    a_codes = (torch.empty((R_cap, H), dtype=torch.uint8, device=dev)
               if a_codes is None else a_codes)
    a_scales = (torch.empty((R_cap, H // 32), dtype=torch.uint8, device=dev)
                if a_scales is None else a_scales)
    _need_rows(a_codes, "a_codes", torch.uint8, R_cap, H)
    _need_rows(a_scales, "a_scales", torch.uint8, R_cap, H // 32)
    _check("moe_grouped_gemm_gate_up_w4a8", load().moe_grouped_gemm_gate_up_w4a8(
        _ptr(x_codes), _ptr(x_scales), T, _ptr(row_token), _ptr(offsets), E_loc, R_cap, d, H,
        _ptr(w_gu_codes), _ptr(w_gu_scales), beta, linear_beta, _ptr(a_codes), _ptr(a_scales),
        _stream(stream)))
    return a_codes, a_scales


def moe_grouped_gemm_down_combine_w4a8(a_codes, a_scales, offsets, row_gate, slot_row,
                                       w_down_codes, w_down_scales, R_cap, y=None, ws=None,
                                       stream=None):
    """W4A8 down GEMM + combine: MXFP8 a, MXFP4 w_down [E_loc, d, H/2] (+ scales
    [E_loc, d, H/32]) -> y [T, d] bf16."""
    E_loc, d, half = w_down_codes.shape
    H = 2 * half
    T, k = slot_row.shape
    _need_rows(a_codes, "a_codes", torch.uint8, R_cap, H)
    _need_rows(a_scales, "a_scales", torch.uint8, R_cap, H // 32)
    _need(w_down_codes, "w_down_codes", torch.uint8)
    _need(w_down_scales, "w_down_scales", torch.uint8, (E_loc, d, H // 32))
    _need(offsets, "offsets", torch.int32, (E_loc + 1,))
    _need_rows(row_gate, "row_gate", torch.float32, R_cap)
    _need(slot_row, "slot_row", torch.int32)
    dev = a_codes.device
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, (T, d))
    need = workspace_size(MOE_WS_DOWN_COMBINE, T=T, E_loc=E_loc, k=k, d=d, H=H, R_cap=R_cap)
    ws = _ws(need, dev) if ws is None else _need_ws(ws)
    _check("moe_grouped_gemm_down_combine_w4a8", load().moe_grouped_gemm_down_combine_w4a8(
        _ptr(a_codes), _ptr(a_scales), _ptr(offsets), _ptr(row_gate), _ptr(slot_row), T, k,
        E_loc, R_cap, H, d, _ptr(w_down_codes), _ptr(w_down_scales), _ptr(y), _ptr(ws),
        ws.numel(), _stream(stream)))
    return y


def moe_router_bwd(gates, dp, out=None, stream=None):
    T, k = gates.shape
    _need(gates, "gates", torch.float32)
    _need(dp, "dp", torch.float32, (T, k))
    out = torch.empty_like(gates) if out is None else out
    _check("moe_router_bwd", load().moe_router_bwd(_ptr(gates), _ptr(dp), T, k, _ptr(out),
                                                   _stream(stream)))
    return out
