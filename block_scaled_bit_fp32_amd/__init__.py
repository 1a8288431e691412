"""Python binding of libmoe_mi355x.so, the MI355X (gfx950) decode MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch provides device memory and the current stream. Importing this package fails
loudly if the shared library has not been built (``__graft_entry__.build()``); there is
no CPU fallback.

Names follow include/moe.h:
    route(layer, x, ws)                  -> topk_ids, topk_w, xq
    expert_forward(layer, x, xq, ids, w, ws, debug=False) -> y (BF16) [, debug dict]
    forward(layer, x, ws)                -> y, topk_ids, topk_w, xq
    forward_noalloc(layer, x)            -> y, topk_ids, topk_w, xq (library scratch)
    forward_fused(layer, r, gamma, eps, ws) -> r + y, x = RMSNorm(r), topk_ids, topk_w, xq
    quantize_nvfp4_4o6(x)                -> codes, scales, gscale, choice
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_ELAUNCH = 0, -1, -2, -3, -4
WFMT = {"bf16": 0, "nvfp4": 1, "mxfp4": 2, "mxfp8": 3}
AFMT = {"bf16": 0, "nvfp4_4o6": 1, "fp8_token": 2, "mxfp4": 3, "mxfp8": 4}
SCORE = {"sigmoid": 0, "softmax": 1}
ABI_VERSION = 5


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


class WeightsT(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("gscale", ctypes.c_void_p)]


class LayerT(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("has_shared", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("wfmt", ctypes.c_int32), ("shared_wfmt", ctypes.c_int32), ("afmt", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("w13", WeightsT), ("w2", WeightsT), ("sh13", WeightsT), ("sh2", WeightsT),
                ("router_score", ctypes.c_int32), ("bias_select_only", ctypes.c_int32)]


class DebugT(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("hq_codes", ctypes.c_void_p),
                ("hq_scales", ctypes.c_void_p), ("hq_scale", ctypes.c_void_p), ("path", ctypes.c_int32)]


PATH_AUTO, PATH_GEMV, PATH_GROUPED = 0, 1, 2


class NormT(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("eps", ctypes.c_float)]


class KernelTimeT(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


# Every symbol include/moe.h declares, with its ctypes signature.
_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "moe_layer_check": (_I32, [ctypes.POINTER(LayerT), _I32, ctypes.c_char_p, _SZ]),
    "moe_workspace_bytes": (_SZ, [ctypes.POINTER(LayerT), _I32]),
    "moe_xq_bytes": (_SZ, [ctypes.POINTER(LayerT), _I32]),
    "moe_workspace_init": (_I32, [_P, _SZ, _P]),
    "moe_route": (_I32, [ctypes.POINTER(LayerT), _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_forward": (_I32, [ctypes.POINTER(LayerT), _P, _P, _I32, _P, _P, _P, _P, _SZ,
                                  ctypes.POINTER(DebugT), _P]),
    "moe_forward": (_I32, [ctypes.POINTER(LayerT), _P, _I32, _P, _P, _P, _P, _P, _SZ,
                           ctypes.POINTER(DebugT), _P]),
    "moe_forward_fused": (_I32, [ctypes.POINTER(LayerT), ctypes.POINTER(NormT), _P, _I32, _P, _P, _P, _P, _P, _P,
                                 _SZ, ctypes.POINTER(DebugT), _P]),
    "moe_forward_noalloc": (_I32, [ctypes.POINTER(LayerT), _P, _I32, _P, _P, _P, _P,
                                   ctypes.POINTER(DebugT), _P]),
    "moe_noalloc_scratch_bytes": (_SZ, []),
    "quantize_nvfp4_4o6": (_I32, [_P, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_requant_mxfp4": (_I32, [_P, ctypes.c_int64, _I32, _P, _P, _P]),
    "moe_requant_nvfp4": (_I32, [_P, _I32, ctypes.c_int64, _I32, _P, _P, _P, _P]),
    "moe_requant_mxfp8": (_I32, [_P, ctypes.c_int64, _I32, _P, _P, _P]),
    "moe_requant_fp8_block_mxfp4": (_I32, [_P, _P, ctypes.c_int64, _I32, _I32, _I32, _P, _P, _P]),
    "moe_profile_begin": (_I32, []),
    "moe_profile_end": (_I32, [ctypes.POINTER(KernelTimeT), _I32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_I32, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {lib.moe_abi_version()} != {ABI_VERSION}")
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, _lib.moe_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """One layer's weights in device memory plus the moe_layer_t that points at them.

    Built from the host arrays of ``synth.make_layer`` (storage formats, stacked
    [n][rows][...]); ``copy()`` makes an independent device replica with the same bytes.
    """

    def __init__(self, cfg, tensors: dict):
        self.cfg = cfg
        self.t = tensors
        self.struct = LayerT()
        s = self.struct
        s.H, s.I, s.E, s.k = cfg.H, cfg.I, cfg.E, cfg.k
        s.has_shared = 1 if cfg.has_shared else 0
        s.I_shared = cfg.Ish if cfg.has_shared else 0
        s.wfmt = WFMT[cfg.wfmt]
        s.shared_wfmt = WFMT[cfg.shared_wfmt]
        s.afmt = AFMT[cfg.afmt]
        s.router_w = _ptr(tensors["router_w"])
        s.router_bias = _ptr(tensors.get("router_bias"))
        s.router_score = SCORE[getattr(cfg, "score", "sigmoid")]
        s.bias_select_only = 1 if getattr(cfg, "bias_select_only", False) else 0
        for name in ("w13", "w2", "sh13", "sh2"):
            part = tensors.get(name)
            if part is None:
                continue
            setattr(s, name, WeightsT(_ptr(part["codes"]), _ptr(part.get("scales")),
                                      _ptr(part.get("gscale"))))

    @classmethod
    def from_host(cls, layer: dict, device="cuda") -> "DeviceLayer":
        cfg = layer["cfg"]
        if layer["expert_ids"] != list(range(cfg.E)):
            raise ValueError("the device layer needs every routed expert")
        t = {"router_w": _dev(layer["router_w"], device),
             "router_bias": _dev(layer["router_bias"], device)}
        for name in ("w13", "w2", "sh13", "sh2"):
            part = layer[name]
            t[name] = None if part is None else {k: _dev(v, device) for k, v in part.items()}
        return cls(cfg, t)

    def copy(self) -> "DeviceLayer":
        def cp(v):
            if v is None:
                return None
            if isinstance(v, dict):
                return {k: cp(x) for k, x in v.items()}
            return v.clone()
        return DeviceLayer(self.cfg, {k: cp(v) for k, v in self.t.items()})

    def nbytes_expert(self, which: str, e: int) -> int:
        """Weight bytes of routed expert e ("routed") or of the shared expert."""
        parts = ("w13", "w2") if which == "routed" else ("sh13", "sh2")
        n = 0
        for name in parts:
            for v in self.t[name].values():
                if v is not None:
                    n += v[e].numel() * v.element_size()
        return n

    def check(self, max_tokens: int) -> str:
        buf = ctypes.create_string_buffer(4096)
        _lib.moe_layer_check(ctypes.byref(self.struct), max_tokens, buf, len(buf))
        return buf.value.decode()


def layer_check(layer: DeviceLayer, max_tokens: int):
    buf = ctypes.create_string_buffer(4096)
    st = _lib.moe_layer_check(ctypes.byref(layer.struct), max_tokens, buf, len(buf))
    return st, buf.value.decode()


class Workspace:
    """Device workspace for calls with up to ``max_tokens`` tokens, zeroed on creation."""

    def __init__(self, layer: DeviceLayer, max_tokens: int, device="cuda"):
        n = _lib.moe_workspace_bytes(ctypes.byref(layer.struct), max_tokens)
        if n == 0:
            raise MoeError(MOE_EUNSUPPORTED, layer.check(max_tokens))
        self.max_tokens = max_tokens
        self.buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.t = self.buf[off:off + n]
        self.nbytes = n
        _check(_lib.moe_workspace_init(self.t.data_ptr(), n, _stream()))

    @property
    def ptr(self) -> int:
        return self.t.data_ptr()


def _bits16(x: torch.Tensor) -> torch.Tensor:
    if x.element_size() != 2 or not x.is_contiguous():
        raise ValueError("expected a contiguous 2-byte (BF16 bits) tensor")
    return x


def xq_bytes(layer: DeviceLayer, T: int) -> int:
    return _lib.moe_xq_bytes(ctypes.byref(layer.struct), T)


def _aligned_empty(nbytes: int, device) -> torch.Tensor:
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def route(layer: DeviceLayer, x: torch.Tensor, ws: Workspace, out=None):
    """moe_route: returns (topk_ids int32 [T,k], topk_w FP32 [T,k], xq uint8 or None)."""
    x = _bits16(x)
    T = x.shape[0]
    k = layer.cfg.k
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
        nq = xq_bytes(layer, T)
        xq = _aligned_empty(nq, x.device) if nq else None
    else:
        ids, w, xq = out
    _check(_lib.moe_route(ctypes.byref(layer.struct), x.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                          _ptr(xq), ws.ptr, ws.nbytes, _stream()))
    return ids, w, xq


def split_xq(layer: DeviceLayer, xq: torch.Tensor, T: int) -> dict:
    """Views of the parts of an xq buffer (layout in include/moe.h)."""
    H = layer.cfg.H

    def part(nbytes):
        return (nbytes + 255) // 256 * 256

    if layer.cfg.afmt == "nvfp4_4o6":
        a, b = part(T * H // 2), part(T * H // 16)
        return {"codes": xq[:T * H // 2].view(T, H // 2),
                "scales": xq[a:a + T * H // 16].view(T, H // 16),
                "g": xq[a + b:a + b + 4 * T].view(torch.float32)}
    if layer.cfg.afmt == "fp8_token":
        a = part(T * H)
        return {"codes": xq[:T * H].view(T, H), "s": xq[a:a + 4 * T].view(torch.float32)}
    if layer.cfg.afmt in ("mxfp4", "mxfp8"):
        n = T * H // 2 if layer.cfg.afmt == "mxfp4" else T * H
        a = part(n)
        return {"codes": xq[:n].view(T, n // T), "scales": xq[a:a + T * H // 32].view(T, H // 32)}
    return {}


def expert_forward(layer: DeviceLayer, x: torch.Tensor, xq, ids: torch.Tensor, w: torch.Tensor,
                   ws: Workspace, debug: bool = False, y: Optional[torch.Tensor] = None,
                   path: int = PATH_AUTO):
    """moe_expert_forward: returns y (BF16 [T,H]); with debug=True also a dict of h and
    the quantized h fields (pair p = t*k + j; rows T*k + t are the shared expert).
    ``path`` picks the expert kernels (PATH_AUTO, PATH_GEMV, PATH_GROUPED)."""
    x = _bits16(x)
    T = x.shape[0]
    cfg = layer.cfg
    if y is None:
        y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=x.device)
    dbg = DebugT(None, None, None, None, path) if path != PATH_AUTO else None
    dd = {}
    if debug:
        rows = T * cfg.k + (T if cfg.has_shared else 0)
        hs = max(cfg.I, cfg.Ish if cfg.has_shared else 0)
        dd["h"] = torch.zeros((rows, hs), dtype=torch.float32, device=x.device)
        P = T * cfg.k
        if cfg.afmt == "nvfp4_4o6":
            dd["hq_codes"] = _aligned_empty(P * cfg.I // 2, x.device).view(P, cfg.I // 2)
            dd["hq_scales"] = torch.empty((P, cfg.I // 16), dtype=torch.uint8, device=x.device)
            dd["hq_scale"] = torch.empty(P, dtype=torch.float32, device=x.device)
        elif cfg.afmt == "fp8_token":
            dd["hq_codes"] = _aligned_empty(P * cfg.I, x.device).view(P, cfg.I)
            dd["hq_scale"] = torch.empty(P, dtype=torch.float32, device=x.device)
        elif cfg.afmt in ("mxfp4", "mxfp8"):
            n = cfg.I // 2 if cfg.afmt == "mxfp4" else cfg.I
            dd["hq_codes"] = _aligned_empty(P * n, x.device).view(P, n)
            dd["hq_scales"] = torch.empty((P, cfg.I // 32), dtype=torch.uint8, device=x.device)
        dbg = DebugT(_ptr(dd.get("h")), _ptr(dd.get("hq_codes")), _ptr(dd.get("hq_scales")),
                     _ptr(dd.get("hq_scale")), path)
    _check(_lib.moe_expert_forward(ctypes.byref(layer.struct), x.data_ptr(), _ptr(xq), T,
                                   ids.data_ptr(), w.data_ptr(), y.data_ptr(), ws.ptr, ws.nbytes,
                                   ctypes.byref(dbg) if dbg is not None else None, _stream()))
    return (y, dd) if debug else y


def forward(layer: DeviceLayer, x: torch.Tensor, ws: Workspace, out=None, path: int = PATH_AUTO):
    """moe_forward (route and experts in one call): returns (y BF16 [T,H], topk_ids int32
    [T,k], topk_w FP32 [T,k], xq uint8 or None). ``out`` = (y, ids, w, xq) reuses buffers."""
    x = _bits16(x)
    T = x.shape[0]
    cfg = layer.cfg
    if out is None:
        y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=x.device)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=x.device)
        nq = xq_bytes(layer, T)
        xq = _aligned_empty(nq, x.device) if nq else None
    else:
        y, ids, w, xq = out
    dbg = DebugT(None, None, None, None, path) if path != PATH_AUTO else None
    _check(_lib.moe_forward(ctypes.byref(layer.struct), x.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                            _ptr(xq), y.data_ptr(), ws.ptr, ws.nbytes,
                            ctypes.byref(dbg) if dbg is not None else None, _stream()))
    return y, ids, w, xq


def forward_fused(layer: DeviceLayer, resid: torch.Tensor, gamma: torch.Tensor, eps: float, ws: Workspace,
                  out=None, resid_out: Optional[torch.Tensor] = None, path: int = PATH_AUTO):
    """moe_forward_fused: x = RMSNorm(resid) * gamma (BF16), the layer on x, and the residual
    stream resid + y. Returns (resid_out, x, topk_ids, topk_w, xq); ``out`` = (x, ids, w,
    xq) reuses buffers; ``resid_out`` may be ``resid`` itself (in place)."""
    resid = _bits16(resid)
    gamma = _bits16(gamma)
    T = resid.shape[0]
    cfg = layer.cfg
    if out is None:
        x = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=resid.device)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=resid.device)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=resid.device)
        nq = xq_bytes(layer, T)
        xq = _aligned_empty(nq, resid.device) if nq else None
    else:
        x, ids, w, xq = out
    if resid_out is None:
        resid_out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=resid.device)
    norm = NormT(gamma.data_ptr(), float(eps))
    dbg = DebugT(None, None, None, None, path) if path != PATH_AUTO else None
    _check(_lib.moe_forward_fused(ctypes.byref(layer.struct), ctypes.byref(norm), resid.data_ptr(), T, x.data_ptr(),
                                  ids.data_ptr(), w.data_ptr(), _ptr(xq), resid_out.data_ptr(), ws.ptr, ws.nbytes,
                                  ctypes.byref(dbg) if dbg is not None else None, _stream()))
    return resid_out, x, ids, w, xq


def forward_noalloc(layer: DeviceLayer, x: torch.Tensor, out=None, path: int = PATH_AUTO):
    """moe_forward_noalloc: moe_forward on the library's static per-GPU scratch (no
    workspace argument). Returns (y, topk_ids, topk_w, xq); ``out`` reuses buffers."""
    x = _bits16(x)
    T = x.shape[0]
    cfg = layer.cfg
    if out is None:
        y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=x.device)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=x.device)
        nq = xq_bytes(layer, T)
        xq = _aligned_empty(nq, x.device) if nq else None
    else:
        y, ids, w, xq = out
    dbg = DebugT(None, None, None, None, path) if path != PATH_AUTO else None
    _check(_lib.moe_forward_noalloc(ctypes.byref(layer.struct), x.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                                    _ptr(xq), y.data_ptr(), ctypes.byref(dbg) if dbg is not None else None,
                                    _stream()))
    return y, ids, w, xq


def noalloc_scratch_bytes() -> int:
    return _lib.moe_noalloc_scratch_bytes()


def quantize_nvfp4_4o6(x: torch.Tensor, want_choice: bool = True):
    """Four-Over-Six NVFP4 rows: returns (codes [rows, cols/2], scales [rows, cols/16],
    gscale [rows], choice [rows, cols/16] or None)."""
    x = _bits16(x)
    rows, cols = x.shape
    codes = _aligned_empty(rows * cols // 2, x.device).view(rows, cols // 2)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(rows, dtype=torch.float32, device=x.device)
    choice = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device) if want_choice else None
    _check(_lib.quantize_nvfp4_4o6(x.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                   g.data_ptr(), _ptr(choice), _stream()))
    return codes, scales, g, choice


def requant_mxfp4(w: torch.Tensor):
    """moe_requant_mxfp4 of BF16 rows w [rows, cols]: returns (codes [rows, cols/2],
    E8M0 scales [rows, cols/32]), the MOE_W_MXFP4 layout."""
    w = _bits16(w)
    rows, cols = w.shape
    codes = _aligned_empty(rows * cols // 2, w.device).view(rows, cols // 2)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=w.device)
    _check(_lib.moe_requant_mxfp4(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def requant_mxfp8(w: torch.Tensor):
    """moe_requant_mxfp8 of BF16 rows w [rows, cols]: returns (E4M3 codes [rows, cols],
    E8M0 scales [rows, cols/32]), the MOE_W_MXFP8 layout."""
    w = _bits16(w)
    rows, cols = w.shape
    codes = _aligned_empty(rows * cols, w.device).view(rows, cols)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=w.device)
    _check(_lib.moe_requant_mxfp8(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def requant_fp8_block_mxfp4(w: torch.Tensor, block_scales: torch.Tensor, block_rows: int, block_cols: int):
    """moe_requant_fp8_block_mxfp4 of E4M3 bytes w [rows, cols] (uint8) with FP32 block
    scales [ceil(rows/block_rows), ceil(cols/block_cols)]: returns (codes [rows, cols/2],
    E8M0 scales [rows, cols/32]), the MOE_W_MXFP4 layout."""
    if w.dtype != torch.uint8 or w.dim() != 2 or block_scales.dtype != torch.float32:
        raise TypeError("w must be uint8 [rows, cols] and block_scales float32")
    w = w.contiguous()
    block_scales = block_scales.contiguous()
    rows, cols = w.shape
    codes = _aligned_empty(rows * cols // 2, w.device).view(rows, cols // 2)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=w.device)
    _check(_lib.moe_requant_fp8_block_mxfp4(w.data_ptr(), block_scales.data_ptr(), rows, cols, block_rows, block_cols,
                                            codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def requant_nvfp4(w: torch.Tensor):
    """moe_requant_nvfp4 of BF16 tensors w [n, rows, cols]: returns (codes [n, rows, cols/2],
    E4M3 scales [n, rows, cols/16], gscale [n] FP32), the MOE_W_NVFP4 layout."""
    w = _bits16(w)
    n, rows, cols = w.shape
    codes = _aligned_empty(n * rows * cols // 2, w.device).view(n, rows, cols // 2)
    scales = torch.empty((n, rows, cols // 16), dtype=torch.uint8, device=w.device)
    g = torch.empty(n, dtype=torch.float32, device=w.device)
    _check(_lib.moe_requant_nvfp4(w.data_ptr(), n, rows, cols, codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
                                  _stream()))
    return codes, scales, g


def profile_begin() -> None:
    """Start timing every kernel the library launches (see moe_profile_begin)."""
    _check(_lib.moe_profile_begin())


def profile_end() -> dict:
    """End the timing session: {kernel kind: (launches, total ms)}."""
    arr = (KernelTimeT * 32)()
    n = _lib.moe_profile_end(arr, 32)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def routed_bytes(layer: DeviceLayer, ids: np.ndarray, T: int) -> int:
    """Algorithmic HBM bytes of one layer pass: the router weight (and bias), the unique
    routed experts named in ``ids``, the shared expert, x and y (BF16)."""
    cfg = layer.cfg
    b = cfg.E * cfg.H * 4 + (cfg.E * 4 if layer.t.get("router_bias") is not None else 0)
    per = layer.nbytes_expert("routed", 0)          # every routed expert has the same size
    b += per * len(np.unique(np.asarray(ids)))
    if cfg.has_shared:
        b += layer.nbytes_expert("shared", 0)
    return b + 2 * T * cfg.H * 2
