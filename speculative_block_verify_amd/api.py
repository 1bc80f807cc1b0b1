"""Thin ctypes binding of libmoeverify.so (include/moe_verify.h).

Each ``moe_verify_*`` function here has the name of the C entry point it
calls and only marshals arguments: torch tensors become device pointers,
the current torch stream becomes the HIP stream.  All computation runs in
the HIP library; if the library is missing, loading raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeverify.so")

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_WORKSPACE = -4
MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID_BIAS = 1
MOE_REGIME_AUTO = 0
MOE_REGIME_VERIFY = 1
MOE_REGIME_GROUPED = 2

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class moe_nvfp4(ctypes.Structure):
    _fields_ = [("q", _c_void_p), ("s", _c_void_p), ("ts", _c_void_p)]


class moe_cfg(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("n_experts", _i32), ("top_k", _i32), ("inter", _i32),
                ("shared_inter", _i32), ("score_fn", _i32), ("norm_topk", _i32),
                ("routed_scale", ctypes.c_float), ("rms_eps", ctypes.c_float), ("max_rows", _i32),
                ("regime", _i32)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("router_w", _c_void_p), ("router_bias", _c_void_p),
                ("gate", moe_nvfp4), ("up", moe_nvfp4), ("down", moe_nvfp4),
                ("sh_gate", moe_nvfp4), ("sh_up", moe_nvfp4), ("sh_down", moe_nvfp4)]


class moe_route_out(ctypes.Structure):
    _fields_ = [("ids", _c_void_p), ("w", _c_void_p), ("n_unique", _c_void_p), ("uniq", _c_void_p),
                ("off", _c_void_p), ("asg", _c_void_p), ("inv", _c_void_p)]


class moe_debug(ctypes.Structure):
    _fields_ = [("logits", _c_void_p), ("ids", _c_void_p), ("w", _c_void_p), ("n_unique", _c_void_p),
                ("uniq", _c_void_p), ("off", _c_void_p), ("asg", _c_void_p), ("inv", _c_void_p),
                ("x_in", _c_void_p), ("y32", _c_void_p)]


EXPORTS = ["moe_verify_workspace_bytes", "moe_verify_layer", "moe_verify_layer_grouped", "moe_verify_stack",
           "moe_verify_stack_timed", "moe_verify_route",
           "moe_verify_dequant_nvfp4", "moe_stack_graph_create", "moe_stack_graph_launch",
           "moe_stack_graph_destroy", "moe_verify_weight_bytes", "moe_verify_last_error",
           "moe_verify_version"]

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoeverify.so is not built: run `python -m speculative_block_verify_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, Z = _c_void_p, ctypes.c_size_t
    cfgp = ctypes.POINTER(moe_cfg)
    wp = ctypes.POINTER(moe_layer_weights)
    L.moe_verify_workspace_bytes.restype = Z
    L.moe_verify_workspace_bytes.argtypes = [cfgp]
    L.moe_verify_layer.restype = ctypes.c_int
    L.moe_verify_layer.argtypes = [cfgp, wp, P, _i32, P, P, P, P, Z, P, ctypes.POINTER(moe_debug)]
    L.moe_verify_layer_grouped.restype = ctypes.c_int
    L.moe_verify_layer_grouped.argtypes = [cfgp, wp, P, _i32, P, P, P, P, Z, P, ctypes.POINTER(moe_debug)]
    L.moe_verify_stack.restype = ctypes.c_int
    L.moe_verify_stack.argtypes = [cfgp, wp, _i32, P, _i32, P, P, P, Z, P, ctypes.POINTER(moe_debug)]
    L.moe_verify_stack_timed.restype = ctypes.c_int
    L.moe_verify_stack_timed.argtypes = [cfgp, wp, _i32, P, _i32, P, P, P, Z, P, ctypes.POINTER(ctypes.c_float)]
    L.moe_verify_route.restype = ctypes.c_int
    L.moe_verify_route.argtypes = [cfgp, P, P, _i32, ctypes.POINTER(moe_route_out), P, Z, P]
    L.moe_verify_dequant_nvfp4.restype = ctypes.c_int
    L.moe_verify_dequant_nvfp4.argtypes = [ctypes.POINTER(moe_nvfp4), _i32, _i32, _i32, P, P]
    L.moe_stack_graph_create.restype = ctypes.c_int
    L.moe_stack_graph_create.argtypes = [cfgp, wp, _i32, P, _i32, P, P, P, Z, P, ctypes.POINTER(P)]
    L.moe_stack_graph_launch.restype = ctypes.c_int
    L.moe_stack_graph_launch.argtypes = [P, P]
    L.moe_stack_graph_destroy.restype = None
    L.moe_stack_graph_destroy.argtypes = [P]
    L.moe_verify_weight_bytes.restype = Z
    L.moe_verify_weight_bytes.argtypes = [cfgp, _i32, _i32, _i32, _i32]
    L.moe_verify_last_error.restype = ctypes.c_char_p
    L.moe_verify_last_error.argtypes = []
    L.moe_verify_version.restype = ctypes.c_int
    L.moe_verify_version.argtypes = []
    _lib = L
    return L


class MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("moe_verify error %d: %s" % (code, msg))
        self.code = code


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoEError(rc, moe_verify_last_error())


# ---------------------------------------------------------------------------
# marshalling
# ---------------------------------------------------------------------------


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


_BITS16 = (torch.int16, torch.uint16, torch.bfloat16)


def _stream(stream=None):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def make_cfg(shape, max_rows: int, score_fn: int = MOE_SCORE_SOFTMAX, norm_topk: int = 1,
             routed_scale: float = 1.0, rms_eps: float = 1e-6, regime: int = MOE_REGIME_AUTO) -> moe_cfg:
    return moe_cfg(shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter,
                   score_fn, norm_topk, routed_scale, rms_eps, max_rows, regime)


def _mat(m) -> moe_nvfp4:
    if m is None:
        return moe_nvfp4(None, None, None)
    return moe_nvfp4(_ptr(m["q"], torch.uint8, "q"), _ptr(m["s"], torch.uint8, "s"),
                     _ptr(m["ts"], torch.float32, "ts"))


def make_weights(w: Dict[str, object]) -> moe_layer_weights:
    """Weight struct for one layer from a dict of device tensors (the layout
    documented in include/moe_verify.h).  The tensors must stay alive."""
    return moe_layer_weights(_ptr(w["router_w"], _BITS16, "router_w"),
                             _ptr(w.get("router_bias"), torch.float32, "router_bias"),
                             _mat(w["gate"]), _mat(w["up"]), _mat(w["down"]),
                             _mat(w.get("sh_gate")), _mat(w.get("sh_up")), _mat(w.get("sh_down")))


def make_debug(**arrays) -> moe_debug:
    d = moe_debug()
    for k, v in arrays.items():
        setattr(d, k, _ptr(v, None, k))
    return d


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------


def moe_verify_version() -> int:
    return lib().moe_verify_version()


def moe_verify_last_error() -> str:
    return lib().moe_verify_last_error().decode()


def moe_verify_workspace_bytes(cfg: moe_cfg) -> int:
    n = lib().moe_verify_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MoEError(MOE_ERR_INVALID, moe_verify_last_error())
    return n


def moe_verify_weight_bytes(cfg: moe_cfg, n_unique: int, K: int, with_shared: bool = True,
                            with_router: bool = True) -> int:
    return lib().moe_verify_weight_bytes(ctypes.byref(cfg), n_unique, K, int(with_shared), int(with_router))


def moe_verify_layer(cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                     workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                     residual: Optional[torch.Tensor] = None, debug: Optional[moe_debug] = None,
                     stream=None) -> None:
    K = x.shape[0]
    _check(lib().moe_verify_layer(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x, _BITS16, "x"), K,
                                  _ptr(residual, _BITS16, "residual"), _ptr(y, _BITS16, "y"),
                                  _ptr(y32, torch.float32, "y32"), _ptr(workspace, None, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream),
                                  ctypes.byref(debug) if debug is not None else None))


def moe_verify_layer_grouped(cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                             workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                             residual: Optional[torch.Tensor] = None, debug: Optional[moe_debug] = None,
                             stream=None) -> None:
    K = x.shape[0]
    _check(lib().moe_verify_layer_grouped(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x, _BITS16, "x"), K,
                                          _ptr(residual, _BITS16, "residual"), _ptr(y, _BITS16, "y"),
                                          _ptr(y32, torch.float32, "y32"), _ptr(workspace, None, "workspace"),
                                          workspace.numel() * workspace.element_size(), _stream(stream),
                                          ctypes.byref(debug) if debug is not None else None))


def _layer_array(layers: Sequence[moe_layer_weights]):
    arr = (moe_layer_weights * len(layers))(*layers)
    return arr


def moe_verify_stack(cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                     workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                     debug: Optional[moe_debug] = None, stream=None) -> None:
    arr = _layer_array(layers)
    _check(lib().moe_verify_stack(ctypes.byref(cfg), arr, len(layers), _ptr(x, _BITS16, "x"), x.shape[0],
                                  _ptr(y, _BITS16, "y"), _ptr(y32, torch.float32, "y32"),
                                  _ptr(workspace, None, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream),
                                  ctypes.byref(debug) if debug is not None else None))


def moe_verify_stack_timed(cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                           workspace: torch.Tensor, y32: Optional[torch.Tensor] = None, stream=None):
    """Returns per-kernel durations in ms as a list of (route, gateup, down)
    per layer."""
    arr = _layer_array(layers)
    ms = (ctypes.c_float * (3 * len(layers)))()
    _check(lib().moe_verify_stack_timed(ctypes.byref(cfg), arr, len(layers), _ptr(x, _BITS16, "x"), x.shape[0],
                                        _ptr(y, _BITS16, "y"), _ptr(y32, torch.float32, "y32"),
                                        _ptr(workspace, None, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream), ms))
    return [(ms[3 * l], ms[3 * l + 1], ms[3 * l + 2]) for l in range(len(layers))]


def moe_verify_route(cfg: moe_cfg, logits: torch.Tensor, out: Dict[str, torch.Tensor],
                     bias: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    ro = moe_route_out(*[_ptr(out[k], None, k) for k in ("ids", "w", "n_unique", "uniq", "off", "asg", "inv")])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_verify_route(ctypes.byref(cfg), _ptr(logits, torch.float32, "logits"),
                                  _ptr(bias, torch.float32, "bias"), logits.shape[0], ctypes.byref(ro),
                                  _ptr(workspace, None, "workspace"), nbytes, _stream(stream)))


def moe_verify_dequant_nvfp4(m: Dict[str, torch.Tensor], out: torch.Tensor, stream=None) -> None:
    E, rows, half = m["q"].shape
    mm = _mat(m)
    _check(lib().moe_verify_dequant_nvfp4(ctypes.byref(mm), E, rows, half * 2, _ptr(out, torch.float32, "out"),
                                          _stream(stream)))


class StackGraph:
    """moe_stack_graph_create / _launch / _destroy."""

    def __init__(self, cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                 workspace: torch.Tensor, y32: Optional[torch.Tensor] = None, stream=None):
        self._keep = (cfg, list(layers), x, y, workspace, y32)
        arr = _layer_array(layers)
        h = _c_void_p()
        _check(lib().moe_stack_graph_create(ctypes.byref(cfg), arr, len(layers), _ptr(x, _BITS16, "x"),
                                            x.shape[0], _ptr(y, _BITS16, "y"), _ptr(y32, torch.float32, "y32"),
                                            _ptr(workspace, None, "workspace"),
                                            workspace.numel() * workspace.element_size(), _stream(stream),
                                            ctypes.byref(h)))
        self.handle = h

    def launch(self, stream=None) -> None:
        _check(lib().moe_stack_graph_launch(self.handle, _stream(stream)))

    def close(self) -> None:
        if self.handle:
            lib().moe_stack_graph_destroy(self.handle)
            self.handle = _c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_stack_graph_create(*args, **kwargs) -> StackGraph:
    return StackGraph(*args, **kwargs)


# ---------------------------------------------------------------------------
# conveniences for callers holding torch tensors
# ---------------------------------------------------------------------------


def alloc_workspace(cfg: moe_cfg, device="cuda") -> torch.Tensor:
    n = moe_verify_workspace_bytes(cfg)
    return torch.empty(n, dtype=torch.uint8, device=device)


def to_device(w: Dict[str, object], device="cuda") -> Dict[str, object]:
    out = {}
    for k, v in w.items():
        if v is None:
            out[k] = None
        elif isinstance(v, dict):
            out[k] = {kk: vv.to(device).contiguous() for kk, vv in v.items()}
        else:
            out[k] = v.to(device).contiguous()
    return out
