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
MOE_REGIME_VERIFY_ONE_LAUNCH = 3

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
                ("sh_gate", moe_nvfp4), ("sh_up", moe_nvfp4), ("sh_down", moe_nvfp4),
                ("norm_w", _c_void_p)]


class moe_route_out(ctypes.Structure):
    _fields_ = [("ids", _c_void_p), ("w", _c_void_p), ("n_unique", _c_void_p), ("uniq", _c_void_p),
                ("off", _c_void_p), ("asg", _c_void_p), ("inv", _c_void_p)]


class moe_greedy_out(ctypes.Structure):
    _fields_ = [("target", _c_void_p), ("target_logit", _c_void_p), ("n_accepted", _c_void_p),
                ("emitted", _c_void_p), ("n_emitted", _c_void_p)]


class moe_dense_weights(ctypes.Structure):
    _fields_ = [("gate", _c_void_p), ("up", _c_void_p), ("down", _c_void_p), ("norm_w", _c_void_p)]


class moe_kv_ring(ctypes.Structure):
    _fields_ = [("k", _c_void_p), ("v", _c_void_p), ("len", _c_void_p), ("n_layers", _i32), ("n_kv", _i32),
                ("head_dim", _i32), ("window", _i32), ("capacity", _i32)]


class moe_debug(ctypes.Structure):
    _fields_ = [("logits", _c_void_p), ("ids", _c_void_p), ("w", _c_void_p), ("n_unique", _c_void_p),
                ("uniq", _c_void_p), ("off", _c_void_p), ("asg", _c_void_p), ("inv", _c_void_p),
                ("x_in", _c_void_p), ("y32", _c_void_p), ("res_in", _c_void_p), ("status", _c_void_p)]


EXPORTS = ["moe_verify_workspace_bytes", "moe_verify_layer", "moe_verify_layer_grouped", "moe_verify_stack",
           "moe_verify_layer_noalloc", "moe_verify_noalloc_scratch_bytes",
           "moe_verify_lm_head_workspace_bytes", "moe_verify_lm_head_greedy",
           "moe_verify_stack_timed", "moe_verify_route", "moe_verify_stream_read",
           "moe_verify_dequant_nvfp4", "moe_stack_graph_create", "moe_stack_graph_launch",
           "moe_stack_graph_destroy", "moe_verify_weight_bytes", "moe_dense_workspace_bytes", "moe_dense_mlp",
           "moe_prefill_workspace_bytes", "moe_prefill_stack", "moe_kv_ring_capacity", "moe_kv_ring_bytes",
           "moe_kv_ring_reset", "moe_kv_ring_write", "moe_kv_ring_write_layer", "moe_kv_ring_commit",
           "moe_kv_ring_window",
           "moe_verify_last_error", "moe_verify_version"]

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
    L.moe_verify_layer_noalloc.restype = ctypes.c_int
    L.moe_verify_layer_noalloc.argtypes = [cfgp, wp, P, _i32, P, P, P, P, ctypes.POINTER(moe_debug)]
    L.moe_verify_noalloc_scratch_bytes.restype = Z
    L.moe_verify_noalloc_scratch_bytes.argtypes = []
    L.moe_verify_lm_head_workspace_bytes.restype = Z
    L.moe_verify_lm_head_workspace_bytes.argtypes = [_i32, _i32]
    L.moe_verify_lm_head_greedy.restype = ctypes.c_int
    L.moe_verify_lm_head_greedy.argtypes = [P, _i32, P, _i32, _i32, P, ctypes.c_float, P,
                                            ctypes.POINTER(moe_greedy_out), P, Z, P]
    L.moe_verify_stack.restype = ctypes.c_int
    L.moe_verify_stack.argtypes = [cfgp, wp, _i32, P, P, _i32, P, P, P, Z, P, ctypes.POINTER(moe_debug)]
    L.moe_verify_stack_timed.restype = ctypes.c_int
    L.moe_verify_stack_timed.argtypes = [cfgp, wp, _i32, P, P, _i32, P, P, P, Z, P, ctypes.POINTER(ctypes.c_float)]
    L.moe_verify_route.restype = ctypes.c_int
    L.moe_verify_route.argtypes = [cfgp, P, P, _i32, ctypes.POINTER(moe_route_out), P, Z, P]
    L.moe_verify_stream_read.restype = ctypes.c_int
    L.moe_verify_stream_read.argtypes = [P, Z, P, P]
    L.moe_verify_dequant_nvfp4.restype = ctypes.c_int
    L.moe_verify_dequant_nvfp4.argtypes = [ctypes.POINTER(moe_nvfp4), _i32, _i32, _i32, P, P]
    L.moe_stack_graph_create.restype = ctypes.c_int
    L.moe_stack_graph_create.argtypes = [cfgp, wp, _i32, P, P, _i32, P, P, P, Z, P, ctypes.POINTER(P)]
    L.moe_stack_graph_launch.restype = ctypes.c_int
    L.moe_stack_graph_launch.argtypes = [P, P]
    L.moe_stack_graph_destroy.restype = None
    L.moe_stack_graph_destroy.argtypes = [P]
    L.moe_verify_weight_bytes.restype = Z
    L.moe_verify_weight_bytes.argtypes = [cfgp, _i32, _i32, _i32, _i32]
    dwp = ctypes.POINTER(moe_dense_weights)
    L.moe_dense_workspace_bytes.restype = Z
    L.moe_dense_workspace_bytes.argtypes = [_i32, _i32, _i32]
    L.moe_dense_mlp.restype = ctypes.c_int
    L.moe_dense_mlp.argtypes = [P, _i32, _i32, _i32, dwp, P, ctypes.c_float, P, P, P, P, Z, P]
    L.moe_prefill_workspace_bytes.restype = Z
    L.moe_prefill_workspace_bytes.argtypes = [cfgp, _i32]
    L.moe_prefill_stack.restype = ctypes.c_int
    L.moe_prefill_stack.argtypes = [cfgp, dwp, _i32, wp, _i32, P, P, _i32, P, P, P, P, Z, P,
                                    ctypes.POINTER(moe_debug)]
    rp = ctypes.POINTER(moe_kv_ring)
    L.moe_kv_ring_capacity.restype = _i32
    L.moe_kv_ring_capacity.argtypes = [_i32, _i32]
    L.moe_kv_ring_bytes.restype = Z
    L.moe_kv_ring_bytes.argtypes = [_i32, _i32, _i32, _i32]
    L.moe_kv_ring_reset.restype = ctypes.c_int
    L.moe_kv_ring_reset.argtypes = [rp, _i32, P]
    L.moe_kv_ring_write.restype = ctypes.c_int
    L.moe_kv_ring_write.argtypes = [rp, P, P, _i32, P]
    L.moe_kv_ring_write_layer.restype = ctypes.c_int
    L.moe_kv_ring_write_layer.argtypes = [rp, _i32, P, P, _i32, P]
    L.moe_kv_ring_commit.restype = ctypes.c_int
    L.moe_kv_ring_commit.argtypes = [rp, P, _i32, P]
    L.moe_kv_ring_window.restype = ctypes.c_int
    L.moe_kv_ring_window.argtypes = [rp, _i32, _i32, P, P, P]
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


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor", numel: Optional[int] = None,
         device: Optional[torch.device] = None) -> Optional[int]:
    """Device pointer of a contiguous GPU tensor, after checking its dtype,
    its size (at least numel elements) and that it lives on `device` (when
    given).  Raises before anything reaches the library: a host pointer or a
    short buffer would otherwise become an out-of-bounds GPU access."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (is on %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the call's tensors are on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s has %d elements, needs at least %d" % (name, t.numel(), numel))
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


def _check_mat(m, name: str, E: int, rows: int, cols: int, device, shapes_only: bool = False) -> None:
    want = {"q": (E, rows, cols // 2), "s": (E, rows, cols // 16), "ts": (E,)}
    for k, shp in want.items():
        t = m[k]
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != shp:
            raise ValueError("%s.%s has shape %s, expected %s" % (
                name, k, None if not isinstance(t, torch.Tensor) else tuple(t.shape), shp))
        if not shapes_only:
            _ptr(t, torch.float32 if k == "ts" else torch.uint8, "%s.%s" % (name, k), device=device)


def _mat(m, name: str = "matrix") -> moe_nvfp4:
    if m is None:
        return moe_nvfp4(None, None, None)
    return moe_nvfp4(_ptr(m["q"], torch.uint8, name + ".q"), _ptr(m["s"], torch.uint8, name + ".s"),
                     _ptr(m["ts"], torch.float32, name + ".ts"))


def check_weights(w: Dict[str, object], cfg: moe_cfg, device=None) -> None:
    """Shapes, dtypes and device of one layer's weight tensors against cfg
    (every shape first, then dtypes and devices)."""
    H, E, I, Is = cfg.hidden, cfg.n_experts, cfg.inter, cfg.shared_inter
    mats = [("gate", E, I, H), ("up", E, I, H), ("down", E, H, I)]
    if Is > 0:
        mats += [("sh_gate", 1, Is, H), ("sh_up", 1, Is, H), ("sh_down", 1, H, Is)]
    rw = w["router_w"]
    if not isinstance(rw, torch.Tensor) or tuple(rw.shape) != (E, H):
        raise ValueError("router_w must have shape (%d, %d)" % (E, H))
    for nm, e, rows, cols in mats:
        if w.get(nm) is None:
            raise ValueError("%s missing" % nm)
        _check_mat(w[nm], nm, e, rows, cols, device, shapes_only=True)
    _ptr(rw, _BITS16, "router_w", device=device)
    if w.get("router_bias") is not None:
        _ptr(w["router_bias"], torch.float32, "router_bias", numel=E, device=device)
    for nm, e, rows, cols in mats:
        _check_mat(w[nm], nm, e, rows, cols, device)
    if w.get("norm_w") is not None:
        _ptr(w["norm_w"], _BITS16, "norm_w", numel=H, device=device)


def make_weights(w: Dict[str, object], cfg: Optional[moe_cfg] = None) -> moe_layer_weights:
    """Weight struct for one layer from a dict of device tensors (the layout
    documented in include/moe_verify.h; 'norm_w' optional).  With cfg, the
    tensors' shapes are checked against it.  The tensors must stay alive."""
    if cfg is not None:
        check_weights(w, cfg)
    return moe_layer_weights(_ptr(w["router_w"], _BITS16, "router_w"),
                             _ptr(w.get("router_bias"), torch.float32, "router_bias"),
                             _mat(w["gate"], "gate"), _mat(w["up"], "up"), _mat(w["down"], "down"),
                             _mat(w.get("sh_gate"), "sh_gate"), _mat(w.get("sh_up"), "sh_up"),
                             _mat(w.get("sh_down"), "sh_down"), _ptr(w.get("norm_w"), _BITS16, "norm_w"))


# per-layer sizes of the debug arrays, in elements, for K rows
def _debug_sizes(cfg: moe_cfg, K: int) -> Dict[str, int]:
    n, H = K * cfg.top_k, cfg.hidden
    return {"logits": K * cfg.n_experts, "ids": n, "w": n, "n_unique": 1, "uniq": n, "off": n + 1, "asg": n,
            "inv": n, "x_in": K * H, "y32": K * H, "res_in": K * H, "status": 1}


def make_debug(**arrays) -> moe_debug:
    d = moe_debug()
    for k, v in arrays.items():
        if v is not None and not isinstance(v, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % k)
        setattr(d, k, None if v is None else v.data_ptr())
    d._tensors = dict(arrays)
    return d


def _check_debug(debug: Optional[moe_debug], cfg: moe_cfg, K: int, layers: int, device) -> None:
    if debug is None:
        return
    sizes = _debug_sizes(cfg, K)
    for k, t in getattr(debug, "_tensors", {}).items():
        if k not in sizes:
            raise ValueError("unknown debug array %s" % k)
        _ptr(t, None, "debug." + k, numel=sizes[k] * layers, device=device)


def _rows(x: torch.Tensor, cfg: moe_cfg, name: str = "x") -> int:
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != cfg.hidden:
        raise ValueError("%s must be a 2-D tensor [K, %d]" % (name, cfg.hidden))
    return x.shape[0]


def _ws(workspace: torch.Tensor, device) -> tuple:
    _ptr(workspace, None, "workspace", device=device)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


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


def _layer_call(fn, cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                workspace: torch.Tensor, y32, residual, debug, stream) -> None:
    K = _rows(x, cfg)
    dev = x.device
    KH = K * cfg.hidden
    px = _ptr(x, _BITS16, "x", device=dev)
    py = _ptr(y, _BITS16, "y", numel=KH, device=dev)
    py32 = _ptr(y32, torch.float32, "y32", numel=KH, device=dev)
    pr = _ptr(residual, _BITS16, "residual", numel=KH, device=dev)
    _check_debug(debug, cfg, K, 1, dev)
    pw, nw = _ws(workspace, dev)
    _check(fn(ctypes.byref(cfg), ctypes.byref(weights), px, K, pr, py, py32, pw, nw, _stream(stream),
              ctypes.byref(debug) if debug is not None else None))


def moe_verify_layer(cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                     workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                     residual: Optional[torch.Tensor] = None, debug: Optional[moe_debug] = None,
                     stream=None) -> None:
    _layer_call(lib().moe_verify_layer, cfg, weights, x, y, workspace, y32, residual, debug, stream)


def moe_verify_layer_grouped(cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                             workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                             residual: Optional[torch.Tensor] = None, debug: Optional[moe_debug] = None,
                             stream=None) -> None:
    _layer_call(lib().moe_verify_layer_grouped, cfg, weights, x, y, workspace, y32, residual, debug, stream)


def moe_verify_layer_noalloc(cfg: moe_cfg, weights: moe_layer_weights, x: torch.Tensor, y: torch.Tensor,
                             y32: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                             debug: Optional[moe_debug] = None, stream=None) -> None:
    """moe_verify_layer on the library's fixed scratch array (no workspace)."""
    K = _rows(x, cfg)
    dev = x.device
    KH = K * cfg.hidden
    px = _ptr(x, _BITS16, "x", device=dev)
    py = _ptr(y, _BITS16, "y", numel=KH, device=dev)
    py32 = _ptr(y32, torch.float32, "y32", numel=KH, device=dev)
    pr = _ptr(residual, _BITS16, "residual", numel=KH, device=dev)
    _check_debug(debug, cfg, K, 1, dev)
    _check(lib().moe_verify_layer_noalloc(ctypes.byref(cfg), ctypes.byref(weights), px, K, pr, py, py32,
                                          _stream(stream), ctypes.byref(debug) if debug is not None else None))


def moe_verify_noalloc_scratch_bytes() -> int:
    return lib().moe_verify_noalloc_scratch_bytes()


def _layer_array(layers: Sequence[moe_layer_weights]):
    arr = (moe_layer_weights * len(layers))(*layers)
    return arr


def _stack_io(cfg: moe_cfg, layers, x, y, y32, residual):
    if len(layers) < 1:
        raise ValueError("need at least one layer")
    K = _rows(x, cfg)
    dev = x.device
    KH = K * cfg.hidden
    return (K, dev, _ptr(x, _BITS16, "x", device=dev), _ptr(residual, _BITS16, "residual", numel=KH, device=dev),
            _ptr(y, _BITS16, "y", numel=KH, device=dev), _ptr(y32, torch.float32, "y32", numel=KH, device=dev))


def moe_verify_stack(cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                     workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                     debug: Optional[moe_debug] = None, stream=None,
                     residual: Optional[torch.Tensor] = None) -> None:
    K, dev, px, pr, py, py32 = _stack_io(cfg, layers, x, y, y32, residual)
    _check_debug(debug, cfg, K, len(layers), dev)
    pw, nw = _ws(workspace, dev)
    arr = _layer_array(layers)
    _check(lib().moe_verify_stack(ctypes.byref(cfg), arr, len(layers), px, pr, K, py, py32, pw, nw,
                                  _stream(stream), ctypes.byref(debug) if debug is not None else None))


def moe_verify_stack_timed(cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                           workspace: torch.Tensor, y32: Optional[torch.Tensor] = None, stream=None,
                           residual: Optional[torch.Tensor] = None):
    """Returns per-kernel durations in ms as a list of (router + gate/up,
    down) per layer."""
    K, dev, px, pr, py, py32 = _stack_io(cfg, layers, x, y, y32, residual)
    pw, nw = _ws(workspace, dev)
    arr = _layer_array(layers)
    ms = (ctypes.c_float * (2 * len(layers)))()
    _check(lib().moe_verify_stack_timed(ctypes.byref(cfg), arr, len(layers), px, pr, K, py, py32, pw, nw,
                                        _stream(stream), ms))
    return [(ms[2 * l], ms[2 * l + 1]) for l in range(len(layers))]


def moe_verify_route(cfg: moe_cfg, logits: torch.Tensor, out: Dict[str, torch.Tensor],
                     bias: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2 or logits.shape[1] != cfg.n_experts:
        raise ValueError("logits must be a 2-D tensor [K, %d]" % cfg.n_experts)
    K, dev = logits.shape[0], logits.device
    n = K * cfg.top_k
    sizes = {"ids": n, "w": n, "n_unique": 1, "uniq": n, "off": n + 1, "asg": n, "inv": n}
    ro = moe_route_out(*[_ptr(out[k], None, k, numel=sizes[k], device=dev)
                         for k in ("ids", "w", "n_unique", "uniq", "off", "asg", "inv")])
    pw, nw = (None, 0) if workspace is None else _ws(workspace, dev)
    _check(lib().moe_verify_route(ctypes.byref(cfg), _ptr(logits, torch.float32, "logits", device=dev),
                                  _ptr(bias, torch.float32, "bias", numel=cfg.n_experts, device=dev), K,
                                  ctypes.byref(ro), pw, nw, _stream(stream)))


def moe_verify_dequant_nvfp4(m: Dict[str, torch.Tensor], out: torch.Tensor, stream=None) -> None:
    E, rows, half = m["q"].shape
    dev = m["q"].device
    _check_mat(m, "matrix", E, rows, half * 2, dev)
    mm = _mat(m)
    _check(lib().moe_verify_dequant_nvfp4(ctypes.byref(mm), E, rows, half * 2,
                                          _ptr(out, torch.float32, "out", numel=E * rows * half * 2, device=dev),
                                          _stream(stream)))


def moe_verify_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream every byte of src (a GPU tensor, size a multiple of 16 bytes)
    once; sink: a one-element int32 GPU tensor."""
    dev = src.device
    nbytes = src.numel() * src.element_size()
    _check(lib().moe_verify_stream_read(_ptr(src, None, "src", device=dev), nbytes,
                                        _ptr(sink, torch.int32, "sink", numel=1, device=dev), _stream(stream)))


def moe_verify_lm_head_workspace_bytes(vocab: int, K: int) -> int:
    n = lib().moe_verify_lm_head_workspace_bytes(vocab, K)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID, moe_verify_last_error())
    return n


GREEDY_FIELDS = ("target", "target_logit", "n_accepted", "emitted", "n_emitted")


def alloc_greedy_out(K: int, device="cuda") -> Dict[str, torch.Tensor]:
    return {"target": torch.empty(K, dtype=torch.int32, device=device),
            "target_logit": torch.empty(K, dtype=torch.float32, device=device),
            "n_accepted": torch.empty(1, dtype=torch.int32, device=device),
            "emitted": torch.empty(K, dtype=torch.int32, device=device),
            "n_emitted": torch.empty(1, dtype=torch.int32, device=device)}


def moe_verify_lm_head_greedy(x: torch.Tensor, w: torch.Tensor, out: Dict[str, torch.Tensor],
                              workspace: torch.Tensor, draft: Optional[torch.Tensor] = None,
                              tie_tol: float = 1e-6, logits: Optional[torch.Tensor] = None, stream=None) -> None:
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [K, hidden]")
    if not isinstance(w, torch.Tensor) or w.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError("w must be a 2-D tensor [vocab, %d]" % x.shape[1])
    K, H = x.shape
    V = w.shape[0]
    dev = x.device
    sizes = {"target": K, "target_logit": K, "n_accepted": 1, "emitted": K, "n_emitted": 1}
    types = {"target": torch.int32, "target_logit": torch.float32, "n_accepted": torch.int32,
             "emitted": torch.int32, "n_emitted": torch.int32}
    go = moe_greedy_out(*[_ptr(out[k], types[k], k, numel=sizes[k], device=dev) for k in GREEDY_FIELDS])
    pd = _ptr(draft, torch.int32, "draft", numel=K - 1, device=dev) if K > 1 else None
    pw, nw = _ws(workspace, dev)
    _check(lib().moe_verify_lm_head_greedy(_ptr(x, _BITS16, "x", device=dev), K, _ptr(w, _BITS16, "w", device=dev),
                                           V, H, pd, float(tie_tol),
                                           _ptr(logits, torch.float32, "logits", numel=K * V, device=dev),
                                           ctypes.byref(go), pw, nw, _stream(stream)))


# ---------------------------------------------------------------------------
# the dense first layer and the prefill stack
# ---------------------------------------------------------------------------


def make_dense_weights(w: Dict[str, object], hidden: Optional[int] = None) -> moe_dense_weights:
    """ctypes view of the dense layer's bf16 weights (w['gate'], w['up']
    [inter, hidden], w['down'] [hidden, inter], optional w['norm_w'] [hidden]),
    after checking their shapes and that they share one GPU."""
    g, u, d = w["gate"], w["up"], w["down"]
    for name, t in (("gate", g), ("up", u), ("down", d)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("dense %s must be a 2-D tensor" % name)
    I, H = g.shape
    if hidden is not None and H != hidden:
        raise ValueError("dense gate has %d columns, hidden is %d" % (H, hidden))
    if tuple(u.shape) != (I, H) or tuple(d.shape) != (H, I):
        raise ValueError("dense up %s / down %s do not match gate %s" % (tuple(u.shape), tuple(d.shape), (I, H)))
    dev = g.device
    nw = w.get("norm_w")
    return moe_dense_weights(_ptr(g, _BITS16, "dense gate", device=dev), _ptr(u, _BITS16, "dense up", device=dev),
                             _ptr(d, _BITS16, "dense down", device=dev),
                             _ptr(nw, _BITS16, "dense norm_w", numel=H, device=dev))


def moe_dense_workspace_bytes(hidden: int, inter: int, max_rows: int) -> int:
    n = lib().moe_dense_workspace_bytes(hidden, inter, max_rows)
    if n == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, moe_verify_last_error())
    return n


def moe_dense_mlp(x: torch.Tensor, w: Dict[str, object], y: torch.Tensor, y32: torch.Tensor,
                  workspace: torch.Tensor, residual: Optional[torch.Tensor] = None, eps: float = 1e-6,
                  x_next: Optional[torch.Tensor] = None, stream=None) -> None:
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, hidden]")
    T, H = x.shape
    dw = make_dense_weights(w, H)
    I = w["gate"].shape[0]
    dev = x.device
    pw, nw = _ws(workspace, dev)
    _check(lib().moe_dense_mlp(_ptr(x, _BITS16, "x", device=dev), T, H, I, ctypes.byref(dw),
                               _ptr(residual, _BITS16, "residual", numel=T * H, device=dev), float(eps),
                               _ptr(y, _BITS16, "y", numel=T * H, device=dev),
                               _ptr(y32, torch.float32, "y32", numel=T * H, device=dev),
                               _ptr(x_next, _BITS16, "x_next", numel=T * H, device=dev), pw, nw, _stream(stream)))


def moe_prefill_workspace_bytes(cfg: moe_cfg, dense_inter: int) -> int:
    n = lib().moe_prefill_workspace_bytes(ctypes.byref(cfg), dense_inter)
    if n == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, moe_verify_last_error())
    return n


def moe_prefill_stack(cfg: moe_cfg, dense: Dict[str, object], layers: Sequence[moe_layer_weights], x: torch.Tensor,
                      y: torch.Tensor, workspace: torch.Tensor, y32: Optional[torch.Tensor] = None,
                      dense_y32: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                      debug: Optional[moe_debug] = None, stream=None) -> None:
    """The dense first layer, then the MoE layers (moe_prefill_stack)."""
    T, dev, px, pr, py, py32 = _stack_io(cfg, layers, x, y, y32, residual)
    _check_debug(debug, cfg, T, len(layers), dev)
    dw = make_dense_weights(dense, cfg.hidden)
    I = dense["gate"].shape[0]
    pw, nw = _ws(workspace, dev)
    arr = _layer_array(layers)
    _check(lib().moe_prefill_stack(ctypes.byref(cfg), ctypes.byref(dw), I, arr, len(layers), px, pr, T, py, py32,
                                   _ptr(dense_y32, torch.float32, "dense_y32", numel=T * cfg.hidden, device=dev),
                                   pw, nw, _stream(stream), ctypes.byref(debug) if debug is not None else None))


# ---------------------------------------------------------------------------
# the sliding-window KV ring of the verify step
# ---------------------------------------------------------------------------


class KvRing:
    """Device tensors of one sequence's sliding-window KV ring (keys and
    values bf16 [n_layers, n_kv, capacity, head_dim], the int32 committed
    length) and the calls on it."""

    def __init__(self, n_layers: int, n_kv: int, head_dim: int, window: int, max_rows: int, device):
        cap = lib().moe_kv_ring_capacity(window, max_rows)
        if cap == 0:
            raise MoEError(MOE_ERR_INVALID, moe_verify_last_error())
        self.shape = (n_layers, n_kv, cap, head_dim)
        self.k = torch.zeros(self.shape, dtype=torch.int16, device=device)
        self.v = torch.zeros(self.shape, dtype=torch.int16, device=device)
        self.len = torch.zeros(1, dtype=torch.int32, device=device)
        self.window, self.device = window, self.k.device
        self.ring = moe_kv_ring(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr(), n_layers, n_kv,
                                head_dim, window, cap)

    def reset(self, length: int = 0, stream=None) -> None:
        _check(lib().moe_kv_ring_reset(ctypes.byref(self.ring), length, _stream(stream)))

    def write(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        """k_new, v_new: bf16 [n_layers, K, n_kv, head_dim]."""
        L, n_kv, _, D = self.shape
        if k_new.dim() != 4 or tuple(k_new.shape) != (L, k_new.shape[1], n_kv, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [%d, K, %d, %d] (got %s, %s)" % (L, n_kv, D, tuple(k_new.shape),
                                                                                 tuple(v_new.shape)))
        K = k_new.shape[1]
        _check(lib().moe_kv_ring_write(ctypes.byref(self.ring), _ptr(k_new, _BITS16, "k_new", device=self.device),
                                       _ptr(v_new, _BITS16, "v_new", device=self.device), K, _stream(stream)))

    def write_layer(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        """k_new, v_new: bf16 [K, n_kv, head_dim], the block's rows of one
        layer."""
        _, n_kv, _, D = self.shape
        if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (n_kv, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [K, %d, %d] (got %s, %s)" % (n_kv, D, tuple(k_new.shape),
                                                                             tuple(v_new.shape)))
        K = k_new.shape[0]
        _check(lib().moe_kv_ring_write_layer(ctypes.byref(self.ring), layer,
                                             _ptr(k_new, _BITS16, "k_new", device=self.device),
                                             _ptr(v_new, _BITS16, "v_new", device=self.device), K, _stream(stream)))

    def commit(self, n_accepted: torch.Tensor, K: int, stream=None) -> None:
        """n_accepted: device int32 [1] (e.g. the greedy step's count)."""
        _check(lib().moe_kv_ring_commit(ctypes.byref(self.ring),
                                        _ptr(n_accepted, torch.int32, "n_accepted", numel=1, device=self.device),
                                        K, _stream(stream)))

    def window_of(self, layer: int, K: int, stream=None):
        """(keys, values) bf16 [K, n_kv, window, head_dim]: what each row of
        the last written block sees of `layer`."""
        _, n_kv, _, D = self.shape
        ko = torch.empty(K, n_kv, self.window, D, dtype=torch.int16, device=self.device)
        vo = torch.empty_like(ko)
        _check(lib().moe_kv_ring_window(ctypes.byref(self.ring), layer, K, ko.data_ptr(), vo.data_ptr(),
                                        _stream(stream)))
        return ko, vo


class StackGraph:
    """moe_stack_graph_create / _launch / _destroy."""

    def __init__(self, cfg: moe_cfg, layers: Sequence[moe_layer_weights], x: torch.Tensor, y: torch.Tensor,
                 workspace: torch.Tensor, y32: Optional[torch.Tensor] = None, stream=None,
                 residual: Optional[torch.Tensor] = None):
        self.handle = _c_void_p()
        self._keep = (cfg, list(layers), x, y, workspace, y32, residual)
        K, dev, px, pr, py, py32 = _stack_io(cfg, layers, x, y, y32, residual)
        pw, nw = _ws(workspace, dev)
        arr = _layer_array(layers)
        h = _c_void_p()
        _check(lib().moe_stack_graph_create(ctypes.byref(cfg), arr, len(layers), px, pr, K, py, py32, pw, nw,
                                            _stream(stream), ctypes.byref(h)))
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
