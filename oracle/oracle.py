"""ctypes front end of the C oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the CPU
baseline of bench.py.  It marshals numpy arrays into the single-threaded C
oracle and back; every piece of arithmetic lives in the C file.

Byte accounting (``nvfp4_matrix_bytes`` / ``layer_bytes``) restates the
layout the pages' byte budget implies: PR #844 section 2 ("Where the time
goes") and section 8 (16 expert tiles per layer ~9.4 MB; 1.10 GB routed per
step at two rows, 0.55 GB at one).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants mistakes in a copy of the C source points this at the
# mutated build; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("SBV_ORACLE_LIB")

SCORE_SOFTMAX = 0
SCORE_SIGMOID_BIAS = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, -O2, no fast-math)."""
    if _LIB_OVERRIDE:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        D, I, F, P = ctypes.c_double, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        L.orc_e2m1.restype = D; L.orc_e2m1.argtypes = [I]
        L.orc_e4m3fn.restype = D; L.orc_e4m3fn.argtypes = [I]
        L.orc_bf16.restype = D; L.orc_bf16.argtypes = [I]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16; L.orc_f32_to_bf16.argtypes = [F]
        L.orc_nvfp4_weight.restype = D
        L.orc_nvfp4_weight.argtypes = [P, P, P, I, I, I, I, I]
        L.orc_nvfp4_dequant.restype = None
        L.orc_nvfp4_dequant.argtypes = [P, P, P, I, I, I, P]
        L.orc_router.restype = None; L.orc_router.argtypes = [P, P, I, I, I, P]
        L.orc_key.restype = F; L.orc_key.argtypes = [F, P, I, I]
        L.orc_topk.restype = None; L.orc_topk.argtypes = [P, P, I, I, I, I, I, P, P]
        L.orc_dedup.restype = I; L.orc_dedup.argtypes = [P, I, I, P, P, P, P]
        L.orc_expert_ffn.restype = None
        L.orc_expert_ffn.argtypes = [P, I, I] + [P, P, P] * 3 + [I, P]
        L.orc_moe_layer.restype = None
        L.orc_moe_layer.argtypes = [I] * 8 + [D, P, P, P] + [P, P, P] * 6 + [P, P, P, P, P]
        L.orc_rmsnorm_bf16.restype = None; L.orc_rmsnorm_bf16.argtypes = [P, I, I, D, P, P]
        L.orc_bf16_round.restype = None; L.orc_bf16_round.argtypes = [P, I, P]
        L.orc_lm_head.restype = None; L.orc_lm_head.argtypes = [P, P, I, I, I, P]
        L.orc_greedy_accept.restype = I; L.orc_greedy_accept.argtypes = [P, I, I, P, D, P, P, P]
        L.orc_dense_mlp.restype = None; L.orc_dense_mlp.argtypes = [P, I, I, I, P, P, P, P, P]
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _np(t, dtype) -> np.ndarray:
    """torch tensor / numpy array -> contiguous numpy array of dtype (bit view
    for the integer types)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(t)
    if a.dtype != dtype:
        if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return a


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mat(m) -> Optional[Dict[str, np.ndarray]]:
    if m is None:
        return None
    return {"q": _np(m["q"], np.uint8), "s": _np(m["s"], np.uint8), "ts": _np(m["ts"], np.float32)}


# ---------------------------------------------------------------------------
# elementwise decoders
# ---------------------------------------------------------------------------


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def e4m3fn(byte: int) -> float:
    return lib().orc_e4m3fn(int(byte))


def bf16(bits: int) -> float:
    return lib().orc_bf16(int(bits))


def f32_to_bf16(f: float) -> int:
    return int(lib().orc_f32_to_bf16(float(f)))


def dequant(mat, e: int) -> np.ndarray:
    """Expert e of an NVFP4 matrix as float64 [rows, cols]."""
    m = _mat(mat)
    E, rows, half = m["q"].shape
    cols = half * 2
    out = np.empty((rows, cols), np.float64)
    lib().orc_nvfp4_dequant(_p(m["q"]), _p(m["s"]), _p(m["ts"]), rows, cols, e, _p(out))
    return out


# ---------------------------------------------------------------------------
# steps of the layer
# ---------------------------------------------------------------------------


def router(x, router_w) -> np.ndarray:
    x = _np(x, np.uint16); wr = _np(router_w, np.uint16)
    K, H = x.shape; E = wr.shape[0]
    out = np.empty((K, E), np.float32)
    lib().orc_router(_p(x), _p(wr), K, E, H, _p(out))
    return out


def key(logit: float, bias, e: int, score_fn: int) -> float:
    b = _np(bias, np.float32)
    return lib().orc_key(float(logit), _p(b), int(e), int(score_fn))


def topk(logits, k: int, score_fn: int = SCORE_SOFTMAX, norm_topk: int = 1, bias=None):
    l = _np(logits, np.float32)
    K, E = l.shape
    b = _np(bias, np.float32)
    if score_fn == SCORE_SIGMOID_BIAS and b is None:
        raise ValueError("sigmoid scoring needs a bias vector")
    ids = np.empty((K, k), np.int32)
    w = np.empty((K, k), np.float64)
    lib().orc_topk(_p(l), _p(b), K, E, k, score_fn, norm_topk, _p(ids), _p(w))
    return ids, w


def dedup(ids, n_experts: int):
    flat = _np(ids, np.int32).reshape(-1)
    n = flat.size
    uniq = np.zeros(max(n, 1), np.int32); off = np.zeros(n + 1, np.int32)
    asg = np.zeros(max(n, 1), np.int32); inv = np.zeros(max(n, 1), np.int32)
    U = lib().orc_dedup(_p(flat), n, n_experts, _p(uniq), _p(off), _p(asg), _p(inv))
    return {"n_unique": U, "uniq": uniq[:U].copy(), "off": off[:U + 1].copy(),
            "asg": asg[:n].copy(), "inv": inv[:n].copy()}


def expert_ffn(xrow, gate, up, down, e: int) -> np.ndarray:
    x = _np(xrow, np.uint16).reshape(-1)
    g, u, d = _mat(gate), _mat(up), _mat(down)
    I = g["q"].shape[1]; H = x.size
    out = np.empty(H, np.float64)
    lib().orc_expert_ffn(_p(x), H, I, _p(g["q"]), _p(g["s"]), _p(g["ts"]),
                         _p(u["q"]), _p(u["s"]), _p(u["ts"]),
                         _p(d["q"]), _p(d["s"]), _p(d["ts"]), e, _p(out))
    return out


def moe_layer(w: Dict[str, object], x, top_k: int, score_fn: int = SCORE_SOFTMAX,
              norm_topk: int = 1, routed_scale: float = 1.0, residual=None) -> Dict[str, np.ndarray]:
    """One MoE layer on bf16 rows x [K, H] (int16/uint16 bit patterns).
    Returns logits fp32 [K,E], ids [K,k], w [K,k] (without routed_scale),
    y float64 [K,H], y32 float32 [K,H]."""
    xa = _np(x, np.uint16)
    K, H = xa.shape
    wr = _np(w["router_w"], np.uint16)
    E = wr.shape[0]
    bias = _np(w.get("router_bias"), np.float32)
    if score_fn == SCORE_SIGMOID_BIAS and bias is None:
        raise ValueError("sigmoid scoring needs a bias vector")
    g, u, d = _mat(w["gate"]), _mat(w["up"]), _mat(w["down"])
    I = g["q"].shape[1]
    sg, su, sd = _mat(w.get("sh_gate")), _mat(w.get("sh_up")), _mat(w.get("sh_down"))
    Is = sg["q"].shape[1] if sg is not None else 0
    res = _np(residual, np.uint16)
    logits = np.empty((K, E), np.float32)
    ids = np.empty((K, top_k), np.int32)
    wts = np.empty((K, top_k), np.float64)
    y = np.empty((K, H), np.float64)

    def trip(m):
        return (None, None, None) if m is None else (_p(m["q"]), _p(m["s"]), _p(m["ts"]))

    lib().orc_moe_layer(K, H, E, top_k, I, Is, score_fn, norm_topk, float(routed_scale),
                        _p(xa), _p(wr), _p(bias), *trip(g), *trip(u), *trip(d),
                        *trip(sg), *trip(su), *trip(sd), _p(res),
                        _p(logits), _p(ids), _p(wts), _p(y))
    return {"logits": logits, "ids": ids, "w": wts, "y": y, "y32": y.astype(np.float32)}


def rmsnorm_bf16(y, eps: float = 1e-6, gamma=None) -> np.ndarray:
    """bf16(fp32(gamma * y / sqrt(mean(y^2) + eps))) per row; gamma bf16 [H]
    bit patterns or None (ones)."""
    ya = np.ascontiguousarray(np.asarray(y, np.float64))
    K, H = ya.shape
    g = _np(gamma, np.uint16)
    if g is not None and g.size != H:
        raise ValueError("gamma has %d entries, expected %d" % (g.size, H))
    out = np.empty((K, H), np.uint16)
    lib().orc_rmsnorm_bf16(_p(ya), K, H, float(eps), _p(g), _p(out))
    return out


def bf16_round(y) -> np.ndarray:
    """bf16 bit patterns of y rounded to binary32, then to bf16 (nearest, ties
    to even): the bf16 output y of a layer next to its fp32 result."""
    ya = np.ascontiguousarray(np.asarray(y, np.float64))
    out = np.empty(ya.shape, np.uint16)
    lib().orc_bf16_round(_p(ya), ya.size, _p(out))
    return out


def moe_stack(layers: List[Dict[str, object]], x, top_k: int, eps: float = 1e-6,
              score_fn: int = SCORE_SOFTMAX, norm_topk: int = 1,
              routed_scale: float = 1.0, residual=None) -> List[Dict[str, np.ndarray]]:
    """Free-running stack.  Layer l+1 consumes bf16(RMSNorm(y_l)) scaled by
    layer l's norm weight ('norm_w', bf16 [H]; absent = ones); the stack
    output is the last layer's y before any norm.

    residual None: no residual anywhere.  residual given (bf16 [K, H]): the
    decoder's residual stream of PR #844 section 4 item 4 -- layer 0 adds
    `residual`, layer l >= 1 adds the previous layer's bf16 output
    bf16(y_{l-1}), so the stream carried between layers is each layer's bf16
    output.  Returns one record per layer with its bf16 input under 'x_in'
    and its residual input (or None) under 'res_in'."""
    out = []
    xa = _np(x, np.uint16)
    res = _np(residual, np.uint16)
    for l, w in enumerate(layers):
        rec = moe_layer(w, xa, top_k, score_fn, norm_topk, routed_scale, residual=res)
        rec["x_in"] = xa
        rec["res_in"] = res
        out.append(rec)
        if l + 1 < len(layers):
            xa = rmsnorm_bf16(rec["y"], eps, w.get("norm_w"))
            if res is not None:
                res = bf16_round(rec["y"])
    return out


def dense_mlp(w: Dict[str, object], x, residual=None) -> Dict[str, np.ndarray]:
    """The target's dense first layer (README "Why this challenge exists":
    a SwiGLU MLP of intermediate 8192 in place of the MoE block), bf16
    weights w['gate'], w['up'] [I, H] and w['down'] [H, I]; float64
    y [T, H] = down . (silu(gate . x) * (up . x)) (+ residual)."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    wg, wu, wd = _np(w["gate"], np.uint16), _np(w["up"], np.uint16), _np(w["down"], np.uint16)
    I = wg.shape[0]
    if wg.shape != (I, H) or wu.shape != (I, H) or wd.shape != (H, I):
        raise ValueError("dense MLP weights have shapes %s %s %s for hidden %d" % (wg.shape, wu.shape, wd.shape, H))
    res = _np(residual, np.uint16)
    y = np.empty((T, H), np.float64)
    lib().orc_dense_mlp(_p(xa), T, H, I, _p(wg), _p(wu), _p(wd), _p(res), _p(y))
    return {"y": y, "y32": y.astype(np.float32)}


def dense_moe_stack(dense: Dict[str, object], layers: List[Dict[str, object]], x, top_k: int, eps: float = 1e-6,
                    score_fn: int = SCORE_SOFTMAX, norm_topk: int = 1, routed_scale: float = 1.0,
                    residual=None) -> List[Dict[str, np.ndarray]]:
    """The prefill stack of the target: the dense first layer, then the MoE
    layers, with the same glue between every pair (bf16(RMSNorm(y) * the
    layer's norm weight 'norm_w')) and the same residual stream as
    moe_stack.  Records: the dense layer's first (its 'y', 'y32', 'x_in',
    'res_in'), then one per MoE layer."""
    xa = _np(x, np.uint16)
    res = _np(residual, np.uint16)
    rec = dense_mlp(dense, xa, residual=res)
    rec["x_in"] = xa
    rec["res_in"] = res
    out = [rec]
    if layers:
        x1 = rmsnorm_bf16(rec["y"], eps, dense.get("norm_w"))
        r1 = None if res is None else bf16_round(rec["y"])
        out += moe_stack(layers, x1, top_k, eps, score_fn, norm_topk, routed_scale, residual=r1)
    return out


# ---------------------------------------------------------------------------
# verify-row lm_head and greedy acceptance
# ---------------------------------------------------------------------------


def lm_head(x, w) -> np.ndarray:
    """float64 logits [K, V] = bf16 x [K, H] . bf16 W [V, H]^T."""
    xa = _np(x, np.uint16); wa = _np(w, np.uint16)
    K, H = xa.shape
    V = wa.shape[0]
    if wa.shape[1] != H:
        raise ValueError("W has %d columns, x has %d" % (wa.shape[1], H))
    out = np.empty((K, V), np.float64)
    lib().orc_lm_head(_p(xa), _p(wa), K, V, H, _p(out))
    return out


def greedy_accept(logits, draft, tie_tol: float = 1e-6):
    """Greedy verification of one block (orc_greedy_accept): returns
    {'target': [K], 'accepted': a, 'emitted': [a + 1]}."""
    l = np.ascontiguousarray(np.asarray(logits, np.float64))
    K, V = l.shape
    d = np.ascontiguousarray(np.asarray(draft, np.int32).reshape(-1))
    if d.size != max(K - 1, 0):
        raise ValueError("need K - 1 = %d draft tokens, got %d" % (K - 1, d.size))
    tgt = np.empty(K, np.int32)
    em = np.empty(K, np.int32)
    n = np.zeros(1, np.int32)
    a = lib().orc_greedy_accept(_p(l), K, V, _p(d) if d.size else None, float(tie_tol), _p(tgt), _p(em), _p(n))
    return {"target": tgt, "accepted": int(a), "emitted": em[: int(n[0])].copy()}


def lm_head_bytes(vocab: int, hidden: int, K: int) -> int:
    """Algorithmic HBM bytes of one verify step's lm_head: the bf16 matrix
    once, the K bf16 rows in."""
    return vocab * hidden * 2 + K * hidden * 2


# ---------------------------------------------------------------------------
# byte accounting
# ---------------------------------------------------------------------------


def nvfp4_matrix_bytes(rows: int, cols: int, tensor_scale: bool = True) -> int:
    """Codes (half a byte per weight) + one E4M3 scale per 16 weights (+ one
    fp32 tensor scale)."""
    return rows * cols // 2 + rows * cols // 16 + (4 if tensor_scale else 0)


def expert_bytes(hidden: int, inter: int) -> int:
    return 2 * nvfp4_matrix_bytes(inter, hidden) + nvfp4_matrix_bytes(hidden, inter)


def layer_step_bytes(hidden: int, n_experts: int, inter: int, shared_inter: int,
                     n_unique: int, K: int, with_router: bool = True) -> int:
    """Algorithmic HBM bytes of one verify step through one layer: router
    (bf16), each unique routed expert once, the shared expert, x in and y out
    (bf16)."""
    b = n_unique * expert_bytes(hidden, inter)
    if shared_inter:
        b += expert_bytes(hidden, shared_inter)
    if with_router:
        b += 2 * n_experts * hidden
    return b + 2 * 2 * K * hidden
