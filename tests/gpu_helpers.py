"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI
with debug outputs, and compare against the oracle.

Comparison rules (written out here and in the tests):
  * logits: |gpu - oracle| <= 1e-5 * max|oracle| + (bound from any bf16
    differences of the layer input, for chained layers);
  * selection: ids bit-exact on every row whose oracle keys have no
    near-tie (adjacent gap among the first k+1 sorted keys below twice the
    logit tolerance); near-tie rows only need a valid selection and are left
    out of the output comparison;
  * dedup lists: bit-exact against the oracle's dedup of the oracle's ids;
  * weights: |dw| <= 1e-6 |w| + 2 * (logit tolerance) * w;
  * output: max|y32 - y_oracle| <= 2e-3 * max|y_oracle| over the compared
    rows; y (bf16) is the round-to-nearest-even of y32.
  * chained layers: a row whose bf16 input already differs from the
    oracle's (a rounding-boundary flip of an earlier layer's output) is held
    to 1e-2 * max|y_oracle| instead, since the two sides no longer evaluate
    the same input.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from speculative_block_verify_amd import api
from tests import refdecode as ref

Y_TOL = 2e-3
CHAIN_Y_TOL = 1e-2
LOGIT_RTOL = 1e-5


def run_layer(cfg, wd, x, residual=None, ws=None, grouped=False):
    """moe_verify_layer (or moe_verify_layer_grouped) with every debug array;
    returns numpy arrays."""
    K, H = x.shape
    E, k = cfg.n_experts, cfg.top_k
    dev = x.device
    n = K * k
    dbg_t = {
        "logits": torch.empty(K, E, dtype=torch.float32, device=dev),
        "ids": torch.empty(n, dtype=torch.int32, device=dev),
        "w": torch.empty(n, dtype=torch.float32, device=dev),
        "n_unique": torch.empty(1, dtype=torch.int32, device=dev),
        "uniq": torch.empty(n, dtype=torch.int32, device=dev),
        "off": torch.empty(n + 1, dtype=torch.int32, device=dev),
        "asg": torch.empty(n, dtype=torch.int32, device=dev),
        "inv": torch.empty(n, dtype=torch.int32, device=dev),
        "x_in": torch.empty(K, H, dtype=torch.int16, device=dev),
        "y32": torch.empty(K, H, dtype=torch.float32, device=dev),
    }
    y = torch.empty(K, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, H, dtype=torch.float32, device=dev)
    if ws is None:
        ws = api.alloc_workspace(cfg, dev)
    fn = api.moe_verify_layer_grouped if grouped else api.moe_verify_layer
    fn(cfg, api.make_weights(wd), x, y, ws, y32=y32, residual=residual, debug=api.make_debug(**dbg_t))
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in dbg_t.items()}
    out["y"] = y.cpu().numpy().view(np.uint16)
    out["y32_out"] = y32.cpu().numpy()
    out["ids"] = out["ids"].reshape(K, k)
    out["w"] = out["w"].reshape(K, k)
    return out


def run_stack_debug(cfg, layers_dev, x, n_layers):
    K, H = x.shape
    E, k = cfg.n_experts, cfg.top_k
    dev = x.device
    n = K * k
    L = n_layers
    dbg_t = {
        "logits": torch.empty(L, K, E, dtype=torch.float32, device=dev),
        "ids": torch.empty(L, n, dtype=torch.int32, device=dev),
        "w": torch.empty(L, n, dtype=torch.float32, device=dev),
        "n_unique": torch.empty(L, dtype=torch.int32, device=dev),
        "uniq": torch.empty(L, n, dtype=torch.int32, device=dev),
        "off": torch.empty(L, n + 1, dtype=torch.int32, device=dev),
        "asg": torch.empty(L, n, dtype=torch.int32, device=dev),
        "inv": torch.empty(L, n, dtype=torch.int32, device=dev),
        "x_in": torch.empty(L, K, H, dtype=torch.int16, device=dev),
        "y32": torch.empty(L, K, H, dtype=torch.float32, device=dev),
    }
    y = torch.empty(K, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, H, dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(cfg, dev)
    api.moe_verify_stack(cfg, [api.make_weights(w) for w in layers_dev], x, y, ws, y32=y32,
                         debug=api.make_debug(**dbg_t))
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in dbg_t.items()}
    out["y"] = y.cpu().numpy().view(np.uint16)
    out["y32_out"] = y32.cpu().numpy()
    return out


def oracle_keys(logits: np.ndarray, bias, score_fn: int) -> np.ndarray:
    K, E = logits.shape
    if score_fn == orc.SCORE_SOFTMAX:
        return logits.astype(np.float64)
    return np.array([[orc.key(logits[r, e], bias, e, score_fn) for e in range(E)] for r in range(K)])


def near_tie_rows(keys: np.ndarray, k: int, tol: np.ndarray) -> np.ndarray:
    """Rows whose first k+1 sorted keys have an adjacent gap below 2*tol."""
    out = np.zeros(keys.shape[0], bool)
    for r in range(keys.shape[0]):
        s = np.sort(keys[r])[::-1][: min(k + 1, keys.shape[1])]
        out[r] = bool(np.any(np.diff(s) > -2 * tol[r])) if s.size > 1 else False
    return out


def bf16_of(y32: np.ndarray) -> np.ndarray:
    return ref.f32_to_bf16_bits(y32)


def compare_layer(gpu, orec, k: int, n_experts: int, score_fn: int = 0, bias=None,
                  logit_tol=None, label="", rows=None, y_tol=None):
    """Assert the rules above; return a small report dict.  rows (bool mask)
    restricts the comparison to some rows (the dedup lists, which mix all
    rows, are then not compared)."""
    if rows is not None and not np.all(rows):
        sel = np.nonzero(rows)[0]
        gpu = {kk: gpu[kk][sel] for kk in ("logits", "ids", "w", "y32")}
        orec = {kk: orec[kk][sel] for kk in ("logits", "ids", "w", "y")}
        if logit_tol is not None:
            logit_tol = np.asarray(logit_tol)[sel]
        if y_tol is not None:
            y_tol = np.asarray(y_tol)[sel]
        rep = compare_layer(gpu, orec, k, n_experts, score_fn, bias, logit_tol, label, None, y_tol)
        rep["partial_rows"] = True
        return rep
    K = orec["logits"].shape[0]
    ol = orec["logits"].astype(np.float64)
    gl = gpu["logits"].astype(np.float64)
    base_tol = LOGIT_RTOL * np.abs(ol).max()
    tol = np.full(K, base_tol) if logit_tol is None else base_tol + np.asarray(logit_tol)
    dl = np.abs(gl - ol).max(axis=1)
    assert np.all(dl <= tol), "%s logits off: %s > %s" % (label, dl, tol)
    if score_fn == orc.SCORE_SIGMOID_BIAS:
        tol = tol * 0.25 + 1e-7  # sigmoid' <= 1/4
    keys = oracle_keys(orec["logits"], bias, score_fn)
    tie = near_tie_rows(keys, k, tol)
    ok = ~tie
    np.testing.assert_array_equal(gpu["ids"][ok], orec["ids"][ok], err_msg=label + " ids")
    # a near-tie row must still pick experts whose oracle keys are within tol of the k-th
    for r in np.nonzero(tie)[0]:
        kth = np.sort(keys[r])[::-1][k - 1]
        assert np.all(keys[r][gpu["ids"][r]] >= kth - 2 * tol[r]), label + " invalid near-tie selection"
    if not tie.any() and "asg" in gpu:
        d = orc.dedup(orec["ids"], n_experts)
        U = d["n_unique"]
        assert int(gpu["n_unique"].reshape(-1)[0]) == U, label + " n_unique"
        np.testing.assert_array_equal(gpu["uniq"][:U], d["uniq"], err_msg=label + " uniq")
        np.testing.assert_array_equal(gpu["off"][:U + 1], d["off"], err_msg=label + " off")
        np.testing.assert_array_equal(gpu["asg"], d["asg"], err_msg=label + " asg")
        np.testing.assert_array_equal(gpu["inv"], d["inv"], err_msg=label + " inv")
    wt = 1e-6 * np.abs(orec["w"][ok]) + 2 * tol[ok, None] * np.abs(orec["w"][ok]) + 1e-12
    assert np.all(np.abs(gpu["w"][ok] - orec["w"][ok]) <= wt), label + " weights"
    yo = orec["y"]
    scale = np.abs(yo).max()
    rowtol = np.full(K, Y_TOL) if y_tol is None else np.asarray(y_tol, np.float64)
    errs = np.abs(gpu["y32"].astype(np.float64) - yo)
    roww = errs.max(axis=1)
    bad = ok & (roww > rowtol * scale)
    assert not bad.any(), "%s y32 max err %s > %s" % (label, roww[bad], rowtol[bad] * scale)
    err = errs[ok]
    maxerr = float(err.max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(err) / max(np.linalg.norm(yo[ok]), 1e-30)) if err.size else 0.0
    return {"max_abs_over_max_ref": maxerr / scale, "rel_l2": rel_l2, "near_ties": int(tie.sum())}


def compare_stack(gpu, layers_host, x0: np.ndarray, k: int, n_experts: int, eps: float = 1e-6,
                  score_fn: int = 0, rs: float = 1.0, label=""):
    """Free-running comparison of a stack: the oracle chains its own layers.
    A row leaves the comparison after a layer where it legitimately selected
    other experts (a near-tie in the oracle's keys); other rows continue."""
    K = x0.shape[0]
    alive = np.ones(K, bool)
    xo = np.ascontiguousarray(x0).view(np.uint16)
    reps = []
    for l, w in enumerate(layers_host):
        orec = orc.moe_layer(w, xo, k, score_fn, 1, rs)
        g = {kk: gpu[kk][l] for kk in ("logits", "ids", "w", "n_unique", "uniq", "off", "asg", "inv",
                                       "x_in", "y32")}
        g["ids"] = g["ids"].reshape(K, k)
        g["w"] = g["w"].reshape(K, k)
        g["n_unique"] = np.array([g["n_unique"]])
        xg = ref.bf16_to_f64(g["x_in"].view(np.uint16))
        xr = ref.bf16_to_f64(xo)
        wr_max = np.abs(ref.bf16_to_f64(np.asarray(w["router_w"]).view(np.uint16))).max(axis=0)
        ltol = (np.abs(xg - xr) * wr_max[None, :]).sum(axis=1) * 1.01
        ytol = np.where((g["x_in"].view(np.uint16) != xo).any(axis=1), CHAIN_Y_TOL, Y_TOL)
        rep = compare_layer(g, orec, k, n_experts, score_fn, None, ltol, "%s layer %d" % (label, l), alive, ytol)
        rep["x_in_bf16_diffs"] = int((g["x_in"].view(np.uint16) != xo).sum())
        reps.append(rep)
        diverged = np.any(g["ids"] != orec["ids"], axis=1)
        alive &= ~diverged
        if not alive.any():
            break
        xo = orc.rmsnorm_bf16(orec["y"], eps)
    return reps, alive
