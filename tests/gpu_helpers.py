"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI
with debug outputs, and compare against the oracle.

Comparison rules (written out here and in the tests):
  * logits: |gpu - oracle| <= 1e-5 * max|oracle|;
  * selection: ids bit-exact on every row whose oracle keys have no
    near-tie (adjacent gap among the first k+1 sorted keys below twice the
    logit tolerance); near-tie rows only need a valid selection and are left
    out of the output comparison;
  * dedup lists: bit-exact against the oracle's dedup of the oracle's ids;
  * weights: |dw| <= 1e-6 |w| + 2 * (logit tolerance) * w;
  * output: max|y32 - y_oracle| <= 2e-3 * max|y_oracle| over the compared
    rows; y (bf16) is the round-to-nearest-even of y32.
  * stacked layers, every layer at the same 2e-3 bar: the oracle runs its
    own chain, and where the GPU's bf16 input of a layer differs from the
    oracle's, the GPU's value must be the bf16 rounding of a value within
    the error bound of the oracle's own unrounded value (the previous
    layer's measured output deviation carried through the normalisation,
    plus fp32 rounding): another correct result of the definition.  The
    oracle chain adopts such a rounding and evaluates the layer on it;
    nothing else from the GPU enters the oracle.  Separately, the GPU's
    input of layer l+1 must be the RMSNorm of its own y32 of layer l within
    fp32 rounding (the glue, counted re-roundings per row bounded).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from speculative_block_verify_amd import api
from tests import refdecode as ref

Y_TOL = 2e-3
LOGIT_RTOL = 1e-5
# fp32 error of the normalisation (sum of squares over <= 2048 terms in a
# tree, sqrt, divide, two products), in units of 2^-24 of the value; generous
GLUE_ULPS32 = 16.0


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
        "status": torch.full((1,), -1, dtype=torch.int32, device=dev),
    }
    y = torch.empty(K, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, H, dtype=torch.float32, device=dev)
    if ws is None:
        ws = api.alloc_workspace(cfg, dev)
    fn = api.moe_verify_layer_grouped if grouped else api.moe_verify_layer
    fn(cfg, api.make_weights(wd), x, y, ws, y32=y32, residual=residual, debug=api.make_debug(**dbg_t))
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in dbg_t.items()}
    assert np.all(out["status"] == 0), "an in-kernel hand-off wait gave up"
    out["y"] = y.cpu().numpy().view(np.uint16)
    out["y32_out"] = y32.cpu().numpy()
    out["ids"] = out["ids"].reshape(K, k)
    out["w"] = out["w"].reshape(K, k)
    return out


def run_stack_debug(cfg, layers_dev, x, n_layers, residual=None):
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
        "status": torch.full((L,), -1, dtype=torch.int32, device=dev),
    }
    if residual is not None:
        dbg_t["res_in"] = torch.empty(L, K, H, dtype=torch.int16, device=dev)
    y = torch.empty(K, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, H, dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(cfg, dev)
    api.moe_verify_stack(cfg, [api.make_weights(w, cfg) for w in layers_dev], x, y, ws, y32=y32,
                         debug=api.make_debug(**dbg_t), residual=residual)
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in dbg_t.items()}
    assert np.all(out["status"] == 0), "an in-kernel hand-off wait gave up: %s" % out["status"]
    out["y"] = y.cpu().numpy().view(np.uint16)
    out["y32_out"] = y32.cpu().numpy()
    return out


def run_prefill_debug(cfg, dense_dev, layers_dev, x, residual=None):
    """moe_prefill_stack with per-MoE-layer debug arrays and the dense
    layer's fp32 output; returns numpy arrays (rows as given)."""
    T, H = x.shape
    E, k, L = cfg.n_experts, cfg.top_k, len(layers_dev)
    dev = x.device
    n = T * k
    dbg_t = {
        "logits": torch.empty(L, T, E, dtype=torch.float32, device=dev),
        "ids": torch.empty(L, n, dtype=torch.int32, device=dev),
        "w": torch.empty(L, n, dtype=torch.float32, device=dev),
        "n_unique": torch.empty(L, dtype=torch.int32, device=dev),
        "uniq": torch.empty(L, n, dtype=torch.int32, device=dev),
        "off": torch.empty(L, n + 1, dtype=torch.int32, device=dev),
        "asg": torch.empty(L, n, dtype=torch.int32, device=dev),
        "inv": torch.empty(L, n, dtype=torch.int32, device=dev),
        "x_in": torch.empty(L, T, H, dtype=torch.int16, device=dev),
        "y32": torch.empty(L, T, H, dtype=torch.float32, device=dev),
        "status": torch.full((L,), -1, dtype=torch.int32, device=dev),
    }
    if residual is not None:
        dbg_t["res_in"] = torch.empty(L, T, H, dtype=torch.int16, device=dev)
    y = torch.empty(T, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(T, H, dtype=torch.float32, device=dev)
    yd = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    I = dense_dev["gate"].shape[0]
    ws = torch.empty(api.moe_prefill_workspace_bytes(cfg, I), dtype=torch.uint8, device=dev)
    api.moe_prefill_stack(cfg, dense_dev, [api.make_weights(w, cfg) for w in layers_dev], x, y, ws, y32=y32,
                          dense_y32=yd, residual=residual, debug=api.make_debug(**dbg_t))
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in dbg_t.items()}
    assert np.all(out["status"] == 0), "an in-kernel hand-off wait gave up: %s" % out["status"]
    out["y"] = y.cpu().numpy().view(np.uint16)
    out["y32_out"] = y32.cpu().numpy()
    out["dense_y32"] = yd.cpu().numpy()
    return out


def oracle_dense_rows(w, x, residual=None, threads: int = 16) -> np.ndarray:
    """orc.dense_mlp over the rows of x in chunks on parallel host threads
    (each row's output depends on that row alone); float64 y."""
    from concurrent.futures import ThreadPoolExecutor
    wh = {kk: (None if v is None else np.ascontiguousarray(v.cpu().numpy() if hasattr(v, "cpu") else v))
          for kk, v in w.items()}
    xa = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x)).view(np.uint16)
    ra = None if residual is None else np.ascontiguousarray(
        np.asarray(residual.cpu() if hasattr(residual, "cpu") else residual)).view(np.uint16)
    T = xa.shape[0]
    bounds = np.linspace(0, T, min(threads, T) + 1).astype(int)
    parts = [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    with ThreadPoolExecutor(len(parts)) as ex:
        ys = list(ex.map(lambda ab: orc.dense_mlp(wh, np.ascontiguousarray(xa[ab[0]:ab[1]]),
                                                  residual=None if ra is None else
                                                  np.ascontiguousarray(ra[ab[0]:ab[1]]))["y"], parts))
    return np.concatenate(ys)


def oracle_layer_rows(w, x, k: int, score_fn: int = 0, rs: float = 1.0, residual=None, threads: int = 16):
    """orc.moe_layer over the rows of x in chunks on parallel host threads
    (the layer is defined row by row: each row's routing and FFN depend on
    that row alone, so the chunks' results are the layer's rows; the C
    oracle runs with the interpreter lock released)."""
    from concurrent.futures import ThreadPoolExecutor
    xa = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x)).view(np.uint16)
    ra = None if residual is None else np.ascontiguousarray(
        np.asarray(residual.cpu() if hasattr(residual, "cpu") else residual)).view(np.uint16)
    T = xa.shape[0]
    orc.moe_layer(w, xa[:1], k, score_fn, 1, rs, residual=None if ra is None else ra[:1])  # tables built once
    bounds = np.linspace(0, T, min(threads, T) + 1).astype(int)
    parts = [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    with ThreadPoolExecutor(len(parts)) as ex:
        recs = list(ex.map(lambda ab: orc.moe_layer(w, np.ascontiguousarray(xa[ab[0]:ab[1]]), k, score_fn, 1, rs,
                                                    residual=None if ra is None else
                                                    np.ascontiguousarray(ra[ab[0]:ab[1]])), parts))
    return {kk: np.concatenate([r[kk] for r in recs]) for kk in ("logits", "ids", "w", "y", "y32")}


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
                  label="", rows=None):
    """Assert the rules above; return a small report dict.  rows (bool mask)
    restricts the comparison to some rows (the dedup lists, which mix all
    rows, are then not compared)."""
    if rows is not None and not np.all(rows):
        sel = np.nonzero(rows)[0]
        gpu = {kk: gpu[kk][sel] for kk in ("logits", "ids", "w", "y32")}
        orec = {kk: orec[kk][sel] for kk in ("logits", "ids", "w", "y")}
        rep = compare_layer(gpu, orec, k, n_experts, score_fn, bias, label, None)
        rep["partial_rows"] = True
        return rep
    K = orec["logits"].shape[0]
    ol = orec["logits"].astype(np.float64)
    gl = gpu["logits"].astype(np.float64)
    tol = np.full(K, LOGIT_RTOL * np.abs(ol).max())
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
    errs = np.abs(gpu["y32"].astype(np.float64) - yo)
    roww = errs.max(axis=1)
    bad = ok & (roww > Y_TOL * scale)
    assert not bad.any(), "%s y32 max err %s > %s" % (label, roww[bad], Y_TOL * scale)
    err = errs[ok]
    maxerr = float(err.max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(err) / max(np.linalg.norm(yo[ok]), 1e-30)) if err.size else 0.0
    return {"max_abs_over_max_ref": maxerr / scale, "rel_l2": rel_l2, "near_ties": int(tie.sum()),
            "tie_rows": tie}


# ---------------------------------------------------------------------------
# bf16 roundings
# ---------------------------------------------------------------------------


def _rounding_interval(bits: np.ndarray):
    """The interval of reals that round (to nearest) to each bf16 value:
    halfway to its neighbours on either side."""
    b = bits.astype(np.int64)
    sign = (b & 0x8000) != 0
    mag = b & 0x7FFF
    val = lambda m: ref.bf16_to_f64(m.astype(np.uint16))  # noqa: E731
    m0 = val(mag)
    below = np.where(mag > 0, val(np.maximum(mag - 1, 0)), -val(np.ones_like(mag)))
    above = val(np.minimum(mag + 1, 0x7F7F))
    lo_m, hi_m = 0.5 * (below + m0), 0.5 * (m0 + above)
    lo = np.where(sign, -hi_m, lo_m)
    hi = np.where(sign, -lo_m, hi_m)
    return lo, hi


def admissible_flips(ref_bits: np.ndarray, pre: np.ndarray, got_bits: np.ndarray, delta: np.ndarray, label: str):
    """Check that got_bits equals ref_bits (the round-to-nearest-even of the
    unrounded values `pre`) except where got_bits is the rounding of some
    value within `delta` of `pre` (the arithmetic's error bound for that
    element).  Returns the mask of elements that differ."""
    diff = got_bits != ref_bits
    if not diff.any():
        return diff
    p = pre[diff]
    d = delta[diff]
    lo, hi = _rounding_interval(got_bits[diff])
    okf = (p + d >= lo) & (p - d <= hi)
    if not okf.all():
        i = np.nonzero(~okf)[0][0]
        r = ref.bf16_to_f64(ref_bits[diff])
        g = ref.bf16_to_f64(got_bits[diff])
        raise AssertionError("%s: bf16 input differs beyond an admissible rounding: unrounded %r (error bound "
                             "%.3g), oracle %r, gpu %r (%d of %d differing elements inadmissible)" % (
                                 label, p[i], d[i], r[i], g[i], int((~okf).sum()), int(diff.sum())))
    return diff


def rmsnorm_pre(y: np.ndarray, eps: float, gamma) -> np.ndarray:
    """Unrounded RMSNorm (times gamma) of each row of y, in float64: the
    definition the glue computes (property checks and rounding distances)."""
    y = np.asarray(y, np.float64)
    inv = 1.0 / np.sqrt((y * y).mean(axis=1, keepdims=True) + eps)
    v = y * inv
    if gamma is not None:
        v = v * ref.bf16_to_f64(np.asarray(gamma).view(np.uint16))[None, :]
    return v


def check_glue(x_next_gpu: np.ndarray, y32_gpu: np.ndarray, eps: float, gamma, label: str, max_flips_per_row=16):
    """Property of the stack glue on the GPU's own values: its input of layer
    l+1 is bf16(gamma * RMSNorm(its y32 of layer l)), up to bf16 roundings of
    values within fp32 rounding distance of a midpoint (counted, bounded)."""
    v = rmsnorm_pre(y32_gpu, eps, gamma)
    want = ref.f32_to_bf16_bits(v.astype(np.float32))
    delta = GLUE_ULPS32 * 2.0 ** -24 * np.abs(v) + 1e-45
    flips = admissible_flips(want, v, x_next_gpu.view(np.uint16), delta, label + " glue")
    per_row = flips.sum(axis=1)
    assert per_row.max() <= max_flips_per_row, "%s glue: %s rounding flips per row" % (label, per_row)
    return int(flips.sum())


def compare_stack(gpu, layers_host, x0: np.ndarray, k: int, n_experts: int, eps: float = 1e-6,
                  score_fn: int = 0, rs: float = 1.0, label="", residual=None, max_flip_frac=0.02, pre=None):
    """Every layer of a stack against the oracle at the 2e-3 bar (rules
    above).  A row leaves the comparison only after a layer where it
    selected other experts at a certified near-tie of the oracle's keys.
    residual: the stack's initial residual (bf16 bits) or None.
    pre: a layer ahead of the MoE layers (the dense first layer of the
    prefill stack), as {'y_oracle': its oracle output on x0, 'y32_gpu': the
    GPU's, 'norm_w': its norm weight or None}; the first MoE layer's input
    and residual are then checked like any later layer's, and x0 is the
    pre-layer's input."""
    layers_host = list(layers_host)
    K, H = x0.shape
    alive = np.ones(K, bool)
    xo = np.ascontiguousarray(x0).view(np.uint16)
    ro = None if residual is None else np.ascontiguousarray(residual).view(np.uint16)
    reps = []
    prev = None
    if pre is not None:
        prev = (pre["y_oracle"], {"norm_w": pre["norm_w"]})
        xo = orc.rmsnorm_bf16(pre["y_oracle"], eps, pre["norm_w"])
        if ro is not None:
            ro = orc.bf16_round(pre["y_oracle"])
    for l, w in enumerate(layers_host):
        g = {kk: gpu[kk][l] for kk in ("logits", "ids", "w", "n_unique", "uniq", "off", "asg", "inv",
                                       "x_in", "y32")}
        g["ids"] = g["ids"].reshape(K, k)
        g["w"] = g["w"].reshape(K, k)
        g["n_unique"] = np.array([g["n_unique"]])
        xg = g["x_in"].view(np.uint16)
        flips_x = flips_r = 0
        glue_flips = 0
        if prev is not None:
            yo_prev, wprev = prev
            y32g_prev = gpu["y32"][l - 1] if l > 0 else pre["y32_gpu"]
            gam = wprev.get("norm_w")
            gam = None if gam is None else np.asarray(gam).view(np.uint16)
            # the glue on the GPU's own values (every row)
            glue_flips = check_glue(xg, y32g_prev, eps, gam, "%s layer %d" % (label, l))
            # the oracle chain: its own unrounded input and the admissible distance
            v = rmsnorm_pre(yo_prev, eps, gam)
            inv_o = 1.0 / np.sqrt((yo_prev ** 2).mean(axis=1, keepdims=True) + eps)
            y64g = y32g_prev.astype(np.float64)
            inv_g = 1.0 / np.sqrt((y64g ** 2).mean(axis=1, keepdims=True) + eps)
            gabs = 1.0 if gam is None else np.abs(ref.bf16_to_f64(gam))[None, :]
            delta = 1.01 * (np.abs(y64g - yo_prev) * inv_o * gabs + np.abs(v) * np.abs(inv_g / inv_o - 1.0)
                            + GLUE_ULPS32 * 2.0 ** -24 * np.abs(v)) + 1e-45
            rows = np.nonzero(alive)[0]
            fx = admissible_flips(xo[rows], v[rows], xg[rows], delta[rows], "%s layer %d input" % (label, l))
            flips_x = int(fx.sum())
            assert fx.sum(axis=1).max() <= max_flip_frac * H, "%s layer %d: %s input flips" % (label, l, fx.sum(1))
            xo = xo.copy()
            xo[rows] = np.where(fx, xg[rows], xo[rows])
            if ro is not None:
                rg = gpu["res_in"][l].view(np.uint16)
                # the residual stream is bf16 of the previous output: exact on the GPU's own values
                np.testing.assert_array_equal(rg, ref.f32_to_bf16_bits(y32g_prev), err_msg="%s layer %d residual"
                                              % (label, l))
                pre = yo_prev.astype(np.float32).astype(np.float64)
                dr = 1.01 * (np.abs(y64g - yo_prev) + 2.0 ** -24 * np.abs(yo_prev)) + 1e-45
                fr = admissible_flips(ro[rows], pre[rows], rg[rows], dr[rows], "%s layer %d residual" % (label, l))
                flips_r = int(fr.sum())
                ro = ro.copy()
                ro[rows] = np.where(fr, rg[rows], ro[rows])
        if ro is not None and l == 0 and pre is None:
            np.testing.assert_array_equal(gpu["res_in"][0].view(np.uint16), ro, err_msg=label + " layer 0 residual")
        # the GPU consumed exactly the oracle chain's input on every compared row
        np.testing.assert_array_equal(xg[alive], xo[alive], err_msg="%s layer %d input" % (label, l))
        orec = orc.moe_layer(w, xo, k, score_fn, 1, rs, residual=ro)
        rep = compare_layer(g, orec, k, n_experts, score_fn, w.get("router_bias"), "%s layer %d" % (label, l), alive)
        rep.update({"input_flips": flips_x, "residual_flips": flips_r, "glue_flips": glue_flips,
                    "rows": int(alive.sum())})
        reps.append(rep)
        # rows that took another (valid) selection at a certified near-tie leave
        diverged = np.any(g["ids"] != orec["ids"], axis=1)
        assert not np.any(diverged & alive & ~_tie_rows_full(rep, alive)), label + " divergence outside a near-tie"
        alive &= ~diverged
        if not alive.any():
            break
        prev = (orec["y"], w)
        xo = orc.rmsnorm_bf16(orec["y"], eps, w.get("norm_w"))
        if ro is not None:
            ro = orc.bf16_round(orec["y"])
    return reps, alive


def _tie_rows_full(rep, alive):
    """The near-tie mask of a (possibly row-restricted) report, over all rows."""
    t = np.zeros(alive.shape, bool)
    t[np.nonzero(alive)[0]] = rep["tie_rows"]
    return t
