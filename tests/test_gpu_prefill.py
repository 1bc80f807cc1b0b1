"""GPU parity of the prefill stack: the target's dense first layer
(moe_dense_mlp) and the dense layer followed by MoE layers
(moe_prefill_stack) against the oracle.

Rules (written out here and in tests/gpu_helpers.py): the dense layer's y32
within 2e-3 of max|y| of the fp64 oracle on the same bf16 input (h reaches
the down GEMM as a bf16 hi + lo pair, so the error is that of fp32 sums),
y = RNE(y32), and the next input x_next = bf16(gamma * RMSNorm(y32)) within
fp32 rounding; every MoE layer after it is held to the stack rules of
compare_stack, with the dense layer as its pre-layer.  Rows are
independent, so the full-size stacks compare sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from speculative_block_verify_amd import api, inputs
from tests import gpu_helpers as gh
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
TINY_SH = inputs.MoEShape(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128)


def say(*a):
    print(*a, flush=True)


def _gamma(H, seed):
    g = torch.Generator().manual_seed(seed)
    return inputs.bf16_bits(0.5 + 1.5 * torch.rand(H, generator=g)).to(DEV)


def _dense_case(T, H, I, seed, residual, gamma):
    say("case: dense T=%d H=%d I=%d residual=%d gamma=%d" % (T, H, I, residual, gamma))
    w = inputs.gen_dense(H, I, seed, device=DEV)
    if gamma:
        w["norm_w"] = _gamma(H, seed)
    x = inputs.gen_x(T, H, seed, device=DEV)
    res = inputs.gen_x(T, H, seed, device=DEV, tag="res") if residual else None
    y = torch.empty(T, H, dtype=torch.int16, device=DEV)
    y32 = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    xn = torch.empty(T, H, dtype=torch.int16, device=DEV)
    ws = torch.empty(api.moe_dense_workspace_bytes(H, I, T), dtype=torch.uint8, device=DEV)
    api.moe_dense_mlp(x, w, y, y32, ws, residual=res, eps=1e-6, x_next=xn)
    torch.cuda.synchronize()
    g32 = y32.cpu().numpy()
    yo = gh.oracle_dense_rows(w, x, residual=res)
    err = np.abs(g32.astype(np.float64) - yo).max() / np.abs(yo).max()
    assert err <= gh.Y_TOL, "dense T=%d: %.3g of max|y|" % (T, err)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16), gh.bf16_of(g32))
    flips = gh.check_glue(xn.cpu().numpy(), g32, 1e-6, None if w["norm_w"] is None else w["norm_w"].cpu().numpy(),
                          "dense T=%d" % T)
    say("  max err / max|y| %.3g, glue re-roundings %d" % (err, flips))
    return err


@pytest.mark.parametrize("T,H,I", [(1, 256, 512), (5, 256, 512), (64, 512, 1024), (130, 256, 768),
                                   (17, 2048, 256), (300, 256, 512), (257, 512, 1024)])
def test_dense_layer_shapes(T, H, I):
    # one row, a ragged token tile, several tiles, several column tiles; from
    # 256 rows the 128 x 128 LDS-ring kernels, with a ragged last tile
    _dense_case(T, H, I, 10 + T, residual=(T % 2 == 1), gamma=(T > 5))


def test_dense_layer_full_size_512_rows():
    """The target's dense layer (hidden 2048, intermediate 8192) on the
    512-row seed prefill: every row against the oracle."""
    err = _dense_case(512, 2048, inputs.DENSE_INTER, 5, residual=True, gamma=True)
    assert err < 1e-4  # fp32 sums of exact products: far inside the bar


def test_dense_layer_is_deterministic():
    T, H, I = 70, 512, 1024
    w = inputs.gen_dense(H, I, 3, device=DEV)
    x = inputs.gen_x(T, H, 3, device=DEV)
    ws = torch.empty(api.moe_dense_workspace_bytes(H, I, T), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(2):
        y = torch.empty(T, H, dtype=torch.int16, device=DEV)
        y32 = torch.empty(T, H, dtype=torch.float32, device=DEV)
        api.moe_dense_mlp(x, w, y, y32, ws)
        torch.cuda.synchronize()
        outs.append(y32.cpu().numpy())
    np.testing.assert_array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def _prefill_case(shape, dense_inter, T, n_moe, seed, residual, gamma, rows=None, label=""):
    say("case: prefill %s T=%d dense_inter=%d moe_layers=%d residual=%d gamma=%d" % (
        label, T, dense_inter, n_moe, residual, gamma))
    dense = inputs.gen_dense(shape.hidden, dense_inter, seed, device=DEV)
    layers = inputs.gen_stack(shape, n_moe, seed + 1, device=DEV)
    if gamma:
        dense["norm_w"] = _gamma(shape.hidden, seed)
        for l, w in enumerate(layers):
            w["norm_w"] = _gamma(shape.hidden, seed + 100 + l)
    x = inputs.gen_x(T, shape.hidden, seed, device=DEV)
    res = inputs.gen_x(T, shape.hidden, seed, device=DEV, tag="res") if residual else None
    cfg = api.make_cfg(shape, T)
    gpu = gh.run_prefill_debug(cfg, dense, layers, x, residual=res)
    np.testing.assert_array_equal(gpu["y32_out"], gpu["y32"][-1])
    np.testing.assert_array_equal(gpu["y"], gh.bf16_of(gpu["y32_out"]))
    sel = np.arange(T) if rows is None else np.asarray(rows)
    xs = x.cpu().numpy()[sel]
    rs = None if res is None else res.cpu().numpy()[sel]
    # the dense layer on its exact input
    yo = gh.oracle_dense_rows(dense, xs, residual=rs)
    err = np.abs(gpu["dense_y32"][sel].astype(np.float64) - yo).max() / np.abs(yo).max()
    assert err <= gh.Y_TOL, "%s dense layer: %.3g" % (label, err)
    # the MoE layers, the dense layer as their pre-layer, on the sampled rows
    sub = {kk: (v[:, sel] if kk in ("logits", "x_in", "y32", "res_in") else v) for kk, v in gpu.items()
           if kk in ("logits", "x_in", "y32", "res_in", "n_unique")}
    k = shape.top_k
    for kk in ("ids", "w"):
        sub[kk] = gpu[kk].reshape(n_moe, T, k)[:, sel].reshape(n_moe, -1)
    # the dedup lists mix rows: recompute them from the sampled rows' ids
    # (compare_stack checks them against the oracle's dedup of its ids)
    sub["uniq"], sub["off"], sub["asg"], sub["inv"], sub["n_unique"] = [], [], [], [], []
    for l in range(n_moe):
        d = orc.dedup(sub["ids"][l].reshape(-1, k), shape.n_experts)
        n = len(sel) * k
        sub["n_unique"].append(d["n_unique"])
        sub["uniq"].append(np.pad(d["uniq"], (0, n - len(d["uniq"]))))
        sub["off"].append(np.pad(d["off"], (0, n + 1 - len(d["off"]))))
        sub["asg"].append(d["asg"])
        sub["inv"].append(d["inv"])
    for kk in ("n_unique", "uniq", "off", "asg", "inv"):
        sub[kk] = np.asarray(sub[kk])
    layers_host = [{kk: (None if v is None else ({q: t.cpu() for q, t in v.items()} if isinstance(v, dict)
                                                  else v.cpu())) for kk, v in w.items()} for w in layers]
    pre = {"y_oracle": yo, "y32_gpu": gpu["dense_y32"][sel],
           "norm_w": None if dense["norm_w"] is None else dense["norm_w"].cpu().numpy()}
    reps, alive = gh.compare_stack(sub, layers_host, xs, k, shape.n_experts, label=label, residual=rs, pre=pre)
    say("  dense err %.3g; MoE layers compared %d, rows alive %d of %d; worst %.3g" % (
        err, len(reps), int(alive.sum()), len(sel), max(r["max_abs_over_max_ref"] for r in reps)))


@pytest.mark.parametrize("T", [17, 40, 300])
def test_prefill_stack_tiny_all_rows(T):
    # grouped MoE kernels (more than 16 rows), norm weights, residual stream;
    # 300 rows: the dense layer's LDS-ring kernels with a ragged last tile
    _prefill_case(TINY_SH, 512, T, 3, 20 + T, residual=True, gamma=True, label="tiny")


def test_prefill_stack_tiny_verify_width_rows():
    # a prefill short enough for the verify-width MoE kernels
    _prefill_case(TINY_SH, 256, 3, 2, 31, residual=False, gamma=True, label="tiny K=3")


def test_prefill_stack_full_size_sampled_rows():
    """The 512-row seed prefill through the dense layer (intermediate 8192)
    and 4 full-size MoE layers; 24 rows spread over the batch compared."""
    rows = np.linspace(0, 511, 24).astype(int)
    _prefill_case(inputs.LAGUNA, inputs.DENSE_INTER, 512, 4, 41, residual=True, gamma=True, rows=rows, label="full")


def test_prefill_stack_40_layers_sampled_rows():
    """The whole prefill FFN stack of the target (dense layer + 39 MoE
    layers) on 512 rows; 6 rows compared through every layer."""
    rows = np.array([0, 101, 202, 303, 404, 511])
    _prefill_case(inputs.LAGUNA, inputs.DENSE_INTER, 512, 39, 51, residual=False, gamma=False, rows=rows,
                  label="40-layer")
