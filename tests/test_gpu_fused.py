"""The one-launch verify layer (MOE_REGIME_VERIFY_ONE_LAUNCH, at most 2
rows: router, gate/up and down workgroups in a single launch with in-kernel
hand-offs) against the two-launch layer (router + gate/up, then down) that
the other regimes run.

Both forms run the same arithmetic in the same order (decode, per-task FMA
chains, cross-lane sums, rank-order combine), so every output and every
debug array must agree bit for bit; the oracle parity of the two-launch
form is covered by the layer and stack tests, and a tiny one-launch case
here is held to the oracle directly.
"""
import numpy as np
import pytest
import torch

from speculative_block_verify_amd import api, inputs
from tests import gpu_helpers as gh
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
TINY_SH = inputs.MoEShape(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128)
MID = inputs.MoEShape(hidden=512, n_experts=64, top_k=4, inter=256, shared_inter=0)
FULL = inputs.LAGUNA
KEYS = ("logits", "ids", "w", "n_unique", "uniq", "off", "asg", "inv", "x_in", "y32", "y", "y32_out")


def say(*a):
    print(*a, flush=True)


def _layer_pair(shape, K, seed, score_fn=api.MOE_SCORE_SOFTMAX, rs=1.0, residual=False):
    w = inputs.gen_layer(shape, seed, device=DEV, with_bias=score_fn == api.MOE_SCORE_SIGMOID_BIAS)
    x = inputs.gen_x(K, shape.hidden, seed, device=DEV)
    res = inputs.gen_x(K, shape.hidden, seed, device=DEV, tag="res") if residual else None
    out = {}
    for name, regime in (("one", api.MOE_REGIME_VERIFY_ONE_LAUNCH), ("split", api.MOE_REGIME_AUTO)):
        cfg = api.make_cfg(shape, K, score_fn=score_fn, routed_scale=rs, regime=regime)
        out[name] = gh.run_layer(cfg, w, x, residual=res)
    return out


def _assert_same(a, b, label):
    n_u = int(a["n_unique"][0])
    for k in KEYS:
        va, vb = a[k], b[k]
        if k == "uniq":
            va, vb = va[:n_u], vb[:n_u]
        if k == "off":
            va, vb = va[: n_u + 1], vb[: n_u + 1]
        np.testing.assert_array_equal(np.asarray(va).view(np.uint8), np.asarray(vb).view(np.uint8),
                                      err_msg="%s: %s differs" % (label, k))


@pytest.mark.parametrize("shape_name,K", [("tiny_shared", 1), ("tiny_shared", 2), ("mid", 1), ("mid", 2),
                                          ("full", 1), ("full", 2)])
def test_one_launch_layer_equals_split_layer(shape_name, K):
    shape = {"tiny_shared": TINY_SH, "mid": MID, "full": FULL}[shape_name]
    for seed in (1, 2):
        say("case: one-launch vs split layer %s K=%d seed=%d" % (shape_name, K, seed))
        p = _layer_pair(shape, K, 300 + seed + 10 * K)
        _assert_same(p["one"], p["split"], "%s K=%d seed=%d" % (shape_name, K, seed))


def test_one_launch_layer_sigmoid_bias_residual_equals_split():
    say("case: one-launch vs split, sigmoid + bias, rs 2.5, residual, full size K=2")
    p = _layer_pair(FULL, 2, 77, score_fn=api.MOE_SCORE_SIGMOID_BIAS, rs=2.5, residual=True)
    _assert_same(p["one"], p["split"], "laguna mode")


def test_one_launch_layer_tiny_no_shared_matches_oracle():
    """The tiny shape without a shared expert (one task per expert) in one
    launch, against the oracle at the layer bar."""
    import oracle as orc
    shape = inputs.TINY
    for K in (1, 2):
        say("case: one-launch tiny K=%d vs oracle" % K)
        w = inputs.gen_layer(shape, 40 + K, device=DEV)
        x = inputs.gen_x(K, shape.hidden, 40 + K, device=DEV)
        gpu = gh.run_layer(api.make_cfg(shape, K, regime=api.MOE_REGIME_VERIFY_ONE_LAUNCH), w, x)
        orec = orc.moe_layer(w, x.cpu(), shape.top_k, 0, 1, 1.0, None)
        say("  ", gh.compare_layer(gpu, orec, shape.top_k, shape.n_experts, label="tiny one-launch"))


def test_one_launch_stack_equals_split_stack_and_graph_replays():
    """Six full-size layers at K=2 with norm weights and the residual
    stream: the one-launch stack equals the split stack in every layer's
    debug arrays, and a graph of it replays to the same bits several times
    with eager work in between."""
    shape, K, L = FULL, 2, 6
    layers = inputs.gen_stack(shape, L, 91, device=DEV)
    g = torch.Generator().manual_seed(91)
    for w in layers:
        w["norm_w"] = inputs.bf16_bits(0.5 + 1.5 * torch.rand(shape.hidden, generator=g)).to(DEV)
    x = inputs.gen_x(K, shape.hidden, 91, device=DEV)
    res = inputs.gen_x(K, shape.hidden, 91, device=DEV, tag="res")
    runs = {}
    for name, regime in (("one", api.MOE_REGIME_VERIFY_ONE_LAUNCH), ("split", api.MOE_REGIME_AUTO)):
        say("case: stack L=%d K=%d %s" % (L, K, name))
        cfg = api.make_cfg(shape, K, regime=regime)
        runs[name] = gh.run_stack_debug(cfg, layers, x, L, residual=res)
    for k in ("logits", "ids", "w", "x_in", "y32", "res_in", "y", "y32_out"):
        np.testing.assert_array_equal(np.asarray(runs["one"][k]).view(np.uint8),
                                      np.asarray(runs["split"][k]).view(np.uint8), err_msg="stack " + k)

    say("case: one-launch stack graph, 4 replays")
    cfg = api.make_cfg(shape, K, regime=api.MOE_REGIME_VERIFY_ONE_LAUNCH)
    wts = [api.make_weights(w, cfg) for w in layers]
    ws = api.alloc_workspace(cfg, DEV)
    y = torch.empty(K, shape.hidden, dtype=torch.int16, device=DEV)
    y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=DEV)
    graph = api.StackGraph(cfg, wts, x, y, ws, y32=y32, residual=res)
    try:
        for rep in range(4):
            y32.fill_(float("nan"))
            graph.launch()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y32.cpu().numpy(), runs["one"]["y32_out"], err_msg="replay %d" % rep)
            np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16), runs["one"]["y"])
            # eager work between replays (another input through the same workspace)
            api.moe_verify_stack(cfg, wts, inputs.gen_x(K, shape.hidden, 92 + rep, device=DEV), y, ws, y32=y32)
            torch.cuda.synchronize()
    finally:
        graph.close()


def test_one_launch_stack_timed_reports_the_whole_layer():
    shape, K, L = FULL, 2, 3
    layers = inputs.gen_stack(shape, L, 17, device=DEV)
    x = inputs.gen_x(K, shape.hidden, 17, device=DEV)
    for regime, one in ((api.MOE_REGIME_VERIFY_ONE_LAUNCH, True), (api.MOE_REGIME_AUTO, False)):
        say("case: stack_timed regime=%d" % regime)
        cfg = api.make_cfg(shape, K, regime=regime)
        wts = [api.make_weights(w, cfg) for w in layers]
        ws = api.alloc_workspace(cfg, DEV)
        y = torch.empty(K, shape.hidden, dtype=torch.int16, device=DEV)
        ms = api.moe_verify_stack_timed(cfg, wts, x, y, ws)
        assert len(ms) == L
        for a, b in ms:
            assert a > 0.0
            assert (b == 0.0) if one else (b > 0.0)
