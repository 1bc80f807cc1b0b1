"""GPU parity of chained layers (a9: RMSNorm glue with its norm weight, the
residual stream, graph launch).

Every layer of every stack is held to the single-layer bar (2e-3 of the
layer's largest output) against the oracle evaluating that layer; the
oracle chain follows its own values and adopts only admissible bf16
roundings (tests/gpu_helpers.py, compare_stack).  The glue itself is
checked on the GPU's own values at fp32 rounding distance.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from speculative_block_verify_amd import api, inputs
from tests import gpu_helpers as gh
from tests import refdecode as ref
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _host_layers(layers_dev):
    for w in layers_dev:
        yield {k: (None if v is None else ({kk: vv.cpu() for kk, vv in v.items()} if isinstance(v, dict) else v.cpu()))
               for k, v in w.items()}


def _with_norm_weights(layers, seed):
    g = torch.Generator().manual_seed(seed)
    for w in layers:
        gv = 0.5 + 1.5 * torch.rand(w["router_w"].shape[1], generator=g)
        w["norm_w"] = inputs.bf16_bits(gv).to(w["router_w"].device)
    return layers


def _stack_case(shape, n_layers, K, seed, label, regime=api.MOE_REGIME_AUTO, residual=False, gamma=False,
                laguna=False, correlated=False):
    say("case: stack %s L=%d K=%d seed=%d regime=%d residual=%d gamma=%d laguna=%d" % (
        label, n_layers, K, seed, regime, residual, gamma, laguna))
    layers = inputs.gen_stack(shape, n_layers, seed, device=DEV, with_bias=laguna)
    if gamma:
        _with_norm_weights(layers, seed)
    x = (inputs.gen_x_correlated if correlated else inputs.gen_x)(K, shape.hidden, seed, device=DEV)
    res = inputs.gen_x(K, shape.hidden, seed, device=DEV, tag="res") if residual else None
    score = api.MOE_SCORE_SIGMOID_BIAS if laguna else api.MOE_SCORE_SOFTMAX
    rs = 2.5 if laguna else 1.0
    cfg = api.make_cfg(shape, K, regime=regime, score_fn=score, routed_scale=rs)
    gpu = gh.run_stack_debug(cfg, layers, x, n_layers, residual=res)
    np.testing.assert_array_equal(gpu["y32_out"], gpu["y32"][-1])
    np.testing.assert_array_equal(gpu["y"], gh.bf16_of(gpu["y32_out"]))
    reps, alive = gh.compare_stack(gpu, _host_layers(layers), x.cpu().numpy(), shape.top_k, shape.n_experts,
                                   label=label, score_fn=score, rs=rs,
                                   residual=None if res is None else res.cpu().numpy())
    worst = max(r["max_abs_over_max_ref"] for r in reps)
    say("  layers compared %d, rows alive at end %s, worst max-abs/max-ref %.3g; input flips %s; glue flips %s"
        % (len(reps), alive.tolist(), worst, [r["input_flips"] for r in reps][:12],
           [r["glue_flips"] for r in reps][:12]))
    # every layer is compared: a row leaves only at a certified near-tie, and
    # at least one row runs through the whole stack
    assert len(reps) == n_layers and alive.any()
    return layers, x, cfg, gpu


def test_stack_tiny_40_layers():
    _stack_case(inputs.TINY, 40, 1, 3, "tiny")


def test_stack_tiny_shared_40_layers_k4():
    shape = inputs.MoEShape(256, 16, 2, 128, 128)
    _stack_case(shape, 40, 4, 5, "tiny-shared")


def test_stack_full_size_4_layers_k2():
    _stack_case(inputs.LAGUNA, 4, 2, 9, "full-4")


@pytest.mark.parametrize("K,regime", [(1, api.MOE_REGIME_AUTO), (4, api.MOE_REGIME_AUTO), (5, api.MOE_REGIME_AUTO),
                                      (8, api.MOE_REGIME_VERIFY), (8, api.MOE_REGIME_AUTO),
                                      (16, api.MOE_REGIME_VERIFY), (16, api.MOE_REGIME_AUTO)])
def test_stack_full_size_6_layers_row_counts(K, regime):
    # verify widths other than the benchmark's two rows, through the RMSNorm
    # glue (sum-of-squares partials of every row, or the grouped combine's
    # normalised next input from 8 rows in the automatic regime) and the stack
    # entry point; 4 and 5 rows run the down kernel's 96 KB and 8-wave shapes
    _stack_case(inputs.LAGUNA, 6, K, 40 + K, "full-6-K%d-r%d" % (K, regime), regime=regime)


@pytest.mark.parametrize("K,regime", [(2, api.MOE_REGIME_AUTO), (16, api.MOE_REGIME_AUTO)])
def test_stack_norm_weight_and_residual_stream(K, regime):
    # the RMSNorm weight of each layer (router prologue at verify width, the
    # grouped combine at 16 rows) and the residual stream updated in place
    _stack_case(inputs.LAGUNA, 5, K, 70 + K, "full-5-gamma-res-K%d" % K, regime=regime, residual=True, gamma=True)


@pytest.mark.parametrize("K", [2, 16])
def test_stack_laguna_mode(K):
    # the pages' router tail (sigmoid + selection bias, normalised top-k,
    # routed scale 2.5) with norm weights and the residual stream
    _stack_case(inputs.LAGUNA, 4, K, 90 + K, "laguna-K%d" % K, residual=True, gamma=True, laguna=True,
                correlated=K > 2)


def test_stack_tiny_gamma_residual_40_layers_both_regimes():
    shape = inputs.MoEShape(256, 16, 2, 128, 128)
    for regime in (api.MOE_REGIME_VERIFY, api.MOE_REGIME_GROUPED):
        _stack_case(shape, 40, 3, 11, "tiny-gamma-res-r%d" % regime, regime=regime, residual=True, gamma=True)


def test_stack_full_size_40_layers_graph_matches_direct_and_oracle():
    """The benchmark's configuration: 40 full-size layers, K = 2, launched as
    a captured graph.  The graph's output must equal the direct call bit for
    bit on every replay (with eager work in between), and every one of the
    direct call's 40 layers must match the oracle."""
    layers, x, cfg, gpu = _stack_case(inputs.LAGUNA, 40, 2, 1, "full-40")
    K, H = x.shape
    y = torch.empty(K, H, dtype=torch.int16, device=DEV)
    y32 = torch.empty(K, H, dtype=torch.float32, device=DEV)
    ws = api.alloc_workspace(cfg, DEV)
    g = api.StackGraph(cfg, [api.make_weights(w) for w in layers], x, y, ws, y32=y32)
    for rep in range(4):
        y32.fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y32.cpu().numpy(), gpu["y32_out"])
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        api.moe_verify_stack(cfg, [api.make_weights(w) for w in layers[:3]], x, y, ws, y32=y32)
        torch.cuda.synchronize()
        del junk
    g.close()


def test_stack_graph_with_residual_matches_direct():
    """A captured stack with norm weights and the residual stream replays to
    the direct call's output bit for bit (the stream is updated in place, so
    every replay must start from the caller's residual again)."""
    say("case: stack graph with residual L=6 K=2")
    shape, n_layers, K = inputs.LAGUNA, 6, 2
    layers = _with_norm_weights(inputs.gen_stack(shape, n_layers, 81, device=DEV), 81)
    x = inputs.gen_x(K, shape.hidden, 81, device=DEV)
    res = inputs.gen_x(K, shape.hidden, 82, device=DEV, tag="res")
    cfg = api.make_cfg(shape, K)
    wts = [api.make_weights(w) for w in layers]
    y = torch.empty(K, shape.hidden, dtype=torch.int16, device=DEV)
    y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=DEV)
    ws = api.alloc_workspace(cfg, DEV)
    api.moe_verify_stack(cfg, wts, x, y, ws, y32=y32, residual=res)
    torch.cuda.synchronize()
    want32 = y32.cpu().numpy().copy()
    g = api.StackGraph(cfg, wts, x, y, ws, y32=y32, residual=res)
    for rep in range(3):
        y32.fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y32.cpu().numpy(), want32)
    g.close()


def test_stack_graph_grouped_regime_16_rows_matches_direct():
    """The K sweep's widest point as the benchmark runs it: 16 correlated rows,
    where the automatic regime picks the grouped kernels, replayed as a
    captured graph.  Every replay (with eager work in between) must equal the
    direct stack call bit for bit; the direct call itself is checked against
    the oracle by the row-count stack tests."""
    say("case: stack graph grouped regime K=16 L=6")
    shape, n_layers, K = inputs.LAGUNA, 6, 16
    layers = inputs.gen_stack(shape, n_layers, 61, device=DEV)
    x = inputs.gen_x_correlated(K, shape.hidden, 61, device=DEV)
    cfg = api.make_cfg(shape, K)
    wts = [api.make_weights(w) for w in layers]
    y = torch.empty(K, shape.hidden, dtype=torch.int16, device=DEV)
    y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=DEV)
    ws = api.alloc_workspace(cfg, DEV)
    api.moe_verify_stack(cfg, wts, x, y, ws, y32=y32)
    torch.cuda.synchronize()
    want32, want = y32.cpu().numpy().copy(), y.cpu().numpy().copy()
    assert np.isfinite(want32).all()
    g = api.StackGraph(cfg, wts, x, y, ws, y32=y32)
    for rep in range(3):
        y32.fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y32.cpu().numpy(), want32)
        np.testing.assert_array_equal(y.cpu().numpy(), want)
        junk = torch.randn(1 << 20, device=DEV).sum()
        api.moe_verify_stack(cfg, wts[:2], x, y, ws, y32=y32)
        torch.cuda.synchronize()
        del junk
    g.close()
