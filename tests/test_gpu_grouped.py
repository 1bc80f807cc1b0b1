"""GPU parity of the grouped (prefill) regime: more than 16 rows, the slots
grouped by expert into tiles of up to 32 tokens, expert GEMMs on the matrix
cores.  Same oracle and comparison rules as the verify-width tests
(tests/gpu_helpers.py); every input is seeded and synthetic.
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


# ---------------------------------------------------------------------------
# selection + grouping from given logits, bit-exact
# ---------------------------------------------------------------------------


def _route(K, E, k, logits, shared=512):
    shape = inputs.MoEShape(hidden=256, n_experts=E, top_k=k, inter=128, shared_inter=shared)
    cfg = api.make_cfg(shape, K)
    n = K * k
    out = {"ids": torch.empty(n, dtype=torch.int32, device=DEV), "w": torch.empty(n, dtype=torch.float32, device=DEV),
           "n_unique": torch.empty(1, dtype=torch.int32, device=DEV),
           "uniq": torch.empty(n, dtype=torch.int32, device=DEV),
           "off": torch.empty(n + 1, dtype=torch.int32, device=DEV),
           "asg": torch.empty(n, dtype=torch.int32, device=DEV), "inv": torch.empty(n, dtype=torch.int32, device=DEV)}
    lt = torch.as_tensor(logits, dtype=torch.float32).contiguous()
    ws = api.alloc_workspace(cfg, DEV)
    api.moe_verify_route(cfg, lt.to(DEV), out, workspace=ws)
    torch.cuda.synchronize()
    got = {kk: v.cpu().numpy() for kk, v in out.items()}
    ids, w = orc.topk(lt.numpy(), k, 0, 1, None)
    np.testing.assert_array_equal(got["ids"].reshape(K, k), ids)
    np.testing.assert_allclose(got["w"].reshape(K, k), w, rtol=1e-6, atol=1e-7)
    d = orc.dedup(ids, E)
    U = d["n_unique"]
    assert int(got["n_unique"][0]) == U
    np.testing.assert_array_equal(got["uniq"][:U], d["uniq"])
    np.testing.assert_array_equal(got["off"][:U + 1], d["off"])
    np.testing.assert_array_equal(got["asg"], d["asg"])
    np.testing.assert_array_equal(got["inv"], d["inv"])
    return U


@pytest.mark.parametrize("K,E,k", [(17, 16, 2), (64, 256, 8), (300, 256, 8), (1024, 64, 4), (40, 1024, 32)])
def test_grouped_route_random_logits(K, E, k):
    say("case: grouped route K=%d E=%d k=%d" % (K, E, k))
    rng = np.random.default_rng(K + 7 * E + k)
    _route(K, E, k, rng.standard_normal((K, E)).astype(np.float32))


def test_grouped_route_ties_and_one_hot_experts():
    say("case: grouped route ties")
    K, E, k = 96, 256, 8
    rng = np.random.default_rng(5)
    l = rng.standard_normal((K, E)).astype(np.float32)
    l[:40] = 0.0                       # 40 all-tied rows: experts 0..7, 40 tokens each (two tiles)
    l[40:50] = np.float32(-1e30)
    l[40:50, 200:208] = 1.0            # ten rows on experts 200..207
    U = _route(K, E, k, l)
    assert U >= 16


# ---------------------------------------------------------------------------
# layers
# ---------------------------------------------------------------------------


def _layer(shape, K, seed, grouped=True, x=None, score_fn=0, rs=1.0, residual=False, label=""):
    say("case: grouped layer %s K=%d seed=%d" % (label, K, seed))
    w = inputs.gen_layer(shape, seed, 0, device=DEV, with_bias=(score_fn == 1))
    x = inputs.gen_x(K, shape.hidden, seed, device=DEV) if x is None else x
    res = inputs.gen_x(K, shape.hidden, seed + 1, device=DEV, tag="res") if residual else None
    cfg = api.make_cfg(shape, max(K, 17), score_fn=score_fn, routed_scale=rs)
    gpu = gh.run_layer(cfg, w, x, residual=res, grouped=grouped)
    orec = orc.moe_layer(w, x.cpu(), shape.top_k, score_fn, 1, rs, None if res is None else res.cpu())
    bias = None if score_fn == 0 else w["router_bias"].cpu().numpy()
    rep = gh.compare_layer(gpu, orec, shape.top_k, shape.n_experts, score_fn, bias, label=label)
    np.testing.assert_array_equal(gpu["y"], gh.bf16_of(gpu["y32"]))
    np.testing.assert_array_equal(gpu["y32"], gpu["y32_out"])
    say("  report:", rep, "n_unique", int(gpu["n_unique"][0]))
    return gpu, orec


@pytest.mark.parametrize("K", [1, 3, 16, 17, 40, 100])
def test_grouped_layer_tiny_shapes(K):
    # hidden 256, 16 experts, top-2, intermediate 128, shared 128; K <= 16 runs
    # the grouped kernels through moe_verify_layer_grouped
    _layer(TINY_SH, K, 200 + K, label="tiny+shared")


@pytest.mark.parametrize("case", ["big", "tiny", "small", "mixed"])
def test_grouped_layer_activation_range_beyond_fp16(case):
    # the router's fp16 copy of x carries a per-row power-of-two scale that
    # the grouped gate/up undoes: rows of any bf16 magnitude match the oracle
    from tests.test_gpu_parity import range_cases
    H = inputs.LAGUNA.hidden
    x = dict(range_cases(H))[case]
    # 24 rows: the case's rows repeated with a few ordinary rows between
    rows = [x[i % x.shape[0]] for i in range(12)] + [inputs.gen_x(12, H, 9)[i] for i in range(12)]
    xr = torch.stack(rows).contiguous().to(DEV)
    gpu, orec = _layer(inputs.LAGUNA, xr.shape[0], 19, x=xr, label="range-" + case)
    assert np.isfinite(gpu["y32"]).all()
    # and each row at the bar of its own largest output (rows of very
    # different magnitude share the layer)
    err = np.abs(gpu["y32"].astype(np.float64) - orec["y"]).max(axis=1)
    assert np.all(err <= 2e-3 * np.abs(orec["y"]).max(axis=1)), err / np.abs(orec["y"]).max(axis=1)


def test_grouped_layer_no_shared_expert():
    _layer(inputs.MoEShape(512, 32, 4, 256, 0), 50, 9, label="no shared")


@pytest.mark.parametrize("shape,K", [
    # hidden 1024 (four gate/up superblocks), intermediate and shared 1024:
    # the down kernel stages 4-superblock rows, one workgroup per compute unit
    (inputs.MoEShape(1024, 64, 4, 1024, 1024), 40),
    # hidden 2048, intermediate 1024 with a shorter shared expert (512): rows
    # of two lengths in the same staged tile width
    (inputs.MoEShape(2048, 128, 8, 1024, 512), 24),
])
def test_grouped_layer_wide_intermediate(shape, K):
    _layer(shape, K, 60 + K, label="wide I=%d Is=%d" % (shape.inter, shape.shared_inter))


@pytest.mark.parametrize("shape,K", [
    # 1024 experts at top-32: 5120 slots (more than the 16 per thread a
    # gate/up workgroup holds in registers while grouping) and the largest
    # per-expert tables
    (inputs.MoEShape(256, 1024, 32, 128, 128), 160),
    # 1000 rows at top-8: 8000 slots and 32 row-bitmap words per expert
    (inputs.MoEShape(256, 64, 8, 128, 128), 1000),
])
def test_grouped_layer_many_slots_and_experts(shape, K):
    _layer(shape, K, 70 + K, label="E=%d k=%d" % (shape.n_experts, shape.top_k))


def test_grouped_layer_correlated_rows_span_several_tiles():
    # rows 1..K/2 are row 0 plus small noise: their experts get ~40+ tokens
    # each, so one expert spans two or three 32-token tiles with a ragged tail
    K = 90
    x = inputs.gen_x_correlated(K, inputs.LAGUNA.hidden, 77, device=DEV)
    gpu, _ = _layer(inputs.LAGUNA, K, 77, x=x, label="correlated")
    counts = np.diff(gpu["off"][: int(gpu["n_unique"][0]) + 1])
    assert counts.max() > 32


def test_grouped_layer_sigmoid_bias_scale_and_residual():
    _layer(inputs.LAGUNA, 48, 21, score_fn=1, rs=2.5, residual=True, label="sigmoid")


def test_grouped_and_verify_width_paths_agree_at_16_rows():
    say("case: grouped vs verify width K=16")
    shape = inputs.LAGUNA
    w = inputs.gen_layer(shape, 41, 0, device=DEV)
    x = inputs.gen_x(16, shape.hidden, 41, device=DEV)
    cfg = api.make_cfg(shape, 16, regime=api.MOE_REGIME_VERIFY)
    a = gh.run_layer(cfg, w, x, grouped=False)
    b = gh.run_layer(cfg, w, x, grouped=True)
    # the two regimes run different router kernels (VALU GEMV, MFMA GEMM):
    # logits agree to the logit bar; selection must then agree on every row
    # whose k-th / (k+1)-th logit gap is above it (no such near tie here)
    la, lb = a["logits"].reshape(16, -1), b["logits"].reshape(16, -1)
    tol = 1e-5 * np.abs(la).max()
    assert np.abs(la - lb).max() <= tol
    srt = -np.sort(-la, axis=1)
    assert (srt[:, shape.top_k - 1] - srt[:, shape.top_k]).min() > 2 * tol
    for kk in ("ids", "n_unique", "uniq", "off", "asg", "inv"):
        np.testing.assert_array_equal(a[kk], b[kk], err_msg=kk)
    np.testing.assert_allclose(a["w"], b["w"], rtol=1e-5, atol=1e-7)
    scale = np.abs(a["y32"]).max()
    assert np.abs(a["y32"] - b["y32"]).max() <= 2 * gh.Y_TOL * scale


def test_few_row_router_matches_many_row_router():
    """Up to 16 rows the grouped layer runs the router's eight column slices as
    workgroups of their own and adds their partial logits in the selection
    launch, in the order the many-row router adds its waves' tiles; it also
    makes the fp16 copy of x there.  Rows 0..15 of a 17-row call (many-row
    router) and of a 16-row call on the same rows must then have the same
    logits, selections and weights bit for bit, and the same outputs."""
    say("case: few-row vs many-row router, 16 / 17 rows")
    shape = inputs.MoEShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512)
    w = inputs.gen_layer(shape, 47, 0, device=DEV)
    x = inputs.gen_x(17, shape.hidden, 47, device=DEV)
    a = gh.run_layer(api.make_cfg(shape, 17), w, x, grouped=True)
    b = gh.run_layer(api.make_cfg(shape, 16), w, x[:16].contiguous(), grouped=True)
    E, k = shape.n_experts, shape.top_k
    np.testing.assert_array_equal(a["logits"].reshape(17, E)[:16].view(np.uint32),
                                  b["logits"].reshape(16, E).view(np.uint32))
    np.testing.assert_array_equal(a["ids"].reshape(17, k)[:16], b["ids"].reshape(16, k))
    np.testing.assert_array_equal(a["w"].reshape(17, k)[:16].view(np.uint32), b["w"].reshape(16, k).view(np.uint32))
    ya, yb = a["y32"].reshape(17, -1)[:16], b["y32"].reshape(16, -1)
    assert np.abs(ya - yb).max() <= 1e-6 * np.abs(ya).max()


def test_grouped_layer_bitwise_invariants():
    say("case: grouped invariants")
    shape = inputs.LAGUNA
    w = inputs.gen_layer(shape, 43, 0, device=DEV)
    cfg = api.make_cfg(shape, 64)
    x = inputs.gen_x(64, shape.hidden, 43, device=DEV)
    a = gh.run_layer(cfg, w, x)
    b = gh.run_layer(cfg, w, x)
    np.testing.assert_array_equal(a["y32"], b["y32"])
    x1 = inputs.gen_x(1, shape.hidden, 44, device=DEV).repeat(40, 1).contiguous()
    c = gh.run_layer(cfg, w, x1)
    for r in range(1, 40):
        np.testing.assert_array_equal(c["y32"][0], c["y32"][r])


def test_grouped_stack_tiny_free_running():
    say("case: grouped stack tiny 6 layers K=40")
    shape, L, K = TINY_SH, 6, 40
    layers = inputs.gen_stack(shape, L, 61, device=DEV)
    x = inputs.gen_x(K, shape.hidden, 61, device=DEV)
    cfg = api.make_cfg(shape, K)
    gpu = gh.run_stack_debug(cfg, layers, x, L)
    host = [{kk: (None if v is None else ({a: b.cpu() for a, b in v.items()} if isinstance(v, dict) else v.cpu()))
             for kk, v in w.items()} for w in layers]
    reps, alive = gh.compare_stack(gpu, host, x.cpu().numpy(), shape.top_k, shape.n_experts, label="grouped stack")
    say("  worst max-abs/max-ref %.3g, rows alive %d" % (max(r["max_abs_over_max_ref"] for r in reps), alive.sum()))
    assert len(reps) == L and alive.any()
    np.testing.assert_array_equal(gpu["y32_out"], gpu["y32"][L - 1])


# ---------------------------------------------------------------------------
# the prefill configuration at full size: 512 rows, hidden 2048, 256 experts,
# top-8, intermediate 512, shared 512 -- every row against the oracle
# ---------------------------------------------------------------------------


def test_grouped_prefill_512_rows():
    say("case: prefill 512 rows")
    shape, T = inputs.LAGUNA, 512
    w = inputs.gen_layer(shape, 512, 0, device=DEV)
    x = inputs.gen_x(T, shape.hidden, 512, device=DEV)
    cfg = api.make_cfg(shape, T)
    gpu = gh.run_layer(cfg, w, x)
    U = int(gpu["n_unique"][0])
    counts = np.diff(gpu["off"][: U + 1])
    say("  experts used %d, tokens per expert min %d mean %.1f max %d" % (U, counts.min(), counts.mean(),
                                                                        counts.max()))
    np.testing.assert_array_equal(gpu["y"], gh.bf16_of(gpu["y32"]))
    host = {kk: (None if v is None else ({a: b.cpu() for a, b in v.items()} if isinstance(v, dict) else v.cpu()))
            for kk, v in w.items()}
    orec = gh.oracle_layer_rows(host, x, shape.top_k)
    rep = gh.compare_layer(gpu, orec, shape.top_k, shape.n_experts, label="prefill 512 rows")
    say("  report:", {k: v for k, v in rep.items() if k != "tie_rows"})


@pytest.mark.parametrize("K,grouped_auto", [(7, False), (8, True)])
def test_automatic_regime_switch_at_8_rows(K, grouped_auto):
    """From 8 rows the automatic regime runs the grouped kernels: its output is
    then bitwise the forced-grouped entry's; below 8 rows it is bitwise the
    forced verify-width kernels'."""
    say("case: automatic regime K=%d" % K)
    shape = inputs.LAGUNA
    w = inputs.gen_layer(shape, 71 + K, 0, device=DEV)
    x = inputs.gen_x(K, shape.hidden, 71 + K, device=DEV)
    auto = gh.run_layer(api.make_cfg(shape, K), w, x)
    if grouped_auto:
        ref = gh.run_layer(api.make_cfg(shape, K), w, x, grouped=True)
    else:
        ref = gh.run_layer(api.make_cfg(shape, K, regime=api.MOE_REGIME_VERIFY), w, x)
    for kk in ("ids", "n_unique", "uniq", "off", "asg", "inv", "y32", "y"):
        np.testing.assert_array_equal(auto[kk], ref[kk], err_msg=kk)
