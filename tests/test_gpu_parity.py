"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input is seeded and synthetic (speculative_block_verify_amd.inputs);
expected values come from the oracle only.  Run on an MI355X:
    python -u -m pytest tests -m gpu -x -v --timeout 300 --timeout-method thread
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


# ---------------------------------------------------------------------------
# a4: the in-kernel NVFP4 decode, bit-exact
# ---------------------------------------------------------------------------


def test_dequant_matches_oracle_bit_exact():
    say("case: dequant all codes")
    # every E2M1 nibble pair and every finite E4M3 scale byte appear
    E, rows, cols = 2, 64, 512
    g = torch.Generator().manual_seed(5)
    q = torch.randint(0, 256, (E, rows, cols // 2), generator=g, dtype=torch.uint8)
    q.view(-1)[:256] = torch.arange(256, dtype=torch.uint8)
    s = torch.randint(0, 256, (E, rows, cols // 16), generator=g, dtype=torch.uint8)
    s.view(-1)[:256] = torch.arange(256, dtype=torch.uint8)
    s[(s == 0x7F) | (s == 0xFF)] = 0x38
    ts = torch.tensor([1.0, 3.0e-5], dtype=torch.float32)
    m = {"q": q, "s": s, "ts": ts}
    md = api.to_device(m)
    out = torch.empty(E, rows, cols, dtype=torch.float32, device=DEV)
    api.moe_verify_dequant_nvfp4(md, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for e in range(E):
        want = orc.dequant(m, e).astype(np.float32)
        np.testing.assert_array_equal(got[e], want)


def test_dequant_every_code_and_scale_by_every_decode_route():
    """Every E2M1 code times every finite E4M3 scale, through the three
    decode routes of the GEMM kernels (fp32, bf16, and the fp16 operand decode
    of the matrix-core gate/up tiles; the kernel marks any disagreement NaN),
    bit-exact against the oracle's fp64 decode rounded to fp32."""
    say("case: dequant every code x scale")
    rows = 256
    codes = np.arange(16, dtype=np.uint8)
    blk = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)      # 16 codes in 8 bytes
    q = np.tile(np.concatenate([blk, blk]), (2, rows, 1))            # two 16-column blocks per row
    sb = np.arange(rows, dtype=np.uint8)
    sb[0x7F], sb[0xFF] = 0x7E, 0xFE                                  # the two NaN codes -> largest finite
    s = np.repeat(sb[None, :, None], 2, axis=2).repeat(2, axis=0)
    m = {"q": torch.as_tensor(q.copy()), "s": torch.as_tensor(s.copy()),
         "ts": torch.tensor([1.0, 3.0e-5], dtype=torch.float32)}
    md = api.to_device(m)
    out = torch.empty(2, rows, 32, dtype=torch.float32, device=DEV)
    api.moe_verify_dequant_nvfp4(md, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any(), "decode routes disagree"
    for e in range(2):
        np.testing.assert_array_equal(got[e], orc.dequant(m, e).astype(np.float32))


# ---------------------------------------------------------------------------
# a2 + a3: selection and dedup from given logits, bit-exact
# ---------------------------------------------------------------------------


def _route_case(K, E, k, logits, score_fn=0, bias=None, norm=1):
    shape = inputs.MoEShape(hidden=256, n_experts=E, top_k=k, inter=128, shared_inter=0)
    cfg = api.make_cfg(shape, max(K, 1), score_fn=score_fn, norm_topk=norm)
    n = K * k
    out = {"ids": torch.empty(n, dtype=torch.int32, device=DEV), "w": torch.empty(n, dtype=torch.float32, device=DEV),
           "n_unique": torch.empty(1, dtype=torch.int32, device=DEV),
           "uniq": torch.empty(n, dtype=torch.int32, device=DEV),
           "off": torch.empty(n + 1, dtype=torch.int32, device=DEV),
           "asg": torch.empty(n, dtype=torch.int32, device=DEV), "inv": torch.empty(n, dtype=torch.int32, device=DEV)}
    lt = torch.as_tensor(logits, dtype=torch.float32).contiguous()
    bt = None if bias is None else torch.as_tensor(bias, dtype=torch.float32).to(DEV)
    api.moe_verify_route(cfg, lt.to(DEV), out, bias=bt)
    torch.cuda.synchronize()
    got = {kk: v.cpu().numpy() for kk, v in out.items()}
    ids, w = orc.topk(lt.numpy(), k, score_fn, norm, None if bias is None else np.asarray(bias, np.float32))
    np.testing.assert_array_equal(got["ids"].reshape(K, k), ids)
    np.testing.assert_allclose(got["w"].reshape(K, k), w, rtol=1e-6, atol=1e-7)
    d = orc.dedup(ids, E)
    U = d["n_unique"]
    assert int(got["n_unique"][0]) == U
    np.testing.assert_array_equal(got["uniq"][:U], d["uniq"])
    np.testing.assert_array_equal(got["off"][:U + 1], d["off"])
    np.testing.assert_array_equal(got["asg"], d["asg"])
    np.testing.assert_array_equal(got["inv"], d["inv"])


@pytest.mark.parametrize("K,E,k", [(1, 16, 2), (2, 256, 8), (16, 256, 8), (4, 1024, 32), (3, 32, 32), (5, 7, 3)])
def test_route_random_logits(K, E, k):
    say("case: route K=%d E=%d k=%d" % (K, E, k))
    rng = np.random.default_rng(K * 1000 + E + k)
    _route_case(K, E, k, rng.standard_normal((K, E)).astype(np.float32))


def test_route_ties_zeros_and_repeats():
    say("case: route ties")
    K, E, k = 4, 256, 8
    l = np.zeros((K, E), np.float32)           # row 0: all tied -> 0..7, w = 1/8
    l[1] = np.repeat(np.arange(32, dtype=np.float32), 8)[::-1]  # blocks of 8 equal values
    l[2, ::3] = 1.0                             # many equal maxima
    l[2, 5] = -0.0
    l[3] = np.float32(-1e30)
    l[3, 200] = 0.0
    _route_case(K, E, k, l)
    # identical rows share every expert: n_unique = k
    rng = np.random.default_rng(3)
    row = rng.standard_normal(E).astype(np.float32)
    _route_case(8, E, k, np.tile(row, (8, 1)))


@pytest.mark.parametrize("norm", [1, 0])
def test_route_sigmoid_bias(norm):
    say("case: route sigmoid norm=%d" % norm)
    rng = np.random.default_rng(11 + norm)
    K, E, k = 3, 256, 8
    l = rng.standard_normal((K, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.01).astype(np.float32)
    _route_case(K, E, k, l, score_fn=1, bias=b, norm=norm)


# ---------------------------------------------------------------------------
# a1-a8: one layer
# ---------------------------------------------------------------------------


def _layer_case(shape, K, seed, score_fn=0, rs=1.0, residual=False, x=None, label="", regime=api.MOE_REGIME_AUTO):
    say("case: layer %s K=%d seed=%d score_fn=%d regime=%d" % (label, K, seed, score_fn, regime))
    w = inputs.gen_layer(shape, seed, 0, device=DEV, with_bias=(score_fn == 1))
    x = inputs.gen_x(K, shape.hidden, seed, device=DEV) if x is None else x
    res = inputs.gen_x(K, shape.hidden, seed + 1, device=DEV, tag="res") if residual else None
    cfg = api.make_cfg(shape, K, score_fn=score_fn, routed_scale=rs, regime=regime)
    gpu = gh.run_layer(cfg, w, x, residual=res)
    orec = orc.moe_layer(w, x.cpu(), shape.top_k, score_fn, 1, rs, None if res is None else res.cpu())
    bias = None if score_fn == 0 else w["router_bias"].cpu().numpy()
    rep = gh.compare_layer(gpu, orec, shape.top_k, shape.n_experts, score_fn, bias, label=label)
    np.testing.assert_array_equal(gpu["y"], gh.bf16_of(gpu["y32"]))
    np.testing.assert_array_equal(gpu["y32"], gpu["y32_out"])
    np.testing.assert_array_equal(gpu["x_in"], x.cpu().numpy())
    say("  report:", rep, "n_unique", int(gpu["n_unique"][0]))
    return gpu, orec, rep


def test_layer_tiny_config():
    # hidden 256, 16 experts, top-2, intermediate 128, no shared expert, one row
    _layer_case(inputs.TINY, 1, 0, label="tiny")


@pytest.mark.parametrize("K", [1, 2, 3, 8, 16])
def test_layer_tiny_shapes_many_rows(K):
    # the verify-width kernels at every row count they serve
    shape = inputs.MoEShape(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128)
    _layer_case(shape, K, 100 + K, label="tiny+shared", regime=api.MOE_REGIME_VERIFY)


def test_layer_full_size_k2():
    # hidden 2048, 256 experts, top-8, intermediate 512, shared 512, two rows
    _layer_case(inputs.LAGUNA, 2, 7, label="full")


@pytest.mark.parametrize("K,regime", [(1, api.MOE_REGIME_AUTO), (3, api.MOE_REGIME_AUTO), (4, api.MOE_REGIME_AUTO),
                                      (5, api.MOE_REGIME_AUTO),
                                      (8, api.MOE_REGIME_VERIFY), (8, api.MOE_REGIME_AUTO),
                                      (16, api.MOE_REGIME_VERIFY), (16, api.MOE_REGIME_AUTO)])
def test_layer_full_size_k_sweep_correlated_rows(K, regime):
    # from 8 rows the automatic regime runs the grouped kernels; the
    # verify-width kernels are also checked at those widths.  The down
    # kernel's staged h (K*8 + K rows of 2304 bytes) picks its shape by size:
    # 3 rows (62 KB) the largest 64 KB case, 4 rows (83 KB) the 96 KB case,
    # 5 rows (104 KB) the first 8-wave case, 16 rows three chunks
    x = inputs.gen_x_correlated(K, inputs.LAGUNA.hidden, 31 + K, device=DEV)
    gpu, _, _ = _layer_case(inputs.LAGUNA, K, 31 + K, x=x, label="ksweep", regime=regime)
    assert int(gpu["n_unique"][0]) <= K * 8


def test_layer_sigmoid_bias_scale_and_residual():
    # the pages' live router form: sigmoid + selection bias, renormalised,
    # routed scale 2.5, decoder residual fused into the combine
    _layer_case(inputs.LAGUNA, 2, 17, score_fn=1, rs=2.5, residual=True, label="sigmoid")


def _scaled_x(K, H, seed, scale):
    g = torch.Generator().manual_seed(seed)
    return inputs.bf16_bits(torch.randn(K, H, generator=g) * scale)


def range_cases(H):
    """Activation rows far outside fp16's range: magnitudes around 1e15
    (beyond 65504), around 1e-10 and 1e-7 (below fp16's normal range 2^-14,
    the first below its smallest subnormal), and rows mixing a few large
    entries with ordinary ones, or one ordinary entry with tiny ones."""
    big = _scaled_x(2, H, 1, 1e15)
    tiny = _scaled_x(2, H, 2, 1e-10)
    small = _scaled_x(2, H, 3, 1e-7)
    mixed = _scaled_x(3, H, 4, 1.0).view(torch.int16)
    f = inputs.bf16_bits(torch.tensor([3e5, -2.5e5, 1e5, -7e4])).view(torch.int16)
    mixed[0, :4] = f
    mixed[1] = _scaled_x(1, H, 5, 1e-7)[0]
    mixed[1, 7] = inputs.bf16_bits(torch.tensor([1.0]))[0]
    return [("big", big), ("tiny", tiny), ("small", small), ("mixed", mixed.contiguous())]


@pytest.mark.parametrize("case", ["big", "tiny", "small", "mixed"])
def test_layer_activation_range_beyond_fp16(case):
    # the gate/up matrix cores take x as fp16 under a per-row power-of-two
    # scale: rows of any bf16 magnitude match the oracle
    H = inputs.LAGUNA.hidden
    x = dict(range_cases(H))[case].to(DEV)
    gpu, orec, rep = _layer_case(inputs.LAGUNA, x.shape[0], 19, x=x, label="range-" + case,
                                 regime=api.MOE_REGIME_VERIFY)
    assert np.isfinite(gpu["y32"]).all()
    # and each row at the bar of its own largest output (rows of very
    # different magnitude share the layer)
    err = np.abs(gpu["y32"].astype(np.float64) - orec["y"]).max(axis=1)
    assert np.all(err <= 2e-3 * np.abs(orec["y"]).max(axis=1)), err / np.abs(orec["y"]).max(axis=1)


def test_layer_other_shapes():
    for shape, K in [(inputs.MoEShape(512, 64, 4, 256, 256), 3), (inputs.MoEShape(1024, 32, 8, 128, 0), 2),
                     (inputs.MoEShape(2048, 128, 8, 1024, 2048), 2)]:
        _layer_case(shape, K, 3, label=str(shape))


# ---------------------------------------------------------------------------
# invariants on the GPU (bitwise)
# ---------------------------------------------------------------------------


def _run_y32(cfg, wd, x):
    K, H = x.shape
    y = torch.empty(K, H, dtype=torch.int16, device=DEV)
    y32 = torch.empty(K, H, dtype=torch.float32, device=DEV)
    ws = api.alloc_workspace(cfg, DEV)
    api.moe_verify_layer(cfg, api.make_weights(wd), x, y, ws, y32=y32)
    torch.cuda.synchronize()
    return y32.cpu().numpy()


def test_invariants_identical_rows_permutation_rerun():
    say("case: invariants")
    shape = inputs.LAGUNA
    w = inputs.gen_layer(shape, 23, 0, device=DEV)
    cfg = api.make_cfg(shape, 8, regime=api.MOE_REGIME_VERIFY)  # the grouped kernels: test_gpu_grouped
    x1 = inputs.gen_x(1, shape.hidden, 23, device=DEV)
    yi = _run_y32(cfg, w, x1.repeat(8, 1).contiguous())
    for r in range(1, 8):
        assert np.array_equal(yi[0], yi[r])
    x = inputs.gen_x(6, shape.hidden, 24, device=DEV)
    y = _run_y32(cfg, w, x)
    perm = [4, 2, 5, 0, 3, 1]
    yp = _run_y32(cfg, w, x[perm].contiguous())
    assert np.array_equal(yp, y[perm])
    assert np.array_equal(_run_y32(cfg, w, x), y)
    # a single row alone gives the same bits as inside a batch
    assert np.array_equal(_run_y32(cfg, w, x[2:3].contiguous())[0], y[2])


def test_invariant_down_tensor_scale_doubles_routed_output():
    say("case: ts doubling")
    shape = inputs.MoEShape(2048, 256, 8, 512, 0)
    w = inputs.gen_layer(shape, 29, 0, device=DEV)
    cfg = api.make_cfg(shape, 2)
    x = inputs.gen_x(2, shape.hidden, 29, device=DEV)
    y = _run_y32(cfg, w, x)
    w2 = dict(w)
    w2["down"] = dict(w["down"])
    w2["down"]["ts"] = (w["down"]["ts"] * 2).contiguous()
    assert np.array_equal(_run_y32(cfg, w2, x), 2 * y)


def test_expert_relabelling_gives_same_output():
    say("case: relabel")
    shape = inputs.MoEShape(2048, 64, 8, 512, 512)
    w = inputs.gen_layer(shape, 37, 0, device=DEV)
    cfg = api.make_cfg(shape, 2)
    x = inputs.gen_x(2, shape.hidden, 37, device=DEV)
    y = _run_y32(cfg, w, x)
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(1)).to(DEV)
    wp = dict(w)
    wp["router_w"] = w["router_w"][perm].contiguous()
    for name in ("gate", "up", "down"):
        wp[name] = {kk: v[perm].contiguous() for kk, v in w[name].items()}
    yp = _run_y32(cfg, wp, x)
    np.testing.assert_allclose(yp, y, rtol=0, atol=2e-3 * np.abs(y).max())
