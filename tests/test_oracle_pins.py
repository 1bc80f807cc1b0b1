"""Pins of the CPU oracle against things other than itself.

Each test names what it pins: a library decode routine, a table from a
specification, a page's printed number, brute force on a tiny case, a
closed form or an invariant.  None of these tests needs a GPU.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle as orc
from speculative_block_verify_amd import inputs
from tests import refdecode as ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    orc.build(force=False)


# ---------------------------------------------------------------------------
# O-1 decode
# ---------------------------------------------------------------------------


def test_e2m1_matches_ocp_table():
    tab = ref.e2m1_table()
    got = np.array([orc.e2m1(c) for c in range(16)])
    np.testing.assert_array_equal(got, tab)
    assert np.signbit(got[8]) and not np.signbit(got[0])
    assert orc.e2m1(7) == 6.0 and orc.e2m1(1) == 0.5


def test_e4m3fn_matches_torch_float8_for_all_256_codes():
    tab = ref.e4m3_table()
    got = np.array([orc.e4m3fn(b) for b in range(256)])
    nan = np.isnan(tab)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], tab[~nan])
    # OCP E4M3FN anchors: max normal 448, min normal 2^-6, min subnormal 2^-9, one.
    assert orc.e4m3fn(0x7E) == 448.0
    assert orc.e4m3fn(0x08) == 2.0 ** -6
    assert orc.e4m3fn(0x01) == 2.0 ** -9
    assert orc.e4m3fn(0x38) == 1.0


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32)
    want = ref.bf16_to_f64(bits.astype(np.uint16))
    lib = orc.lib()
    got = np.array([lib.orc_bf16(int(b)) for b in bits[::7]])
    w = want[::7]
    nan = np.isnan(w)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], w[~nan])


def test_f32_to_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
        # exact halfway cases: low 16 bits = 0x8000 with even and odd kept lsb
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, np.inf, -np.inf], np.float32),
    ])
    want = ref.f32_to_bf16_bits(vals)
    got = np.array([orc.f32_to_bf16(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_dequant_matches_independent_numpy_decode():
    m = inputs.gen_nvfp4(3, 32, 64, "cpu", 7, "pin-deq")
    for e in range(3):
        np.testing.assert_array_equal(orc.dequant(m, e), ref.dequant(m, e))


def test_dequant_round_trips_generator_within_quantisation_step():
    """The generator encodes fp32 weights with torch ops; the oracle decodes
    them with its own C tables.  A swapped nibble, a scale applied to the
    wrong block or a sign slip would break this bound."""
    g = torch.Generator().manual_seed(3)
    w = torch.randn((2, 16, 128), generator=g) * 0.02
    q, s, ts = inputs.quantize_nvfp4(w)
    m = {"q": q, "s": s, "ts": ts}
    for e in range(2):
        deq = orc.dequant(m, e)
        W = w[e].double().numpy()
        step = np.repeat(ref.e4m3_table()[s[e].numpy()], 16, axis=1) * float(ts[e])
        # half the widest E2M1 gap (4 -> 6) is 1.0 step; e4m3 rounding of the
        # scale adds at most 1/16 relative
        assert np.all(np.abs(deq - W) <= 1.0 * step * (1 + 1 / 16) + 1e-12)
        assert np.corrcoef(deq.ravel(), W.ravel())[0, 1] > 0.99


# ---------------------------------------------------------------------------
# O-2 router
# ---------------------------------------------------------------------------


def test_router_matches_float64_matmul():
    x = inputs.gen_x(3, 256, 11)
    wr = inputs.bf16_bits(torch.randn(40, 256, generator=torch.Generator().manual_seed(2)) * 0.02)
    got = orc.router(x, wr)
    want = (ref.bf16_to_f64(x.numpy()) @ ref.bf16_to_f64(wr.numpy()).T).astype(np.float32)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-12)


# ---------------------------------------------------------------------------
# O-3 / O-4 / O-5 selection and weights
# ---------------------------------------------------------------------------


def _brute_topk(keys: np.ndarray, k: int) -> np.ndarray:
    out = []
    for row in keys:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, np.int32)


@pytest.mark.parametrize("E,k", [(16, 2), (256, 8), (64, 64), (7, 1)])
def test_topk_softmax_matches_brute_force_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    l = rng.standard_normal((5, E)).astype(np.float32)
    ids, w = orc.topk(l, k)
    np.testing.assert_array_equal(ids, _brute_topk(l, k))
    # weights: full softmax over all E, restricted to the selection and
    # renormalised (scipy)
    full = softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


def test_topk_ties_go_to_lower_index_and_zero_input_gives_uniform():
    l = np.zeros((2, 16), np.float32)
    ids, w = orc.topk(l, 4)
    np.testing.assert_array_equal(ids, [[0, 1, 2, 3]] * 2)
    assert np.all(w == 0.25)
    l = np.array([[1, 5, 5, 2, 5, 0, 5, 5]], np.float32)
    ids, _ = orc.topk(l, 3)
    np.testing.assert_array_equal(ids, [[1, 2, 4]])
    # -0.0 and +0.0 compare equal: index decides
    l = np.array([[0.0, -0.0, 0.0, -1.0]], np.float32)
    ids, _ = orc.topk(l, 2)
    np.testing.assert_array_equal(ids, [[0, 1]])


def test_topk_k_equals_E_is_the_dense_softmax():
    rng = np.random.default_rng(9)
    l = rng.standard_normal((3, 12)).astype(np.float32)
    ids, w = orc.topk(l, 12)
    dense = softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(dense, ids.astype(np.int64), axis=1), w, rtol=1e-12)


def test_sigmoid_scoring_zero_bias_selects_like_logits_and_bias_forces_selection():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((4, 32)).astype(np.float32)
    zero = np.zeros(32, np.float32)
    ids_s, w_s = orc.topk(l, 4, orc.SCORE_SIGMOID_BIAS, 1, zero)
    ids_l, _ = orc.topk(l, 4)
    # sigmoid is monotone: same experts unless two logits collide after the
    # fp32 sigmoid; with these values they do not
    np.testing.assert_array_equal(ids_s, ids_l)
    sig = expit(np.take_along_axis(l.astype(np.float64), ids_s.astype(np.int64), axis=1))
    np.testing.assert_allclose(w_s, sig / sig.sum(1, keepdims=True), rtol=1e-12)
    # un-normalised weights are the raw sigmoids
    _, w_raw = orc.topk(l, 4, orc.SCORE_SIGMOID_BIAS, 0, zero)
    np.testing.assert_allclose(w_raw, sig, rtol=1e-12)
    # a large bias on one expert puts it first but leaves its weight unbiased
    bias = zero.copy(); bias[17] = 10.0
    ids_b, w_b = orc.topk(l, 4, orc.SCORE_SIGMOID_BIAS, 0, bias)
    assert np.all(ids_b[:, 0] == 17)
    np.testing.assert_allclose(w_b[:, 0], expit(l[:, 17].astype(np.float64)), rtol=1e-12)


# ---------------------------------------------------------------------------
# O-6 dedup
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(5))
def test_dedup_matches_dictionary_brute_force(seed):
    rng = np.random.default_rng(seed)
    K, k, E = rng.integers(1, 17), 8, 32
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(K)]).astype(np.int32)
    d = orc.dedup(ids, E)
    flat = ids.reshape(-1)
    groups = {}
    for slot, e in enumerate(flat):
        groups.setdefault(int(e), []).append(slot)
    uniq = sorted(groups)
    assert d["n_unique"] == len(uniq)
    np.testing.assert_array_equal(d["uniq"], uniq)
    asg = [s for e in uniq for s in groups[e]]
    np.testing.assert_array_equal(d["asg"], asg)
    np.testing.assert_array_equal(d["off"], np.cumsum([0] + [len(groups[e]) for e in uniq]))
    # inverse map and coverage
    assert sorted(d["asg"].tolist()) == list(range(flat.size))
    for slot in range(flat.size):
        assert d["asg"][d["inv"][slot]] == slot
    assert d["off"][-1] == K * k


# ---------------------------------------------------------------------------
# O-7 / O-8 expert FFN and layer
# ---------------------------------------------------------------------------

SMALL = inputs.MoEShape(hidden=64, n_experts=8, top_k=2, inter=32, shared_inter=32)


def _dense_deq(w, shape):
    E = shape.n_experts
    G = np.stack([ref.dequant(w["gate"], e) for e in range(E)])
    U = np.stack([ref.dequant(w["up"], e) for e in range(E)])
    D = np.stack([ref.dequant(w["down"], e) for e in range(E)])
    return G, U, D


def test_expert_ffn_matches_numpy_swiglu():
    w = inputs.gen_layer(SMALL, 5)
    x = inputs.gen_x(1, SMALL.hidden, 5)
    G, U, D = _dense_deq(w, SMALL)
    x64 = ref.bf16_to_f64(x.numpy())[0]
    for e in range(SMALL.n_experts):
        got = orc.expert_ffn(x, w["gate"], w["up"], w["down"], e)
        np.testing.assert_allclose(got, ref.swiglu_ffn(x64, G[e], U[e], D[e]), rtol=1e-10, atol=1e-14)


def _brute_dense_layer(w, shape, x, rs=1.0, residual=None, k=None):
    """Every expert on every row, multiplied by a 0/1 selection mask built
    by brute-force sorting and weighted by the full softmax restricted to the
    selection."""
    k = k or shape.top_k
    G, U, D = _dense_deq(w, shape)
    x64 = ref.bf16_to_f64(x.numpy())
    logits = (x64 @ ref.bf16_to_f64(w["router_w"].numpy()).T).astype(np.float32)
    ids = _brute_topk(logits, k)
    mask = np.zeros_like(logits, dtype=np.float64)
    np.put_along_axis(mask, ids.astype(np.int64), 1.0, axis=1)
    p = softmax(logits.astype(np.float64), axis=1) * mask
    p /= p.sum(1, keepdims=True)
    y = np.zeros_like(x64)
    for e in range(shape.n_experts):
        y += p[:, e:e + 1] * ref.swiglu_ffn(x64, G[e], U[e], D[e])
    y *= rs
    if shape.shared_inter:
        y += ref.swiglu_ffn(x64, ref.dequant(w["sh_gate"], 0), ref.dequant(w["sh_up"], 0),
                            ref.dequant(w["sh_down"], 0))
    if residual is not None:
        y += ref.bf16_to_f64(residual.numpy())
    return y, logits, ids


@pytest.mark.parametrize("rs", [1.0, 2.5])
def test_layer_matches_brute_force_dense_masked_evaluation(rs):
    w = inputs.gen_layer(SMALL, 21)
    x = inputs.gen_x(3, SMALL.hidden, 21)
    res = inputs.gen_x(3, SMALL.hidden, 22, tag="res")
    out = orc.moe_layer(w, x, SMALL.top_k, routed_scale=rs, residual=res)
    want, logits, ids = _brute_dense_layer(w, SMALL, x, rs=rs, residual=res)
    np.testing.assert_array_equal(out["ids"], ids)
    np.testing.assert_allclose(out["logits"], logits, rtol=2e-7)
    np.testing.assert_allclose(out["y"], want, rtol=1e-9, atol=1e-12 * np.abs(want).max())


def test_tiny_config_matches_brute_force():
    """The tiny layer: hidden 256, 16 experts, top-2, intermediate 128, no
    shared expert, one row."""
    w = inputs.gen_layer(inputs.TINY, 0)
    x = inputs.gen_x(1, 256, 0)
    out = orc.moe_layer(w, x, 2)
    want, _, ids = _brute_dense_layer(w, inputs.TINY, x)
    np.testing.assert_array_equal(out["ids"], ids)
    np.testing.assert_allclose(out["y"], want, rtol=1e-9, atol=1e-12 * np.abs(want).max())


def test_k_equals_E_layer_is_dense_softmax_moe():
    shape = inputs.MoEShape(hidden=64, n_experts=4, top_k=4, inter=32, shared_inter=0)
    w = inputs.gen_layer(shape, 8)
    x = inputs.gen_x(2, 64, 8)
    out = orc.moe_layer(w, x, 4)
    G, U, D = _dense_deq(w, shape)
    x64 = ref.bf16_to_f64(x.numpy())
    p = softmax((x64 @ ref.bf16_to_f64(w["router_w"].numpy()).T).astype(np.float32).astype(np.float64), axis=1)
    want = sum(p[:, e:e + 1] * ref.swiglu_ffn(x64, G[e], U[e], D[e]) for e in range(4))
    np.testing.assert_allclose(out["y"], want, rtol=1e-9, atol=1e-13)


def test_single_expert_layer_is_textbook_swiglu_mlp():
    shape = inputs.MoEShape(hidden=64, n_experts=1, top_k=1, inter=32, shared_inter=0)
    w = inputs.gen_layer(shape, 13)
    x = inputs.gen_x(4, 64, 13)
    out = orc.moe_layer(w, x, 1)
    assert np.all(out["w"] == 1.0)
    x64 = ref.bf16_to_f64(x.numpy())
    want = ref.swiglu_ffn(x64, ref.dequant(w["gate"], 0), ref.dequant(w["up"], 0), ref.dequant(w["down"], 0))
    np.testing.assert_allclose(out["y"], want, rtol=1e-10, atol=1e-14)


def test_identical_rows_give_identical_outputs_and_weights_sum_to_one():
    w = inputs.gen_layer(SMALL, 31)
    x1 = inputs.gen_x(1, SMALL.hidden, 31)
    x = x1.repeat(3, 1)
    out = orc.moe_layer(w, x, SMALL.top_k)
    assert np.array_equal(out["y"][0], out["y"][1]) and np.array_equal(out["y"][0], out["y"][2])
    np.testing.assert_allclose(out["w"].sum(1), 1.0, rtol=1e-14)


def test_sigmoid_mode_layer_matches_brute_force():
    w = inputs.gen_layer(SMALL, 41, with_bias=True)
    x = inputs.gen_x(2, SMALL.hidden, 41)
    out = orc.moe_layer(w, x, SMALL.top_k, orc.SCORE_SIGMOID_BIAS, 1, 2.5)
    G, U, D = _dense_deq(w, SMALL)
    x64 = ref.bf16_to_f64(x.numpy())
    logits = (x64 @ ref.bf16_to_f64(w["router_w"].numpy()).T).astype(np.float32)
    bias = w["router_bias"].numpy()
    keys = expit(logits.astype(np.float64)).astype(np.float32) + bias
    ids = _brute_topk(keys, SMALL.top_k)
    np.testing.assert_array_equal(out["ids"], ids)
    sig = expit(np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1))
    wts = sig / sig.sum(1, keepdims=True)
    want = np.zeros_like(x64)
    for r in range(2):
        for j in range(SMALL.top_k):
            e = ids[r, j]
            want[r] += wts[r, j] * ref.swiglu_ffn(x64[r], G[e], U[e], D[e])
    want *= 2.5
    want += ref.swiglu_ffn(x64, ref.dequant(w["sh_gate"], 0), ref.dequant(w["sh_up"], 0), ref.dequant(w["sh_down"], 0))
    np.testing.assert_allclose(out["y"], want, rtol=1e-9, atol=1e-12 * np.abs(want).max())


# ---------------------------------------------------------------------------
# O-9 RMSNorm glue
# ---------------------------------------------------------------------------


def test_rmsnorm_output_has_unit_rms_and_is_scale_invariant():
    rng = np.random.default_rng(0)
    y = rng.standard_normal((3, 512)) * 7.0
    x = orc.rmsnorm_bf16(y, 1e-6)
    xv = ref.bf16_to_f64(x)
    rms = np.sqrt((xv ** 2).mean(1))
    np.testing.assert_allclose(rms, 1.0, atol=2 ** -8)
    # with eps = 0 a power-of-two rescale of y leaves the bf16 output unchanged
    np.testing.assert_array_equal(orc.rmsnorm_bf16(y, 0.0), orc.rmsnorm_bf16(y * 4.0, 0.0))
    # constant rows normalise to exactly one
    c = np.full((1, 64), 3.0)
    assert np.all(ref.bf16_to_f64(orc.rmsnorm_bf16(c, 0.0)) == 1.0)


def test_rmsnorm_gamma_scales_the_normalised_row():
    """RMSNorm with a weight: x = gamma * y / rms(y).  Pins: dividing the
    output by gamma restores unit RMS (so gamma neither enters the norm nor
    lands on another column), gamma = ones equals no gamma, and a
    power-of-two gamma scales the bf16 output exactly."""
    rng = np.random.default_rng(3)
    H = 256
    y = rng.standard_normal((3, H)) * 5.0
    gv = rng.uniform(0.5, 2.0, H)
    gamma = ref.f32_to_bf16_bits(gv)
    x = ref.bf16_to_f64(orc.rmsnorm_bf16(y, 1e-6, gamma))
    ratio = x / ref.bf16_to_f64(gamma)[None, :]
    np.testing.assert_allclose(np.sqrt((ratio ** 2).mean(1)), 1.0, atol=2 ** -8)
    # column by column: each output is its own column's gamma times the plain norm
    plain = ref.bf16_to_f64(orc.rmsnorm_bf16(y, 1e-6))
    np.testing.assert_allclose(ratio, plain, rtol=2 ** -7)
    ones = ref.f32_to_bf16_bits(np.ones(H))
    np.testing.assert_array_equal(orc.rmsnorm_bf16(y, 1e-6, ones), orc.rmsnorm_bf16(y, 1e-6))
    twos = ref.f32_to_bf16_bits(np.full(H, 2.0))
    np.testing.assert_array_equal(ref.bf16_to_f64(orc.rmsnorm_bf16(y, 1e-6, twos)), 2.0 * plain)


def test_stack_feeds_normalised_output_forward():
    layers = inputs.gen_stack(SMALL, 3, 55)
    x = inputs.gen_x(2, SMALL.hidden, 55)
    recs = orc.moe_stack(layers, x, SMALL.top_k)
    for l in range(1, 3):
        np.testing.assert_array_equal(recs[l]["x_in"], orc.rmsnorm_bf16(recs[l - 1]["y"]))
        assert recs[l]["res_in"] is None
    np.testing.assert_array_equal(recs[0]["x_in"], x.numpy().view(np.uint16))


def _silent(layer):
    """A copy of a layer whose down projections (routed and shared) have
    tensor scale 0: every expert FFN then outputs exactly zero."""
    w = dict(layer)
    for m in ("down", "sh_down"):
        if w.get(m) is not None:
            w[m] = dict(w[m], ts=torch.zeros_like(w[m]["ts"]))
    return w


def test_stack_residual_stream_passes_through_silent_layers():
    """Residual stream (the decoder residual of PR #844 section 4 item 4):
    with every FFN output zero, each layer's output is exactly its residual
    input, so the stream carries the initial residual unchanged; after a
    live layer 0, a silent layer 1 outputs layer 0's bf16 output (not the
    initial residual); without a residual, silent layers output zero."""
    layers = inputs.gen_stack(SMALL, 3, 56)
    x = inputs.gen_x(2, SMALL.hidden, 56)
    res = inputs.gen_x(2, SMALL.hidden, 57, tag="res")
    r64 = ref.bf16_to_f64(res.numpy())
    recs = orc.moe_stack([_silent(w) for w in layers], x, SMALL.top_k, residual=res)
    for l in range(3):
        np.testing.assert_array_equal(recs[l]["y"], r64)
        np.testing.assert_array_equal(recs[l]["res_in"], res.numpy().view(np.uint16))
    recs = orc.moe_stack([layers[0], _silent(layers[1])], x, SMALL.top_k, residual=res)
    y0 = recs[0]["y"]
    assert np.abs(y0 - r64).max() > 1e-3          # layer 0 adds its FFN output
    np.testing.assert_array_equal(recs[1]["y"], ref.bf16_to_f64(ref.f32_to_bf16_bits(y0.astype(np.float32))))
    recs = orc.moe_stack([_silent(w) for w in layers], x, SMALL.top_k)
    for l in range(3):
        assert np.all(recs[l]["y"] == 0.0)


def test_stack_uses_each_layers_norm_weight():
    """Layer l's norm weight scales the input of layer l + 1 only."""
    layers = inputs.gen_stack(SMALL, 3, 58)
    rng = np.random.default_rng(58)
    for w in layers:
        w["norm_w"] = torch.as_tensor(ref.f32_to_bf16_bits(rng.uniform(0.5, 2.0, SMALL.hidden)).astype(np.int16))
    x = inputs.gen_x(2, SMALL.hidden, 58)
    recs = orc.moe_stack(layers, x, SMALL.top_k)
    for l in range(1, 3):
        g = ref.bf16_to_f64(layers[l - 1]["norm_w"].numpy())
        ratio = ref.bf16_to_f64(recs[l]["x_in"]) / g[None, :]
        plain = ref.bf16_to_f64(orc.rmsnorm_bf16(recs[l - 1]["y"]))
        np.testing.assert_allclose(ratio, plain, rtol=2 ** -7, atol=1e-30)


# ---------------------------------------------------------------------------
# Byte layout pinned to the pages' numbers
# ---------------------------------------------------------------------------


def test_byte_layout_reproduces_page_numbers():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_budget.json")))
    H, I, L = 2048, 512, g["moe_layers"]
    mat = orc.nvfp4_matrix_bytes(I, H, tensor_scale=False)
    assert mat == orc.nvfp4_matrix_bytes(H, I, tensor_scale=False) == 589_824
    # two rows x top-8 x 3 projections per layer, no dedup, 39 MoE layers
    k2 = L * 2 * 8 * 3 * mat
    assert k2 == 1_104_150_528 and round(k2 / 1e9, 2) == g["routed_bytes_per_step_k2_approx_GB"]
    k1 = L * 1 * 8 * 3 * mat
    assert k1 == 552_075_264 and round(k1 / 1e9, 2) == g["routed_bytes_per_step_k1_approx_GB"]
    tiles = g["expert_tiles_per_layer_k2"] * mat
    assert round(tiles / 1e6, 1) == g["tiles_bytes_per_layer_one_projection_approx_MB"]
    # fused [gate; up] bank duplicates the 4-bit values of every routed expert
    values = I * H // 2
    assert L * 256 * 2 * values / 2 ** 30 == g["fused_gate_up_bank_duplicate_approx_GiB"]
    assert L * 2 * values / 2 ** 20 == g["shared_gate_up_bank_approx_MiB"]
    assert round(g["vocab"] * H * 2 / 1e9, 2) == g["lm_head_approx_GB"]


def test_layer_step_bytes_at_two_rows():
    # 16 unique experts + shared + router + x/y at K = 2
    b = orc.layer_step_bytes(2048, 256, 512, 512, 16, 2)
    assert b == 17 * (3 * 589_824 + 12) + 2 * 256 * 2048 + 4 * 2 * 2048


# ---------------------------------------------------------------------------
# Verify-row lm_head and greedy acceptance
# ---------------------------------------------------------------------------


# ---------------------------------------------------------------------------
# the dense first layer and the prefill stack (README "Why this challenge
# exists": layer 0 is a dense SwiGLU MLP)
# ---------------------------------------------------------------------------


def test_dense_mlp_matches_numpy_swiglu_with_residual():
    w = inputs.gen_dense(64, 96, 71)
    x = inputs.gen_x(3, 64, 71)
    res = inputs.gen_x(3, 64, 72, tag="res")
    got = orc.dense_mlp(w, x, residual=res)["y"]
    dec = lambda t: ref.bf16_to_f64(t.numpy())  # noqa: E731
    want = ref.swiglu_ffn(dec(x), dec(w["gate"]), dec(w["up"]), dec(w["down"])) + dec(res)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(orc.dense_mlp(w, x)["y"], want - dec(res), rtol=1e-10, atol=1e-13)


def test_dense_mlp_closed_forms():
    """One intermediate unit: y[t][n] = down[n] * silu(g_t) * u_t; zero up
    weights: y is the residual exactly; doubled down weights: y doubles."""
    H = 32
    w = inputs.gen_dense(H, 1, 73)
    x = inputs.gen_x(2, H, 73)
    dec = lambda t: ref.bf16_to_f64(np.asarray(t))  # noqa: E731
    x64 = dec(x.numpy())
    g = x64 @ dec(w["gate"].numpy())[0]
    u = x64 @ dec(w["up"].numpy())[0]
    want = (g / (1.0 + np.exp(-g)) * u)[:, None] * dec(w["down"].numpy())[:, 0][None, :]
    np.testing.assert_allclose(orc.dense_mlp(w, x)["y"], want, rtol=1e-12, atol=1e-15)
    w = inputs.gen_dense(H, 40, 74)
    res = inputs.gen_x(2, H, 75, tag="res")
    zero_up = dict(w, up=torch.zeros_like(w["up"]))
    np.testing.assert_array_equal(orc.dense_mlp(zero_up, x, residual=res)["y"], dec(res.numpy()))
    two = ref.f32_to_bf16_bits(2.0 * ref.bf16_to_f64(w["down"].numpy()))
    doubled = dict(w, down=torch.as_tensor(two.astype(np.int16)))
    np.testing.assert_array_equal(orc.dense_mlp(doubled, x)["y"], 2.0 * orc.dense_mlp(w, x)["y"])


def test_dense_moe_stack_glue():
    """The dense layer's record equals dense_mlp on the stack input; the
    first MoE layer consumes bf16(gamma_0 * RMSNorm(y_0)) and, with a
    residual stream, the residual bf16(y_0)."""
    H = SMALL.hidden
    dense = inputs.gen_dense(H, 64, 76)
    rng = np.random.default_rng(76)
    dense["norm_w"] = torch.as_tensor(ref.f32_to_bf16_bits(rng.uniform(0.5, 2.0, H)).astype(np.int16))
    layers = inputs.gen_stack(SMALL, 2, 77)
    x = inputs.gen_x(2, H, 78)
    res = inputs.gen_x(2, H, 79, tag="res")
    recs = orc.dense_moe_stack(dense, layers, x, SMALL.top_k, residual=res)
    assert len(recs) == 3
    np.testing.assert_array_equal(recs[0]["y"], orc.dense_mlp(dense, x, residual=res)["y"])
    np.testing.assert_array_equal(recs[1]["x_in"], orc.rmsnorm_bf16(recs[0]["y"], 1e-6, dense["norm_w"]))
    np.testing.assert_array_equal(recs[1]["res_in"], ref.f32_to_bf16_bits(recs[0]["y"].astype(np.float32)))
    np.testing.assert_array_equal(recs[2]["x_in"], orc.rmsnorm_bf16(recs[1]["y"], 1e-6, layers[0].get("norm_w")))
    assert len(orc.dense_moe_stack(dense, [], x, SMALL.top_k)) == 1


def test_lm_head_matches_float64_matmul():
    rng = np.random.default_rng(21)
    K, V, H = 3, 301, 256
    x = ref.f32_to_bf16_bits(rng.standard_normal((K, H)))
    w = ref.f32_to_bf16_bits(rng.standard_normal((V, H)) * 0.02)
    got = orc.lm_head(x, w)
    want = ref.bf16_to_f64(x) @ ref.bf16_to_f64(w).T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_greedy_target_is_first_maximum_like_numpy_argmax():
    rng = np.random.default_rng(22)
    l = np.round(rng.standard_normal((6, 500)) * 4) / 4      # many exact ties
    l[2] = 0.0                                               # all tied -> token 0
    out = orc.greedy_accept(l, np.zeros(5, np.int32))
    np.testing.assert_array_equal(out["target"], np.argmax(l, axis=1))
    assert out["target"][2] == 0


def _block(K, V, tgt, margin=1.0):
    l = np.zeros((K, V))
    for r, t in enumerate(tgt):
        l[r, t] = margin
    return l


def test_greedy_acceptance_longest_prefix_and_bonus_token():
    V = 50
    tgt = [7, 11, 13, 17]
    l = _block(4, V, tgt)
    # all three drafts match the previous rows' greedy tokens: 3 accepted + bonus
    o = orc.greedy_accept(l, [7, 11, 13])
    assert o["accepted"] == 3 and list(o["emitted"]) == [7, 11, 13, 17]
    # first draft rejected: the target's own token at row 0 only
    o = orc.greedy_accept(l, [8, 11, 13])
    assert o["accepted"] == 0 and list(o["emitted"]) == [7]
    # a later match after a mismatch does not count (prefix)
    o = orc.greedy_accept(l, [7, 12, 13])
    assert o["accepted"] == 1 and list(o["emitted"]) == [7, 11]
    # one row: no draft, the greedy token
    o = orc.greedy_accept(l[:1], [])
    assert o["accepted"] == 0 and list(o["emitted"]) == [7]


def test_greedy_acceptance_true_ties_within_the_pages_tolerance():
    """A draft token whose logit is within 1e-6 of the row's top logit is a
    true tie and is accepted; 2e-6 below is not; with tolerance 0 only exact
    ties count."""
    V = 20
    l = _block(2, V, [4, 9])
    l[0, 5] = 1.0 - 0.5e-6
    o = orc.greedy_accept(l, [5], tie_tol=1e-6)
    assert o["target"][0] == 4 and o["accepted"] == 1 and list(o["emitted"]) == [5, 9]
    assert orc.greedy_accept(l, [5], tie_tol=0.0)["accepted"] == 0
    l[0, 5] = 1.0 - 2e-6
    assert orc.greedy_accept(l, [5], tie_tol=1e-6)["accepted"] == 0
    l[0, 5] = 1.0                                  # exact tie, higher id: not the argmax, still a true tie
    o = orc.greedy_accept(l, [5], tie_tol=0.0)
    assert o["target"][0] == 4 and o["accepted"] == 1


def test_lm_head_bytes_reproduce_the_page_number():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_budget.json")))
    b = orc.lm_head_bytes(g["vocab"], 2048, 0)
    assert b == 411_041_792 and round(b / 1e9, 2) == g["lm_head_approx_GB"]
