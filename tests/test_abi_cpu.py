"""The C ABI library loads, exports every entry point the header declares,
and rejects bad arguments on the host before any GPU work (no GPU needed)."""
import ctypes
import os
import re

import pytest

from speculative_block_verify_amd import api, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:MOE_API\s+)?(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return api.lib()


def test_header_declares_the_expected_surface():
    names = _declared_functions()
    assert set(names) == set(api.EXPORTS), names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert api.moe_verify_version() == 210


def test_struct_layouts_match_header_sizes():
    # pointer-only structs: 3 / 2 + 6*3 + 1 / 7 / 12 pointers; cfg: 11 x 4 bytes
    P = ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(api.moe_nvfp4) == 3 * P
    assert ctypes.sizeof(api.moe_layer_weights) == 21 * P
    assert ctypes.sizeof(api.moe_route_out) == 7 * P
    assert ctypes.sizeof(api.moe_debug) == 12 * P
    assert ctypes.sizeof(api.moe_dense_weights) == 4 * P
    assert ctypes.sizeof(api.moe_cfg) == 44


def _cfg(**kw):
    c = api.make_cfg(inputs.LAGUNA, 2)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes_valid_and_invalid():
    n = api.moe_verify_workspace_bytes(_cfg())
    assert n > 0 and n % 256 == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(hidden=300))) == 0
    assert "hidden" in api.moe_verify_last_error()
    # up to 1024 rows; above 16 the grouped (prefill) limits apply too
    assert api.moe_verify_workspace_bytes(_cfg(max_rows=512)) > n
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(max_rows=1025))) == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(max_rows=17, inter=2048))) == 0
    assert "grouped" in api.moe_verify_last_error()
    assert api.moe_verify_workspace_bytes(_cfg(max_rows=16, inter=2048)) > 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(top_k=300))) == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(inter=500))) == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(score_fn=7))) == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(norm_topk=0))) == 0
    assert api.lib().moe_verify_workspace_bytes(ctypes.byref(_cfg(regime=4))) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _weights(shared=True, bias=False):
    m = api.moe_nvfp4(FAKE, FAKE, FAKE)
    z = api.moe_nvfp4(None, None, None)
    return api.moe_layer_weights(FAKE, FAKE if bias else None, m, m, m,
                                 m if shared else z, m if shared else z, m if shared else z)


def _layer(cfg, w, K=2, x=FAKE, y=FAKE, ws=FAKE, ws_bytes=None, residual=None):
    if ws_bytes is None:
        ws_bytes = api.lib().moe_verify_workspace_bytes(ctypes.byref(cfg)) or 1 << 30
    return api.lib().moe_verify_layer(ctypes.byref(cfg), ctypes.byref(w), x, K, residual, y, None, ws,
                                      ws_bytes, None, None)


@pytest.mark.parametrize("case,code", [
    ("K0", api.MOE_ERR_INVALID), ("K_over", api.MOE_ERR_INVALID), ("x_null", api.MOE_ERR_INVALID),
    ("y_misaligned", api.MOE_ERR_INVALID), ("ws_small", api.MOE_ERR_WORKSPACE),
    ("ws_null", api.MOE_ERR_INVALID), ("bias_with_softmax", api.MOE_ERR_INVALID),
    ("sigmoid_without_bias", api.MOE_ERR_INVALID), ("shared_missing", api.MOE_ERR_INVALID),
    ("shared_unexpected", api.MOE_ERR_INVALID), ("hidden_unsupported", api.MOE_ERR_UNSUPPORTED),
    ("gate_null", api.MOE_ERR_INVALID), ("router_misaligned", api.MOE_ERR_INVALID),
])
def test_layer_argument_errors(case, code):
    cfg, w, kw = _cfg(), _weights(), {}
    if case == "K0": kw["K"] = 0
    elif case == "K_over": kw["K"] = 3
    elif case == "x_null": kw["x"] = None
    elif case == "y_misaligned": kw["y"] = FAKE + 2
    elif case == "ws_small": kw["ws_bytes"] = 1024
    elif case == "ws_null": kw["ws"] = None
    elif case == "bias_with_softmax": w = _weights(bias=True)
    elif case == "sigmoid_without_bias": cfg = _cfg(score_fn=1)
    elif case == "shared_missing": w = _weights(shared=False)
    elif case == "shared_unexpected": cfg = _cfg(shared_inter=0)
    elif case == "hidden_unsupported": cfg = _cfg(hidden=4096)
    elif case == "gate_null": w.gate = api.moe_nvfp4(None, FAKE, FAKE)
    elif case == "router_misaligned": w.router_w = FAKE + 4
    assert _layer(cfg, w, **kw) == code
    assert api.moe_verify_last_error()


def test_grouped_layer_argument_errors():
    L = api.lib()
    cfg = _cfg(inter=2048)  # verify-width cfg; the grouped kernels stop at 1024
    n = L.moe_verify_workspace_bytes(ctypes.byref(cfg))
    rc = L.moe_verify_layer_grouped(ctypes.byref(cfg), ctypes.byref(_weights()), FAKE, 2, None, FAKE, None, FAKE,
                                    n, None, None)
    assert rc == api.MOE_ERR_UNSUPPORTED and "grouped" in api.moe_verify_last_error()
    cfg = _cfg(max_rows=64)
    n = L.moe_verify_workspace_bytes(ctypes.byref(cfg))
    rc = L.moe_verify_layer_grouped(ctypes.byref(cfg), ctypes.byref(_weights()), FAKE, 65, None, FAKE, None, FAKE,
                                    n, None, None)
    assert rc == api.MOE_ERR_INVALID
    # per-kernel timing is verify-width only
    arr = (api.moe_layer_weights * 1)(_weights())
    ms = (ctypes.c_float * 3)()
    rc = L.moe_verify_stack_timed(ctypes.byref(cfg), arr, 1, FAKE, None, 32, FAKE, None, FAKE, n, None, ms)
    assert rc == api.MOE_ERR_UNSUPPORTED
    # the grouped route needs the workspace
    out = api.moe_route_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    rc = L.moe_verify_route(ctypes.byref(cfg), FAKE, None, 32, ctypes.byref(out), None, 0, None)
    assert rc == api.MOE_ERR_INVALID and "workspace" in api.moe_verify_last_error()


def test_stack_and_route_argument_errors():
    cfg = _cfg()
    L = api.lib()
    arr = (api.moe_layer_weights * 2)(_weights(), _weights(shared=False))
    n = L.moe_verify_workspace_bytes(ctypes.byref(cfg))
    rc = L.moe_verify_stack(ctypes.byref(cfg), arr, 2, FAKE, None, 2, FAKE, None, FAKE, n, None, None)
    assert rc == api.MOE_ERR_INVALID and "layer 1" in api.moe_verify_last_error()
    rc = L.moe_verify_stack(ctypes.byref(cfg), arr, 0, FAKE, None, 2, FAKE, None, FAKE, n, None, None)
    assert rc == api.MOE_ERR_INVALID
    arr2 = (api.moe_layer_weights * 2)(_weights(), _weights())
    rc = L.moe_verify_stack(ctypes.byref(cfg), arr2, 2, FAKE, FAKE + 8, 2, FAKE, None, FAKE, n, None, None)
    assert rc == api.MOE_ERR_INVALID and "residual" in api.moe_verify_last_error()
    arr2[1].norm_w = FAKE + 2
    rc = L.moe_verify_stack(ctypes.byref(cfg), arr2, 2, FAKE, None, 2, FAKE, None, FAKE, n, None, None)
    assert rc == api.MOE_ERR_INVALID and "norm_w" in api.moe_verify_last_error()
    out = api.moe_route_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    rc = L.moe_verify_route(ctypes.byref(cfg), FAKE, None, 2, ctypes.byref(out), None, 0, None)
    assert rc == api.MOE_ERR_INVALID
    out.inv = FAKE
    rc = L.moe_verify_route(ctypes.byref(_cfg(score_fn=1)), FAKE, None, 2, ctypes.byref(out), None, 0, None)
    assert rc == api.MOE_ERR_INVALID and "bias" in api.moe_verify_last_error()
    m = api.moe_nvfp4(FAKE, FAKE, FAKE)
    assert L.moe_verify_dequant_nvfp4(ctypes.byref(m), 1, 4, 48, FAKE, None) == api.MOE_ERR_INVALID
    h = ctypes.c_void_p()
    rc = L.moe_stack_graph_create(ctypes.byref(cfg), arr, 2, FAKE, None, 2, FAKE, None, FAKE, n, None,
                                  ctypes.byref(h))
    assert rc == api.MOE_ERR_INVALID and not h.value
    assert L.moe_stack_graph_launch(None, None) == api.MOE_ERR_INVALID
    L.moe_stack_graph_destroy(None)


def test_weight_bytes_counts_unique_experts_once():
    cfg = _cfg()
    one = api.moe_verify_weight_bytes(cfg, 1, 2, with_shared=False, with_router=False) - 4 * 2 * 2048
    assert one == 3 * (512 * 2048 // 2 + 512 * 2048 // 16 + 4)
    full = api.moe_verify_weight_bytes(cfg, 16, 2)
    assert full == 17 * one + 2 * 256 * 2048 + 4 * 2 * 2048


def test_regime_argument_errors():
    # checked before any device work: the verify-width kernels serve at most
    # 16 rows; forcing the grouped kernels applies their shape limits at any K
    L = api.lib()
    cfg = _cfg(max_rows=17, regime=api.MOE_REGIME_VERIFY)
    n = L.moe_verify_workspace_bytes(ctypes.byref(cfg))
    assert n > 0
    assert _layer(cfg, _weights(), K=17, ws_bytes=n) == api.MOE_ERR_UNSUPPORTED
    assert "verify-width" in api.moe_verify_last_error()
    cfg = _cfg(max_rows=17, regime=api.MOE_REGIME_VERIFY_ONE_LAUNCH)
    assert _layer(cfg, _weights(), K=17, ws_bytes=L.moe_verify_workspace_bytes(ctypes.byref(cfg))) == \
        api.MOE_ERR_UNSUPPORTED
    assert "verify-width" in api.moe_verify_last_error()
    cfg = _cfg(inter=2048, regime=api.MOE_REGIME_GROUPED)
    n = L.moe_verify_workspace_bytes(ctypes.byref(cfg))
    assert n > 0
    assert _layer(cfg, _weights(), K=2, ws_bytes=n) == api.MOE_ERR_UNSUPPORTED
    assert "grouped" in api.moe_verify_last_error()


# ---------------------------------------------------------------------------
# The Python binding validates tensors before anything reaches the library
# (host tensors, wrong shapes, short buffers), so no host pointer or short
# buffer becomes a GPU access.  CPU tensors are enough to see every error.
# ---------------------------------------------------------------------------

import torch  # noqa: E402


def _host_layer(shape=inputs.TINY):
    return inputs.gen_layer(shape, 0, 0)


def test_binding_rejects_host_tensors_and_bad_shapes():
    shape = inputs.TINY
    cfg = api.make_cfg(shape, 2)
    w = _host_layer()
    x = inputs.gen_x(2, shape.hidden, 0)
    y = torch.empty(2, shape.hidden, dtype=torch.int16)
    ws = torch.empty(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.make_weights(w)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.check_weights(w, cfg)
    bad = dict(w, gate=dict(w["gate"], q=w["gate"]["q"][:, :, :-1]))
    with pytest.raises(ValueError, match="gate.q has shape"):
        api.check_weights(bad, cfg)
    with pytest.raises(ValueError, match="router_w must have shape"):
        api.check_weights(dict(w, router_w=w["router_w"][:, :-8]), cfg)
    wts = api.moe_layer_weights()
    with pytest.raises(ValueError, match=r"\[K, 256\]"):
        api.moe_verify_layer(cfg, wts, x[:, :128], y, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.moe_verify_layer(cfg, wts, x, y, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.moe_verify_stack(cfg, [wts], x, y, ws)
    with pytest.raises(ValueError, match="at least one layer"):
        api.moe_verify_stack(cfg, [], x, y, ws)
    with pytest.raises(TypeError, match="dtype"):
        api.moe_verify_layer(cfg, wts, x.float(), y, ws)
    out = {k: torch.empty(8, dtype=torch.int32) for k in ("ids", "w", "n_unique", "uniq", "off", "asg", "inv")}
    with pytest.raises(ValueError, match=r"\[K, 16\]"):
        api.moe_verify_route(cfg, torch.zeros(2, 8), out)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.moe_verify_route(cfg, torch.zeros(2, 16), out)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.moe_verify_dequant_nvfp4(w["gate"], torch.empty(16 * 128 * 256))


def test_binding_size_checks_use_k_and_hidden():
    # the size rules themselves, on the marshalling helper: a GPU-less
    # container cannot make GPU tensors, so the device check comes first
    cfg = api.make_cfg(inputs.TINY, 2)
    sizes = api._debug_sizes(cfg, 2)
    assert sizes["logits"] == 2 * 16 and sizes["off"] == 2 * 2 + 1 and sizes["x_in"] == 2 * 256
    assert sizes["res_in"] == sizes["y32"] == 2 * 256
    with pytest.raises(ValueError, match="unknown debug array"):
        api._check_debug(api.make_debug(bogus=torch.empty(1)), cfg, 2, 1, None)


def test_stream_read_argument_errors():
    L = api.lib()
    sink = FAKE
    assert L.moe_verify_stream_read(None, 16, sink, None) == api.MOE_ERR_INVALID
    assert L.moe_verify_stream_read(FAKE + 4, 16, sink, None) == api.MOE_ERR_INVALID
    assert L.moe_verify_stream_read(FAKE, 24, sink, None) == api.MOE_ERR_INVALID
    assert L.moe_verify_stream_read(FAKE, 0, sink, None) == api.MOE_ERR_INVALID
    assert L.moe_verify_stream_read(FAKE, 16, None, None) == api.MOE_ERR_INVALID


def test_noalloc_entry_rejects_a_cfg_beyond_its_scratch_before_device_work():
    L = api.lib()
    assert L.moe_verify_noalloc_scratch_bytes() == 5 << 20
    cfg = _cfg(max_rows=64)  # 7.6 MB of workspace at the full-size shape
    rc = L.moe_verify_layer_noalloc(ctypes.byref(cfg), ctypes.byref(_weights()), FAKE, 2, None, FAKE, None, None,
                                    None)
    assert rc == api.MOE_ERR_UNSUPPORTED and "scratch" in api.moe_verify_last_error()


def test_dense_and_prefill_argument_errors():
    """Checked before any device work: shapes, NULL or misaligned pointers,
    row counts, short workspaces."""
    L = api.lib()
    n = L.moe_dense_workspace_bytes(2048, 8192, 512)
    assert n > 0 and n % 256 == 0
    assert L.moe_dense_workspace_bytes(2048, 8192, 1024) > n
    for H, I, R in ((2048, 100, 512), (2048, 8192 + 64, 8), (100, 8192, 8), (4096, 8192, 8), (2048, 8192, 0)):
        assert L.moe_dense_workspace_bytes(H, I, R) == 0, (H, I, R)
    dw = api.moe_dense_weights(FAKE, FAKE, FAKE, None)

    def dense(x=FAKE, T=4, H=2048, I=8192, w=dw, res=None, eps=1e-6, y=FAKE, y32=FAKE, xn=None, ws=FAKE, nb=n):
        return L.moe_dense_mlp(x, T, H, I, None if w is None else ctypes.byref(w), res, eps, y, y32, xn, ws, nb, None)

    assert dense(T=0) == api.MOE_ERR_INVALID
    assert dense(I=300) == api.MOE_ERR_UNSUPPORTED
    assert dense(w=None) == api.MOE_ERR_INVALID
    assert dense(w=api.moe_dense_weights(FAKE, None, FAKE, None)) == api.MOE_ERR_INVALID
    assert dense(w=api.moe_dense_weights(FAKE, FAKE, FAKE, FAKE + 2)) == api.MOE_ERR_INVALID
    assert dense(y32=None) == api.MOE_ERR_INVALID
    assert dense(xn=FAKE + 8) == api.MOE_ERR_INVALID
    assert dense(eps=-1.0) == api.MOE_ERR_INVALID
    assert dense(ws=None) == api.MOE_ERR_INVALID
    assert dense(nb=L.moe_dense_workspace_bytes(2048, 8192, 4) - 256) == api.MOE_ERR_WORKSPACE

    cfg = _cfg(max_rows=512)
    pn = L.moe_prefill_workspace_bytes(ctypes.byref(cfg), 8192)
    assert pn > L.moe_verify_workspace_bytes(ctypes.byref(cfg)) + n
    assert L.moe_prefill_workspace_bytes(ctypes.byref(cfg), 100) == 0
    layers = (api.moe_layer_weights * 2)(_weights(), _weights())

    def pre(T=512, w=dw, I=8192, nl=2, nb=pn, x=FAKE, y=FAKE):
        return L.moe_prefill_stack(ctypes.byref(cfg), None if w is None else ctypes.byref(w), I, layers, nl, x, None,
                                   T, y, None, None, FAKE, nb, None, None)

    assert pre(T=0) == api.MOE_ERR_INVALID
    assert pre(T=513) == api.MOE_ERR_INVALID
    assert pre(I=100) == api.MOE_ERR_UNSUPPORTED
    assert pre(w=None) == api.MOE_ERR_INVALID
    assert pre(nl=0) == api.MOE_ERR_INVALID
    assert pre(x=None) == api.MOE_ERR_INVALID
    assert pre(nb=pn - 256) == api.MOE_ERR_WORKSPACE


def test_lm_head_argument_errors():
    L = api.lib()
    assert ctypes.sizeof(api.moe_greedy_out) == 5 * ctypes.sizeof(ctypes.c_void_p)
    n = L.moe_verify_lm_head_workspace_bytes(100352, 2)
    assert n > 0 and n % 256 == 0
    assert L.moe_verify_lm_head_workspace_bytes(100352, 17) == 0
    assert L.moe_verify_lm_head_workspace_bytes(0, 2) == 0
    out = api.moe_greedy_out(FAKE, FAKE, FAKE, FAKE, FAKE)

    def call(x=FAKE, K=2, w=FAKE, V=100352, H=2048, draft=FAKE, tol=1e-6, logits=None, o=out, ws=FAKE, nb=n):
        return L.moe_verify_lm_head_greedy(x, K, w, V, H, draft, tol, logits, ctypes.byref(o), ws, nb, None)

    assert call(K=0) == api.MOE_ERR_INVALID
    assert call(K=17) == api.MOE_ERR_INVALID
    assert call(H=3000) == api.MOE_ERR_UNSUPPORTED
    assert call(x=FAKE + 2) == api.MOE_ERR_INVALID
    assert call(draft=None) == api.MOE_ERR_INVALID and "draft" in api.moe_verify_last_error()
    assert call(tol=-1.0) == api.MOE_ERR_INVALID
    assert call(tol=float("nan")) == api.MOE_ERR_INVALID
    assert call(logits=FAKE + 4) == api.MOE_ERR_INVALID
    assert call(nb=n - 16) == api.MOE_ERR_WORKSPACE
    assert call(o=api.moe_greedy_out(FAKE, FAKE, None, FAKE, FAKE)) == api.MOE_ERR_INVALID


def test_kv_ring_argument_errors():
    """The ring's sizes and the checks made before any device work."""
    L = api.lib()
    P = ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(api.moe_kv_ring) == 3 * P + 5 * 4 + (4 if P == 8 else 0)
    assert L.moe_kv_ring_capacity(512, 2) == 513
    assert L.moe_kv_ring_capacity(512, 1) == 512
    assert L.moe_kv_ring_capacity(0, 2) == 0 and L.moe_kv_ring_capacity(512, 0) == 0
    # 30 sliding layers x 8 KV heads x 128 x 513 slots, bf16
    assert L.moe_kv_ring_bytes(30, 8, 128, 513) == 30 * 8 * 128 * 513 * 2
    assert L.moe_kv_ring_bytes(0, 8, 128, 513) == 0

    def ring(k=FAKE, v=FAKE, ln=FAKE, nl=30, nkv=8, D=128, W=512, C=513):
        return api.moe_kv_ring(k, v, ln, nl, nkv, D, W, C)

    def write(r=None, K=2, kn=FAKE, vn=FAKE):
        r = ring() if r is None else r
        return L.moe_kv_ring_write(ctypes.byref(r), kn, vn, K, None)

    assert L.moe_kv_ring_write(None, FAKE, FAKE, 2, None) == api.MOE_ERR_INVALID
    assert write(K=0) == api.MOE_ERR_INVALID
    assert write(K=3) == api.MOE_ERR_INVALID and "capacity" in api.moe_verify_last_error()
    assert write(r=ring(D=100)) == api.MOE_ERR_INVALID and "head_dim" in api.moe_verify_last_error()
    assert write(r=ring(D=0)) == api.MOE_ERR_INVALID
    assert write(r=ring(k=None)) == api.MOE_ERR_INVALID
    assert write(r=ring(v=FAKE + 8)) == api.MOE_ERR_INVALID
    assert write(r=ring(ln=None)) == api.MOE_ERR_INVALID
    assert write(r=ring(nl=0)) == api.MOE_ERR_INVALID
    assert write(r=ring(W=0)) == api.MOE_ERR_INVALID
    assert write(kn=None) == api.MOE_ERR_INVALID
    assert write(vn=FAKE + 2) == api.MOE_ERR_INVALID
    r = ring()
    assert L.moe_kv_ring_write_layer(ctypes.byref(r), 30, FAKE, FAKE, 2, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_write_layer(ctypes.byref(r), -1, FAKE, FAKE, 2, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_write_layer(ctypes.byref(r), 0, FAKE, None, 2, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_write_layer(ctypes.byref(r), 0, FAKE, FAKE, 3, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_commit(ctypes.byref(r), None, 2, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_commit(ctypes.byref(r), FAKE, 3, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_reset(ctypes.byref(r), -1, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_window(ctypes.byref(r), 30, 2, FAKE, FAKE, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_window(ctypes.byref(r), -1, 2, FAKE, FAKE, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_window(ctypes.byref(r), 0, 2, None, FAKE, None) == api.MOE_ERR_INVALID
    assert L.moe_kv_ring_window(ctypes.byref(r), 0, 2, FAKE, FAKE + 4, None) == api.MOE_ERR_INVALID
    with pytest.raises(api.MoEError):
        api.KvRing(30, 8, 128, 0, 2, "cpu")
