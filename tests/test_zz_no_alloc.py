"""The allocation-free entry point (moe_verify_layer_noalloc) against the
workspace entry point (moe_verify_layer) it shares its kernels with: bitwise
equal outputs, on two calls in a row (the second with fewer rows, so the
scratch array holds the first call's contents when the second starts), in
both kernel regimes."""
import numpy as np
import pytest
import torch

from speculative_block_verify_amd import api, inputs
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _both(cfg, wts, x, residual=None):
    K, H = x.shape
    outs = []
    for noalloc in (False, True):
        y = torch.full((K, H), -1, dtype=torch.int16, device=DEV)
        y32 = torch.full((K, H), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.full((K * cfg.top_k,), -1, dtype=torch.int32, device=DEV)
        dbg = api.make_debug(ids=ids)
        if noalloc:
            api.moe_verify_layer_noalloc(cfg, wts, x, y, y32=y32, residual=residual, debug=dbg)
        else:
            ws = api.alloc_workspace(cfg, DEV)
            api.moe_verify_layer(cfg, wts, x, y, ws, y32=y32, residual=residual, debug=dbg)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), y32.cpu().numpy(), ids.cpu().numpy()))
    (ya, y32a, ia), (yb, y32b, ib) = outs
    assert np.isfinite(y32a).all()
    np.testing.assert_array_equal(y32b, y32a)
    np.testing.assert_array_equal(yb, ya)
    np.testing.assert_array_equal(ib, ia)


@pytest.mark.parametrize("regime,K1,K2", [(api.MOE_REGIME_VERIFY, 4, 2), (api.MOE_REGIME_GROUPED, 24, 17)])
def test_noalloc_matches_workspace_entry_on_two_calls(regime, K1, K2):
    say("case: noalloc regime=%d K=%d then K=%d" % (regime, K1, K2))
    shape = inputs.LAGUNA
    w = inputs.gen_layer(shape, 91, 0, device=DEV)
    cfg = api.make_cfg(shape, K1, regime=regime)
    assert api.moe_verify_workspace_bytes(cfg) <= api.moe_verify_noalloc_scratch_bytes()
    wts = api.make_weights(w, cfg)
    x1 = inputs.gen_x(K1, shape.hidden, 91, device=DEV)
    _both(cfg, wts, x1)
    x2 = inputs.gen_x(K2, shape.hidden, 92, device=DEV)
    res = inputs.gen_x(K2, shape.hidden, 93, device=DEV, tag="res")
    _both(cfg, wts, x2, residual=res)


def test_noalloc_rejects_a_cfg_beyond_its_scratch():
    shape = inputs.LAGUNA
    cfg = api.make_cfg(shape, 64)
    assert api.moe_verify_workspace_bytes(cfg) > api.moe_verify_noalloc_scratch_bytes()
    w = inputs.gen_layer(inputs.TINY, 1, 0, device=DEV)
    x = inputs.gen_x(2, shape.hidden, 1, device=DEV)
    y = torch.empty(2, shape.hidden, dtype=torch.int16, device=DEV)
    with pytest.raises(api.MoEError) as e:
        api.moe_verify_layer_noalloc(cfg, api.make_weights(w), x, y)
    assert e.value.code == api.MOE_ERR_UNSUPPORTED and "scratch" in str(e.value)
