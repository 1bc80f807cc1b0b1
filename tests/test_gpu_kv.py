"""GPU parity of the verify step's sliding-window KV ring (moe_kv_ring_*)
against the plain history model (oracle/kv_oracle.py): after every block's
write, what each row of the block sees of every layer must equal the
history's window bit for bit; the commit must drop exactly the rejected
rows.  Sequences run long enough to wrap the ring many times."""
import numpy as np
import pytest
import torch

from oracle import kv_oracle
from speculative_block_verify_amd import api, inputs
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _expected_window(hist, layer, p, W):
    """The history's window at position p, zero rows before position 0, as
    [W, n_kv, D] arrays (the ring's output layout per row, heads first)."""
    ks, vs = hist.window(layer, p)
    pad = W - ks.shape[0]
    if pad:
        z = np.zeros((pad,) + ks.shape[1:], ks.dtype)
        ks, vs = np.concatenate([z, ks]), np.concatenate([z, vs])
    return ks, vs


def _check_block(ring, hist, K, layers, label):
    length = hist.length - K  # the block's first position
    for l in layers:
        ko, vo = ring.window_of(l, K)
        ko = ko.cpu().numpy().view(np.uint16)
        vo = vo.cpu().numpy().view(np.uint16)
        for r in range(K):
            ek, ev = _expected_window(hist, l, length + r, ring.window)
            # ring output [K, n_kv, W, D]; history [W, n_kv, D]
            np.testing.assert_array_equal(ko[r], ek.transpose(1, 0, 2), err_msg="%s layer %d row %d keys" % (label, l, r))
            np.testing.assert_array_equal(vo[r], ev.transpose(1, 0, 2), err_msg="%s layer %d row %d values" % (label, l, r))


def _run(L, n_kv, D, W, max_rows, steps, seed, k_choices, check_every=1, check_layers=None, label=""):
    say("case: kv ring %s L=%d n_kv=%d D=%d W=%d max_rows=%d steps=%d" % (label, L, n_kv, D, W, max_rows, steps))
    rng = np.random.default_rng(seed)
    ring = api.KvRing(L, n_kv, D, W, max_rows, DEV)
    ring.reset(0)
    hist = kv_oracle.KVHistory(L, n_kv, D, W)
    nacc = torch.zeros(1, dtype=torch.int32, device=DEV)
    layers = range(L) if check_layers is None else check_layers
    for s in range(steps):
        K = int(rng.choice(k_choices))
        k = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        ring.write(torch.as_tensor(k.view(np.int16)).to(DEV), torch.as_tensor(v.view(np.int16)).to(DEV))
        hist.write(k, v)
        if s % check_every == 0 or s == steps - 1:
            _check_block(ring, hist, K, layers, "%s step %d" % (label, s))
        a = int(rng.integers(0, K))
        nacc.fill_(a)
        ring.commit(nacc, K)
        hist.commit(a)
    torch.cuda.synchronize()
    assert int(ring.len.item()) == hist.length
    say("  %d positions through a ring of %d slots" % (hist.length, ring.shape[2]))
    return ring, hist


@pytest.mark.parametrize("max_rows,k_choices", [(1, [1]), (2, [1, 2]), (4, [1, 2, 3, 4]), (16, [1, 5, 16])])
def test_ring_matches_history_small(max_rows, k_choices):
    _run(3, 2, 16, 8, max_rows, 80, 10 + max_rows, k_choices, label="small")


def test_ring_matches_history_at_the_target_shape():
    """30 sliding layers of 8 KV heads of head_dim 128, window 512, blocks
    of 2 rows: 600 steps wrap the 513-slot ring about twice."""
    _run(30, 8, 128, 512, 2, 600, 7, [2], check_every=97, check_layers=[0, 13, 29], label="target")


def test_layer_by_layer_writes_as_a_forward_makes_them():
    """A forward writes each sliding layer's rows just before that layer's
    attention reads its window: per step, layer l is written and its window
    checked while the later layers still hold the previous step's state."""
    L, n_kv, D, W, K = 4, 2, 32, 16, 3
    say("case: kv ring per-layer writes L=%d n_kv=%d D=%d W=%d K=%d" % (L, n_kv, D, W, K))
    rng = np.random.default_rng(9)
    ring = api.KvRing(L, n_kv, D, W, K, DEV)
    ring.reset(0)
    hist = kv_oracle.KVHistory(L, n_kv, D, W)
    nacc = torch.zeros(1, dtype=torch.int32, device=DEV)
    for s in range(40):
        k = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        hist.write(k, v)
        for l in range(L):
            ring.write_layer(l, torch.as_tensor(k[l].view(np.int16)).to(DEV), torch.as_tensor(v[l].view(np.int16)).to(DEV))
            _check_block(ring, hist, K, [l], "per-layer step %d" % s)
        a = int(rng.integers(0, K))
        nacc.fill_(a)
        ring.commit(nacc, K)
        hist.commit(a)
    torch.cuda.synchronize()
    assert int(ring.len.item()) == hist.length


def test_commit_reads_the_greedy_steps_acceptance():
    """The ring's commit takes n_accepted straight from the lm_head greedy
    step's output on the device (no host round trip)."""
    K, V, H = 4, 999, 256
    x = inputs.gen_x(K, H, 3, device=DEV)
    w = inputs.gen_lm_head(V, H, 3, device=DEV)
    out = api.alloc_greedy_out(K, DEV)
    ws = torch.empty(api.moe_verify_lm_head_workspace_bytes(V, K), dtype=torch.uint8, device=DEV)
    ring = api.KvRing(2, 1, 8, 4, K, DEV)
    ring.reset(10)
    kn = torch.zeros(2, K, 1, 8, dtype=torch.int16, device=DEV)
    for draft_from_target in (True, False):
        api.moe_verify_lm_head_greedy(x, w, out, ws, draft=torch.zeros(K - 1, dtype=torch.int32, device=DEV))
        if draft_from_target:  # accept everything: drafts equal the greedy tokens
            api.moe_verify_lm_head_greedy(x, w, out, ws, draft=out["target"][:K - 1].clone())
        before = int(ring.len.item())
        ring.write(kn, kn)
        ring.commit(out["n_accepted"], K)
        torch.cuda.synchronize()
        a = int(out["n_accepted"].item())
        assert int(ring.len.item()) == before + 1 + a
        if draft_from_target:
            assert a == K - 1


def test_a_step_replays_in_a_graph():
    """A block's write and commit captured once in a graph and replayed
    with new rows and acceptance counts each time (eager work between the
    replays), against the history model."""
    L, n_kv, D, W, K = 2, 2, 16, 8, 3
    rng = np.random.default_rng(5)
    ring = api.KvRing(L, n_kv, D, W, K, DEV)
    ring.reset(0)
    hist = kv_oracle.KVHistory(L, n_kv, D, W)
    kbuf = torch.zeros(L, K, n_kv, D, dtype=torch.int16, device=DEV)
    vbuf = torch.zeros_like(kbuf)
    nacc = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ring.write(kbuf, vbuf)
            ring.commit(nacc, K)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(12):
        k = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, (L, K, n_kv, D), dtype=np.uint16)
        a = int(rng.integers(0, K))
        kbuf.copy_(torch.as_tensor(k.view(np.int16)))
        vbuf.copy_(torch.as_tensor(v.view(np.int16)))
        nacc.fill_(a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hist.write(k, v)
        hist.commit(a)
        assert int(ring.len.item()) == hist.length, "replay %d" % rep
        # what the next block's rows would see of the committed positions
        length = hist.length
        ko, vo = ring.window_of(0, 1)
        ek, ev = _expected_window(hist, 0, length - 1, W)
        # window_of(K=1) shows position len + 0, not yet written: compare the
        # W - 1 committed positions before it
        np.testing.assert_array_equal(ko.cpu().numpy().view(np.uint16)[0][:, :-1],
                                      ek.transpose(1, 0, 2)[:, 1:], err_msg="replay %d" % rep)
        np.testing.assert_array_equal(vo.cpu().numpy().view(np.uint16)[0][:, :-1],
                                      ev.transpose(1, 0, 2)[:, 1:], err_msg="replay %d" % rep)


def test_commit_clamps_the_acceptance_count():
    """A count outside [0, K - 1] read on the device is clamped: a negative
    one keeps row 0 only, one of K or more keeps the whole block."""
    say("case: kv ring commit clamp")
    K = 3
    ring = api.KvRing(1, 1, 8, 4, K, DEV)
    ring.reset(5)
    kn = torch.zeros(1, K, 1, 8, dtype=torch.int16, device=DEV)
    nacc = torch.zeros(1, dtype=torch.int32, device=DEV)
    expect = 5
    for a, kept in ((-7, 1), (99, K), (K - 1, K), (0, 1), (K, K)):
        ring.write(kn, kn)
        nacc.fill_(a)
        ring.commit(nacc, K)
        expect += kept
        torch.cuda.synchronize()
        assert int(ring.len.item()) == expect, (a, kept)
