"""Pins of the sliding-window KV cache model (oracle/kv_oracle.py) against
what the definition and the pages fix: a rollback leaves exactly the
history of a sequence that wrote only the kept rows; a window holds the
last W positions in order and slides by one per position; the
concatenating cache's copy traffic reproduces the page's 0.126 GB per step
(PR #844 section 2; tests/golden/page_byte_budget.json).

The checks are functions of the module, so test_oracle_kv_mutations.py can
run them against planted mistakes."""
import json
import os

import numpy as np
import pytest

from oracle import kv_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_byte_budget.json")


def _rows(rng, L, K, H=2, D=4):
    k = rng.integers(0, 1 << 16, (L, K, H, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (L, K, H, D), dtype=np.uint16)
    return k, v


def check_rollback_equals_writing_only_kept_rows(kv, seed=0):
    rng = np.random.default_rng(seed)
    L, W = 3, 7
    a = kv.KVHistory(L, 2, 4, W)
    b = kv.KVHistory(L, 2, 4, W)
    for step in range(40):
        K = int(rng.integers(1, 5))
        k, v = _rows(rng, L, K)
        n_acc = int(rng.integers(0, K))
        a.write(k, v)
        a.commit(n_acc)
        keep = 1 + n_acc
        b.write(k[:, :keep], v[:, :keep])
        b.commit(keep - 1)
        assert a.length == b.length
        for l in range(L):
            for p in range(a.length):
                ka, va = a.window(l, p)
                kb, vb = b.window(l, p)
                np.testing.assert_array_equal(ka, kb)
                np.testing.assert_array_equal(va, vb)


def check_window_is_the_last_W_positions(kv, seed=1):
    rng = np.random.default_rng(seed)
    L, W = 2, 5
    h = kv.KVHistory(L, 2, 4, W)
    written = []  # every kept row of layer 1, in order
    for step in range(12):
        K = int(rng.integers(1, 4))
        k, v = _rows(rng, L, K)
        n_acc = int(rng.integers(0, K))
        h.write(k, v)
        # before the commit the window of the block's row r ends at that row
        for r in range(K):
            p = len(written) + r
            ks, _ = h.window(1, p)
            assert ks.shape[0] == min(p + 1, W)
            np.testing.assert_array_equal(ks[-1], k[1, r])
        h.commit(n_acc)
        written += [k[1, r] for r in range(1 + n_acc)]
    for p in range(len(written)):
        ks, _ = h.window(1, p)
        want = np.stack(written[max(0, p - W + 1):p + 1])
        np.testing.assert_array_equal(ks, want)
        if p >= W:
            prev, _ = h.window(1, p - 1)
            np.testing.assert_array_equal(ks[:-1], prev[1:])


def check_commit_bounds(kv):
    h = kv.KVHistory(1, 1, 2, 4)
    k = np.zeros((1, 3, 1, 2), np.uint16)
    h.write(k, k)
    with pytest.raises(RuntimeError):
        h.write(k, k)
    for bad in (-1, 3):
        with pytest.raises(ValueError):
            h.commit(bad)
    h.commit(2)
    assert h.length == 3


def check_page_copy_traffic(kv):
    g = json.load(open(GOLDEN))
    got = kv.copy_bytes_concat(g["sliding_layers"], g["kv_heads"], g["head_dim"], g["sliding_window"], 2)
    assert round(got / 1e9, 3) == g["sliding_cache_concat_approx_GB"]
    # the rebuilt buffer's length at K = 2 (section 8 item 1): one head of
    # one element, keys and values each read and written once
    assert kv.copy_bytes_concat(1, 1, 1, g["sliding_window"], 2, elem=1) == 2 * 2 * g["sliding_cache_rebuild_positions_k2"]
    # an in-place write moves the two new rows only
    assert kv.copy_bytes_in_place(30, 8, 128, 2) == 30 * 2 * 2 * 2 * 8 * 128 * 2


CHECKS = [check_rollback_equals_writing_only_kept_rows, check_window_is_the_last_W_positions, check_commit_bounds,
          check_page_copy_traffic]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_kv_oracle(check):
    check(kv_oracle)
