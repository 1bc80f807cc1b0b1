"""Plain model of the sliding-window KV cache of the verify step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg use it; the HIP path never does, and the two
share no code.

Sources (web pages): mlxfast-challenge-dev PR #844, "Validate submission
a02330a7 ...", section 8 items 1-2 and section 10 ("Next step"): at K >= 2
rows the sliding layers rebuild their cached keys and values by
concatenation on every step, and once the rotating cache has wrapped it
reports itself untrimmable, so a rejecting round replays a whole target
forward; the proposed fix is a cache that takes multi-row writes in place
and can drop the rejected rows.  mlxfast README, "Why this challenge
exists": sliding-window attention layers with a 512-token window, GQA with
8 KV heads of head_dim 128.

The definition kept here is the plain one: the cache is the sequence's full
history of (key, value) rows, one per position, in temporal order.
 * write(rows): a verify step appends its K rows (positions len .. len+K-1);
   row 0 is the last emitted token, rows 1.. are the draft tokens.
 * commit(n_accepted): the step keeps row 0 and the n_accepted accepted
   drafts; the rejected drafts' rows are dropped (len += 1 + n_accepted).
 * window(p): what attention at position p sees of one layer: the rows of
   positions max(0, p - W + 1) .. p, oldest first.
Data movement only: every value is copied bit for bit.
"""
from __future__ import annotations

from typing import List

import numpy as np


class KVHistory:
    """One sequence's keys and values for n_layers layers of n_kv heads of
    head_dim (any dtype; rows are copied unchanged)."""

    def __init__(self, n_layers: int, n_kv: int, head_dim: int, window: int):
        self.n_layers, self.n_kv, self.head_dim, self.W = n_layers, n_kv, head_dim, window
        self.k: List[List[np.ndarray]] = [[] for _ in range(n_layers)]  # [layer][position] -> [n_kv, head_dim]
        self.v: List[List[np.ndarray]] = [[] for _ in range(n_layers)]
        self.pending = 0  # rows of the last write not yet committed

    @property
    def length(self) -> int:
        """Positions held (committed plus the last write's pending rows)."""
        return len(self.k[0])

    def write(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """k_new, v_new: [n_layers, K, n_kv, head_dim], the rows of positions
        length .. length + K - 1."""
        if self.pending:
            raise RuntimeError("the previous write has not been committed")
        L, K = k_new.shape[:2]
        assert L == self.n_layers and v_new.shape == k_new.shape
        for l in range(L):
            for r in range(K):
                self.k[l].append(np.array(k_new[l, r]))
                self.v[l].append(np.array(v_new[l, r]))
        self.pending = K

    def commit(self, n_accepted: int) -> None:
        """Keep row 0 and the first n_accepted drafts of the last write;
        drop the rest."""
        K = self.pending
        if not 0 <= n_accepted <= K - 1:
            raise ValueError("n_accepted %d outside [0, %d]" % (n_accepted, K - 1))
        drop = K - 1 - n_accepted
        for l in range(self.n_layers):
            if drop:
                del self.k[l][-drop:]
                del self.v[l][-drop:]
        self.pending = 0

    def window(self, layer: int, p: int):
        """Keys and values that attention at position p sees in `layer`:
        positions max(0, p - W + 1) .. p, oldest first, as
        [n_positions, n_kv, head_dim] arrays."""
        lo = max(0, p - self.W + 1)
        ks = self.k[layer][lo:p + 1]
        vs = self.v[layer][lo:p + 1]
        return np.stack(ks), np.stack(vs)


def copy_bytes_concat(n_layers: int, n_kv: int, head_dim: int, window: int, K: int, elem: int = 2) -> int:
    """Bytes a concatenating cache moves per verify step for n_layers sliding
    layers: it rebuilds a (window + K - 1)-position key and value buffer
    (read the kept rows and the new ones, write all of them).  PR #844
    section 2 lists this as about 0.126 GB per step on the target (30
    sliding layers, 8 KV heads of 128, window 512, K = 2)."""
    rows = window + K - 1
    per_layer = 2 * (2 * rows * n_kv * head_dim * elem)  # keys and values, each read once and written once
    return n_layers * per_layer


def copy_bytes_in_place(n_layers: int, n_kv: int, head_dim: int, K: int, elem: int = 2) -> int:
    """Bytes an in-place ring write moves per verify step: the K new rows of
    keys and values, read once and written once."""
    return n_layers * 2 * (2 * K * n_kv * head_dim * elem)
