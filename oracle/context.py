"""The drafter's context lifecycle, as the pages keep it — TEST INFRASTRUCTURE ONLY.

Bookkeeping of the docs.rs page "cortiq_engine/dflash.rs" (cortiq-engine
0.8.78), written from its items `queue_context`, `settle`, `push_context`,
`settle_rows` (its closing window drop), `truncate`, `next_position`,
`span`, the `Ctx::dropped` field and the per-layer range of `Drafter::block`
(a layer's first held position is first + dropped). The keys and values
themselves come from the C oracle (`Model.settle`); this module only keeps
which rows exist.

Constants are the page's: at most PENDING_ROWS rows wait; past that the
oldest go through in multiples of CONTEXT_CHUNK. The page's device arm lets
as many rows wait as the widest window plus BLOCK_SLACK when every layer is
windowed; the library is a device arm, so that limit is taken here too.
"""
from __future__ import annotations

import numpy as np

PENDING_ROWS = 512
CONTEXT_CHUNK = 64
BLOCK_SLACK = 256


def pending_limit(windows) -> int:
    if windows and all(w > 0 for w in windows):
        return max(PENDING_ROWS, max(windows) + BLOCK_SLACK)
    return PENDING_ROWS


class Context:
    """first, len, per-layer dropped rows and held K/V, pending tap rows."""

    def __init__(self, model, drop: bool = True):
        self.m = model
        g = model.g
        self.g = g
        self.kd = g["kv_heads"] * g["head_dim"]
        self.tw = g["n_taps"] * g["hidden"]
        self.L = g["layers"]
        self.windows = list(g["windows"])
        self.drop = drop  # False keeps every row (a reference without the window drop)
        self.first = 0
        self.len = 0
        self.dropped = [0] * self.L
        self.k = [np.zeros((0, self.kd), np.float32) for _ in range(self.L)]
        self.v = [np.zeros((0, self.kd), np.float32) for _ in range(self.L)]
        self.pending = np.zeros((0, self.tw), np.float32)
        self.settled_calls = []  # (position, rows) of each settle_rows, for tests

    # -- positions --------------------------------------------------------------
    def next_position(self) -> int:
        return self.first + self.len + self.pending.shape[0]

    def span(self):
        return self.first, self.next_position()

    # -- `truncate` ---------------------------------------------------------------
    def truncate(self, pos: int):
        held = self.first + self.len
        self.pending = self.pending[:max(pos - held, 0)]
        keep = min(max(pos - self.first, 0), self.len)
        for l in range(self.L):
            rows = max(keep - self.dropped[l], 0)
            self.k[l] = self.k[l][:rows]
            self.v[l] = self.v[l][:rows]
            self.dropped[l] = min(self.dropped[l], keep)
        self.len = keep

    # -- `queue_context`, `settle`, `push_context` ---------------------------------
    def queue(self, pos: int, taps: np.ndarray):
        taps = np.asarray(taps, np.float32).reshape(-1, self.tw)
        if pos > self.next_position() or pos < self.first:
            self.truncate(0)
            self.first = pos
        else:
            self.truncate(pos)
        self.pending = np.concatenate([self.pending, taps])
        held = self.pending.shape[0]
        limit = pending_limit(self.windows)
        if held > limit:
            over = min(-(-(held - limit) // CONTEXT_CHUNK) * CONTEXT_CHUNK, held)
            rows, self.pending = self.pending[:over], self.pending[over:]
            self.settle_rows(self.first + self.len, rows)

    def settle(self):
        if self.pending.shape[0]:
            rows, self.pending = self.pending, self.pending[:0]
            self.settle_rows(self.first + self.len, rows)

    def push(self, pos: int, taps: np.ndarray):
        self.queue(pos, taps)
        self.settle()

    # -- `settle_rows` ---------------------------------------------------------------
    def settle_rows(self, pos: int, taps: np.ndarray):
        n = taps.shape[0]
        self.settled_calls.append((pos, n))
        K, V = self.m.settle(taps, pos)
        for l in range(self.L):
            self.k[l] = np.concatenate([self.k[l], K[l]])
            self.v[l] = np.concatenate([self.v[l], V[l]])
        self.len += n
        if not self.drop:
            return
        # no row of a layer sees further back than its window: once a layer
        # holds more than twice its window, it keeps the last window's rows
        for l in range(self.L):
            w = self.windows[l]
            held = self.len - self.dropped[l]
            if w > 0 and held > 2 * w:
                cut = held - w
                self.k[l] = self.k[l][cut:]
                self.v[l] = self.v[l][cut:]
                self.dropped[l] += cut

    # -- `Drafter::block` on the held rows ---------------------------------------------
    def block(self, anchor: int, a: int, k: int, width: int, **kw):
        assert self.pending.shape[0] == 0, "rows wait to become context (settle first)"
        store = [(self.k[l], self.v[l]) for l in range(self.L)]
        return self.m.block(store, self.first, self.len, anchor, a, k, width,
                            dropped=list(self.dropped), **kw)
