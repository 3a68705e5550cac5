"""The context lifecycle through the C-ABI against the oracle's context
(oracle/context.py): the same queue / flush / settle / truncate sequence on
both, the bookkeeping (first position, settled and waiting rows, each layer's
dropped rows) compared exactly after every step, the rows each layer holds
and blocks at the end and inside the context compared to the parity
tolerance. Covers the waiting rows' limit and ring, windowed layers' rings
(wrapping many times, attention ranges that cross the wrap), a full layer's
store growing with its rows kept, and the calls that must fail without
changing anything."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth
from oracle.context import Context, pending_limit

from test_gpu_parity import (check_selection, close, forced_select, held_store, run_block,
                             same_state)

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


class Pair:
    """One library handle and one oracle context, driven together."""

    def __init__(self, orc, g, w, max_context):
        self.g, self.w = g, w
        self.m = orc.Model(g, w)
        self.ctx = Context(self.m)
        self.d = pkg.Drafter(g, w, max_context=max_context,
                             stream=torch.cuda.current_stream(_dev()).cuda_stream)
        self.seed = 100

    def rows(self, n):
        self.seed += 1
        return synth.make_taps(self.g, n, seed=self.seed)

    def queue(self, pos, n):
        t = self.rows(n)
        self.d.queue(pos, n, t.to(_dev()).data_ptr())
        self.ctx.queue(pos, t.numpy())
        same_state(self.d, self.ctx)

    def settle(self, pos, n):
        t = self.rows(n)
        self.d.settle(pos, n, t.to(_dev()).data_ptr())
        self.ctx.push(pos, t.numpy())
        same_state(self.d, self.ctx)

    def flush(self):
        self.d.flush()
        self.ctx.settle()
        same_state(self.d, self.ctx)

    def truncate(self, pos):
        self.d.truncate(pos)
        self.ctx.truncate(pos)
        same_state(self.d, self.ctx)

    def check_rows(self, tag):
        got = held_store(self.d, self.g)
        for l in range(self.g["layers"]):
            assert got[l][0].shape == self.ctx.k[l].shape, (tag, l)
            if got[l][0].size:
                close(got[l][0], self.ctx.k[l], f"{tag} K layer {l}")
                close(got[l][1], self.ctx.v[l], f"{tag} V layer {l}")

    def check_block(self, a, tag, anchor=77, k=None, width=None):
        g = self.g
        k = k or g["block"] - 1
        width = width or g["vocab"]
        got = run_block(self.d, g, anchor, a, k, width)
        ref = self.ctx.block(anchor, a, k, width)
        close(got["hidden"], ref["hidden"], f"{tag} hidden")
        close(got["logits"], ref["logits"], f"{tag} logits")
        close(got["hp"], ref["hp"], f"{tag} hp")
        sel = self.m.select(ref["logits"], ref["hp"], anchor)
        check_selection(got, ref["logits"], sel, tag,
                        forced=forced_select(self.d, g, got, k, width, anchor))
        return got

    def close(self):
        self.d.close()


def test_queue_flush_truncate_sequence(orc):
    """Queue past the waiting limit (the oldest rows settle in 64-row
    multiples), truncate into the waiting rows, flush, rewind into settled
    rows, restart on a gap; a windowed layer drops rows all along."""
    g = synth.small_geometry(windows=[0, 6], no_rope=[1])
    w = synth.make_weights(g, seed=21)
    p = Pair(orc, g, w, max_context=4000)
    try:
        assert pending_limit(g["windows"]) == 512
        p.queue(30, 100)                      # waits
        p.queue(130, 500)                     # 600 wait: the oldest 128 settle
        assert p.ctx.len == 128
        p.check_rows("queued")
        with pytest.raises(pkg.DflashError) as e:  # rows wait: no block, nothing changes
            run_block(p.d, g, 5, 400, 3, 1000)
        assert e.value.code == pkg.DFLASH_EINVAL
        same_state(p.d, p.ctx)
        p.truncate(400)                       # cuts the waiting rows
        p.flush()
        p.check_rows("flushed")
        end = p.ctx.first + p.ctx.len
        p.check_block(end, "after flush")
        base = p.ctx.first + p.ctx.dropped[1]
        p.check_block(base + 5, "inside, within reach")
        p.check_block(base - 4, "inside, past the held rows")
        p.settle(380, 50)                     # rewind into settled rows
        p.queue(430, 5)
        p.flush()
        p.check_rows("rewound")
        p.check_block(435, "rewound")
        p.settle(500, 20)                     # gap: restart
        p.check_rows("restarted")
        p.check_block(520, "restarted")
        p.queue(505, 0)                       # n = 0 applies the rule only
        p.queue(515, 700)                     # one call past the limit from the caller's rows
        p.settle(600, 3)                      # rewind into the waiting rows, then settle all
        p.check_rows("rewound into waiting")
        p.check_block(603, "rewound into waiting")
    finally:
        p.close()


def test_all_windowed_limit_and_wrapping_rings(orc):
    """Every layer windowed: as many rows as the widest window plus 256 may
    wait. Rows come in odd pieces, so both rings wrap many times and the
    300-row window's attention range crosses the wrap."""
    g = synth.small_geometry(windows=[300, 7], no_rope=[0])
    w = synth.make_weights(g, seed=22)
    p = Pair(orc, g, w, max_context=100000)
    try:
        assert pending_limit(g["windows"]) == 556
        pos = 11
        p.settle(pos, 1)
        pos += 1
        for i, n in enumerate([37, 91, 5, 250, 37, 129, 64, 300, 41, 17]):
            if i % 3 == 2:
                p.queue(pos, n)
                p.queue(pos + n, 600)         # past the limit: 64-row multiples settle
                p.flush()
                pos += n + 600
            else:
                p.settle(pos, n)
                pos += n
        assert min(p.ctx.dropped) > 0
        p.check_rows("wrapped")
        p.check_block(pos, "wrapped end")
        base = p.ctx.first + p.ctx.dropped[0]
        p.check_block(base + 299, "window 300 just within reach")
        p.check_block(base + 100, "window 300 past the held rows")
    finally:
        p.close()


def test_full_layer_growth_keeps_rows(orc):
    """A full layer's store starts at 4096 rows and grows (twice its rows,
    at most max_context) keeping what it holds; reserve beyond max_context
    fails without a change."""
    g = synth.small_geometry(windows=[0, 0], no_rope=[])
    w = synth.make_weights(g, seed=23)
    p = Pair(orc, g, w, max_context=9000)
    try:
        p.settle(3, 4000)                     # 3520 then 480 rows: the store takes 4096
        p.settle(4003, 300)                   # grows to 8192, the 4000 rows copied over
        p.check_rows("grown")
        p.check_block(4303, "grown")
        with pytest.raises(pkg.DflashError) as e:
            p.d.reserve(9001)
        assert e.value.code == pkg.DFLASH_ENOMEM
        p.d.reserve(9000)                     # grows to max_context
        same_state(p.d, p.ctx)
        extra = p.rows(4701).to(_dev())
        with pytest.raises(pkg.DflashError) as e:  # 4300 + 4701 rows > 9000: no change
            p.d.settle(4303, 4701, extra.data_ptr())
        assert e.value.code == pkg.DFLASH_ENOMEM
        same_state(p.d, p.ctx)
        with pytest.raises(pkg.DflashError) as e:  # 4224 settle now, but the 477 left to wait
            p.d.queue(4303, 4701, extra.data_ptr())  # could not be settled later
        assert e.value.code == pkg.DFLASH_ENOMEM
        same_state(p.d, p.ctx)
        p.settle(4303, 4700)                  # exactly max_context rows
        p.check_block(9003, "full to max_context")
    finally:
        p.close()
