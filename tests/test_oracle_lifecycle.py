"""Pins of the oracle's context lifecycle (oracle/context.py) against what the
pages fix: the window drop (`settle_rows`: no row of a layer sees further
back than its window) leaves every block at the end of the context
bit-identical, and any block whose window still reaches the first held row;
the pending queue (`queue_context`: at most PENDING_ROWS wait, the oldest go
through in CONTEXT_CHUNK multiples) changes nothing a block sees; a rewind
(`truncate`) after a drop equals building the same rows afresh; the position
rule restarts the context on a gap."""
import numpy as np
import pytest

from block_drafter_settle_amd import synth


@pytest.fixture(scope="module")
def setup(orc):
    from oracle import context as C

    g = synth.small_geometry(windows=[0, 6], no_rope=[1], hidden=128, intermediate=256,
                             vocab=500, mask_token=499)
    w = synth.make_weights(g, seed=11)
    m = orc.Model(g, w)
    taps = synth.make_taps(g, 700, seed=12).numpy()
    return C, g, m, taps


def _same(x, y, what):
    for n in ("logits", "hp", "hidden"):
        assert np.array_equal(x[n], y[n]), (what, n)


def test_window_drop_leaves_block_at_end_bit_identical(setup):
    C, g, m, taps = setup
    ref = C.Context(m, drop=False)
    ref.push(30, taps[:200])
    outs = []
    # the same 200 rows in different pieces: one push; many small pushes;
    # queues past the pending limit, then a settle
    a = C.Context(m)
    a.push(30, taps[:200])
    b = C.Context(m)
    for i in range(0, 200, 7):
        b.push(30 + i, taps[i:min(i + 7, 200)])
    c = C.Context(m)
    c.queue(30, taps[:100])
    c.queue(130, taps[100:200])
    c.settle()
    for ctx in (a, b, c):
        assert ctx.span() == (30, 230)
        assert ctx.dropped[0] == 0 and ctx.dropped[1] > 0           # layer 1 dropped rows
        held = ctx.len - ctx.dropped[1]
        assert 6 <= held <= 12 and ctx.k[1].shape[0] == held        # between w and 2w held
        outs.append(ctx.block(5, 230, 5, 500))
    r = ref.block(5, 230, 5, 500)
    for i, o in enumerate(outs):
        _same(o, r, f"history {i}")


def test_anchor_inside_the_context(setup):
    C, g, m, taps = setup
    ref = C.Context(m, drop=False)
    ref.push(0, taps[:150])
    ctx = C.Context(m)
    ctx.push(0, taps[:150])
    base = ctx.first + ctx.dropped[1]
    w = g["windows"][1]
    # the window of block row 0 starts at a + 1 − w: at or past the first
    # held row, dropping changed nothing the block sees
    a_in = base + w - 1
    _same(ctx.block(9, a_in, 4, 500), ref.block(9, a_in, 4, 500), "within reach")
    # further back the layer sees only its held rows, fewer than without the
    # drop: the outputs move
    a_out = base - 3
    x, y = ctx.block(9, a_out, 4, 500), ref.block(9, a_out, 4, 500)
    assert not np.array_equal(x["hidden"], y["hidden"])


def test_pending_limit_and_queue(setup):
    C, g, m, taps = setup
    assert C.pending_limit(g["windows"]) == C.PENDING_ROWS
    assert C.pending_limit([5, 3]) == C.PENDING_ROWS
    assert C.pending_limit([700, 3]) == 700 + C.BLOCK_SLACK
    ctx = C.Context(m)
    ctx.queue(10, taps[:600])            # 600 wait: 88 over the limit, 128 go through
    assert ctx.settled_calls == [(10, 128)]
    assert ctx.len == 128 and ctx.pending.shape[0] == 472 and ctx.span() == (10, 610)
    ctx.queue(610, taps[600:601])        # 473 wait: under the limit
    assert ctx.settled_calls == [(10, 128)] and ctx.pending.shape[0] == 473
    ctx.truncate(300)                    # pending rows past 300 go
    assert ctx.span() == (10, 300) and ctx.pending.shape[0] == 162
    ctx.settle()
    assert ctx.settled_calls[-1] == (138, 162) and ctx.len == 290
    # queued rows are the rows a push makes
    ref = C.Context(m, drop=False)
    ref.push(10, taps[:290])
    q = C.Context(m, drop=False)
    q.queue(10, taps[:600])
    q.truncate(300)
    q.settle()
    for l in range(g["layers"]):
        assert np.array_equal(q.k[l], ref.k[l]) and np.array_equal(q.v[l], ref.v[l])


def test_rewind_after_drop_equals_fresh(setup):
    C, g, m, taps = setup
    ctx = C.Context(m)
    ctx.push(0, taps[:120])
    base = ctx.first + ctx.dropped[1]
    pos = base - 10                      # below the first held row of layer 1
    ctx.truncate(pos)
    assert ctx.len == pos and ctx.dropped[1] == pos and ctx.k[1].shape[0] == 0
    ctx.push(pos, taps[300:340])
    fresh = C.Context(m)
    fresh.push(0, np.concatenate([taps[:pos], taps[300:340]]))
    assert ctx.span() == fresh.span()
    _same(ctx.block(3, ctx.len, 6, 500), fresh.block(3, fresh.len, 6, 500), "rewind")


def test_position_rule(setup):
    C, g, m, taps = setup
    ctx = C.Context(m)
    ctx.push(50, taps[:20])
    assert ctx.span() == (50, 70)
    ctx.queue(75, taps[:3])              # a gap restarts at 75
    assert ctx.span() == (75, 78) and ctx.len == 0
    ctx.queue(70, taps[:2])              # before first: restart
    assert ctx.span() == (70, 72)
    ctx.queue(71, taps[:4])              # inside: cut at 71, append
    assert ctx.span() == (70, 75)
