"""GPU path against the CPU oracle, on the same seeded inputs, through the
C-ABI. Floating-point outputs must satisfy max|err| ≤ 2e-3·max|ref| per
tensor and call; integer and index work is compared exactly (candidates and
chosen tokens where the oracle's margin exceeds that tolerance)."""
import math

import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth
from margins import record

pytestmark = pytest.mark.gpu

REL = 2e-3


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def close(got, ref, what, rel=REL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    tol = rel * np.abs(ref).max()
    err = np.abs(got - ref).max() if got.size else 0.0
    print(f"{what}: max|err| {err:.3e} tol {tol:.3e}", flush=True)
    record(what, err, tol)
    assert err <= tol, f"{what}: max|err| {err:.3e} > {tol:.3e}"


def make(g, seed, max_context):
    w = synth.make_weights(g, seed=seed)
    stream = torch.cuda.current_stream(_dev()).cuda_stream
    return w, pkg.Drafter(g, w, max_context=max_context, stream=stream)


def run_block(d, g, anchor, a, k, width):
    dev = _dev()
    top = g["selector_top"]
    out = dict(logits=torch.empty(k, width, device=dev),
               cand=torch.empty(k, top, dtype=torch.int32, device=dev),
               unary=torch.empty(k, top, device=dev), score=torch.empty(k, top, device=dev),
               chosen=torch.empty(k, dtype=torch.int32, device=dev),
               hidden=torch.empty(g["block"], g["hidden"], device=dev),
               hp=torch.empty(k, g["selector_rank"], device=dev))
    d.block(anchor, a, k, width, out["logits"].data_ptr(), out["cand"].data_ptr(),
            out["unary"].data_ptr(), out["score"].data_ptr(), out["chosen"].data_ptr())
    d.debug_last_block(out["hidden"].data_ptr(), out["hp"].data_ptr())
    d.sync()
    return {n: t.cpu().numpy() for n, t in out.items()}


def _check_chain_rows(got, ref_sel, rows, stau, what):
    """Scores (within stau) and chosen tokens (where the oracle's best score
    leads the second by more than stau) of the given rows, wherever the
    candidate lists agree."""
    compared = 0
    for j in rows:
        if not np.array_equal(got["cand"][j], ref_sel["cand"][j]):
            continue
        err = np.abs(got["score"][j] - ref_sel["score"][j]).max()
        record(f"{what} score row {j}", err, stau)
        assert err <= stau, f"{what} score row {j}: max|err| {err:.3e} > {stau:.3e}"
        s = np.sort(ref_sel["score"][j])[::-1]
        if s.size < 2 or s[0] - s[1] > stau:
            assert got["chosen"][j] == ref_sel["chosen"][j], (what, "chosen", j)
        compared += 1
    return compared


def check_selection(got, ref_logits, ref_sel, what, forced=None):
    """Candidates where the oracle's neighbouring gaps exceed τ; scores and
    chosen tokens along the chain while it agrees. After the first row where
    the chains part (a candidate list or a chosen token differs), the later
    rows are compared under the oracle's chain: `forced(prev)` re-runs the
    GPU selection on its own logits and projections with each row's
    predecessor forced to the oracle's choice before it."""
    tau = REL * np.abs(ref_logits).max()
    k, top = ref_sel["cand"].shape
    for j in range(k):
        row = np.sort(ref_logits[j])[::-1]
        for t in range(top):
            lo_gap = row[t] - row[t + 1] if t + 1 < row.size else np.inf
            hi_gap = row[t - 1] - row[t] if t > 0 else np.inf
            if lo_gap > tau and hi_gap > tau:
                assert got["cand"][j, t] == ref_sel["cand"][j, t], (what, j, t)
    stau = REL * np.abs(ref_sel["score"]).max()
    part = k
    for j in range(k):
        if (not np.array_equal(got["cand"][j], ref_sel["cand"][j])
                or got["chosen"][j] != ref_sel["chosen"][j]):
            part = j
            break
    _check_chain_rows(got, ref_sel, range(min(part + 1, k)), stau, what)
    if part + 1 < k and forced is not None:
        prev = np.concatenate([[0], ref_sel["chosen"][:-1]]).astype(np.int32)
        again = forced(prev)
        n = _check_chain_rows(again, ref_sel, range(part + 1, k), stau, what + " (forced chain)")
        print(f"{what}: chains part at row {part}; {n} later rows compared under the oracle's "
              "chain", flush=True)
    return part


def forced_select(d, g, got, k, width, anchor):
    """The GPU selection on the block's own logits and selector projections,
    with every row's predecessor forced (`dflash_debug_select`)."""
    dev = _dev()
    top = g["selector_top"]

    def run(prev):
        lg = torch.tensor(got["logits"], device=dev)
        hp = torch.tensor(got["hp"], device=dev)
        fp = torch.tensor(prev, dtype=torch.int32, device=dev)
        out = dict(cand=torch.empty(k, top, dtype=torch.int32, device=dev),
                   unary=torch.empty(k, top, device=dev), score=torch.empty(k, top, device=dev),
                   chosen=torch.empty(k, dtype=torch.int32, device=dev))
        d.debug_select(lg.data_ptr(), hp.data_ptr(), k, width, anchor, fp.data_ptr(),
                       out["cand"].data_ptr(), out["unary"].data_ptr(), out["score"].data_ptr(),
                       out["chosen"].data_ptr())
        d.sync()
        return {n: t.cpu().numpy() for n, t in out.items()}

    return run


def strengthen_codebooks(w, seed=1, std=0.5):
    """Codebooks large enough for the selector to reorder the candidates."""
    rng = np.random.default_rng(seed)
    for name in ("pred_book", "succ_book"):
        w[name] = (rng.standard_normal(w[name].shape) * std).astype(np.float16).view(np.uint16)


# ------------------------------------------------------------------ pieces

@pytest.fixture(scope="module")
def small():
    g = synth.small_geometry(windows=[0, 5], no_rope=[1])
    w, d = make(g, seed=1, max_context=600)
    yield g, w, d
    d.close()


def test_dequant_bit_exact(small, orc):
    g, w, d = small
    dev = _dev()
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    for l in range(g["layers"]):
        for which, name in enumerate(names):
            codes, scale = w["layers"][l][name]
            ref = orc.dequant_q4(codes, scale).astype(np.float32)
            out = torch.empty(ref.shape, device=dev)
            d.debug_dequant(l, which, out.data_ptr())
            d.sync()
            assert np.array_equal(out.cpu().numpy(), ref), (l, name)


@pytest.mark.parametrize("m", [1, 7, 16, 37])
def test_matvec_parity(small, orc, m):
    g, w, d = small
    dev = _dev()
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    rng = np.random.default_rng(m)
    cases = []
    for which, name in enumerate(names):
        codes, scale = w["layers"][1][name]
        cases.append((1, which, ("q4", codes, scale)))
    cases.append((0, pkg.W_ATTN_KPROJ, ("f16", w["layers"][0]["attn_kproj"])))
    cases.append((1, pkg.W_MLP_KPROJ, ("f16", w["layers"][1]["mlp_kproj"])))
    cases.append((0, pkg.W_FC, ("f16", w["fc"])))
    cases.append((0, pkg.W_SEL, ("f16", w["sel_proj"])))
    if m <= 16:
        cases.append((0, pkg.W_HEAD, ("f16", w["head"])))
    for layer, which, mat in cases:
        if mat[0] == "q4":
            rows, cols = mat[1].shape[0], mat[1].shape[1] * 2
        else:
            rows, cols = mat[1].shape
        x = rng.standard_normal((m, cols)).astype(np.float32)
        ref = orc.apply_q4(mat[1], mat[2], x) if mat[0] == "q4" else orc.apply_f16(mat[1], x)
        xd = torch.tensor(x, device=dev)
        y = torch.empty(m, rows, device=dev)
        d.debug_matvec(layer, which, xd.data_ptr(), m, y.data_ptr())
        d.sync()
        close(y.cpu().numpy(), ref, f"matvec {which} m={m}")


# ------------------------------------------------------------------ settle

def held_store(d, g):
    """The rows each layer holds (positions first + dropped .. first + settled)."""
    dev = _dev()
    kd = g["kv_heads"] * g["head_dim"]
    _, settled, _, dropped = d.state()
    out = []
    for l in range(g["layers"]):
        n = settled - dropped[l]
        k = torch.empty(max(n, 1), kd, device=dev)
        v = torch.empty(max(n, 1), kd, device=dev)
        d.debug_read_store(l, dropped[l], n, k.data_ptr(), v.data_ptr())
        out.append((k[:n], v[:n]))
    d.sync()
    return [(k.cpu().numpy(), v.cpu().numpy()) for k, v in out]


def same_state(d, ctx):
    """The library's bookkeeping equals the oracle context's, exactly."""
    first, settled, waiting, dropped = d.state()
    assert (first, settled, waiting, dropped) == (ctx.first, ctx.len, ctx.pending.shape[0],
                                                  list(ctx.dropped)), (d.state(), ctx.span())
    assert d.span() == ctx.span()


# row counts where the kernels change: one 16-row block (the 16-row block
# kernels), 17 and 32 rows (the many-row fc, the small-row int4 K/V), 33
# rows (the many-row K/V), a full 256-row call, and more than one call.
# The handle is shared: each start lies past the previous span's end or at
# or before its first position, so every case settles a fresh context.
@pytest.mark.parametrize("n,first", [(1, 0), (16, 3), (17, 0), (32, 50), (33, 90), (40, 200),
                                     (256, 0), (300, 400)])
def test_settle_parity(small, orc, n, first):
    from oracle.context import Context

    g, w, d = small
    dev = _dev()
    taps = synth.make_taps(g, n, seed=n)
    d.settle(first, n, taps.to(dev).data_ptr())
    assert d.span() == (first, first + n)
    ctx = Context(orc.Model(g, w))
    ctx.push(first, taps.numpy())
    same_state(d, ctx)
    got = held_store(d, g)
    for l in range(g["layers"]):
        close(got[l][0], ctx.k[l], f"settle K layer {l}")
        close(got[l][1], ctx.v[l], f"settle V layer {l}")


def test_settle_position_rule(small):
    g, w, d = small
    dev = _dev()
    taps = synth.make_taps(g, 30, seed=5).to(dev)
    d.truncate(0)                                   # empty context
    d.settle(50, 20, taps.data_ptr())               # an empty context restarts at first_pos
    assert d.span() == (50, 70)
    d.settle(70, 5, taps[20:].data_ptr())           # append
    assert d.span() == (50, 75)
    d.settle(60, 3, taps[10:].data_ptr())           # rewind to 60, then append
    assert d.span() == (50, 63)
    d.settle(90, 2, taps.data_ptr())                # gap: restart
    assert d.span() == (90, 92)
    d.settle(10, 1, taps.data_ptr())                # before first: restart
    assert d.span() == (10, 11)
    d.truncate(10)
    assert d.span() == (10, 10)
    with pytest.raises(pkg.DflashError) as e:
        d.settle(10, 601, taps.data_ptr())          # over max_context: no state change
    assert e.value.code == pkg.DFLASH_ENOMEM and d.span() == (10, 10)


def test_rewind_resettle_equals_fresh(small):
    g, w, d = small
    dev = _dev()
    taps = synth.make_taps(g, 24, seed=8).to(dev)
    other = synth.make_taps(g, 24, seed=9).to(dev)
    d.settle(0, 24, taps.data_ptr())
    fresh, st_fresh = held_store(d, g), d.state()
    d.settle(0, 24, other.data_ptr())
    d.settle(10, 14, taps[10:].data_ptr())
    mixed = held_store(d, g)
    assert d.state() == st_fresh
    for l in range(g["layers"]):
        keep = max(0, 10 - st_fresh[3][l])  # held rows at positions ≥ 10
        assert np.array_equal(fresh[l][0][keep:], mixed[l][0][keep:])
        assert np.array_equal(fresh[l][1][keep:], mixed[l][1][keep:])


# ------------------------------------------------------------------- block

BLOCK_CASES = [
    # geometry overrides, context (first, length), anchor offset from the end, k, width
    (dict(windows=[0, 0], no_rope=[]), (0, 64), 0, 7, 1000),
    (dict(windows=[0, 5], no_rope=[1]), (100, 40), 0, 7, 1000),
    (dict(windows=[3, 33], no_rope=[0]), (20, 150), 0, 3, 1000),
    (dict(windows=[0, 2], no_rope=[]), (0, 0), 0, 7, 1000),          # empty context
    (dict(windows=[0, 0], no_rope=[]), (30, 90), -25, 1, 8),         # anchor inside, min width
    (dict(windows=[0, 0], no_rope=[], block=16), (0, 200), 0, 15, 1000),
    (dict(windows=[0, 0], no_rope=[], kv_heads=4), (5, 70), 3, 7, 999),
    (dict(windows=[0, 0], no_rope=[], heads=8, kv_heads=1, head_dim=128), (0, 300), 0, 7, 1000),
    # 64 context chunks + the block's own rows: more chunk states than merge
    # threads at head_dim 64
    (dict(windows=[0, 0], no_rope=[]), (0, 8190), 0, 7, 1000),
    # chunks longer than 128 keys take an odd number of 32-key steps (352
    # here: 57 chunks, the last one short)
    (dict(windows=[0, 0], no_rope=[]), (0, 20000), 0, 7, 1000),
    # conv kernels other than 4 taps: one tap; more taps than the conv
    # kernels load ahead of their barrier (4), with wider groups; a tap for
    # every block row
    (dict(windows=[0, 0], no_rope=[], conv_kernel=1), (0, 50), 0, 7, 1000),
    (dict(windows=[0, 7], no_rope=[], conv_kernel=6, conv_group=8), (10, 60), 0, 7, 1000),
    (dict(windows=[0, 0], no_rope=[1], block=16, conv_kernel=16, conv_group=16), (0, 100), 0, 15,
     1000),
    # head_dim 256 (two pairs a lane in the q/k norm and rotary, the widest
    # attention tiles), with a window and a no-rope layer
    (dict(windows=[0, 9], no_rope=[1], heads=4, kv_heads=2, head_dim=256), (3, 90), 0, 7, 1000),
    (dict(windows=[0, 0], no_rope=[], heads=2, kv_heads=1, head_dim=256, block=16), (0, 300), 0,
     15, 1000),
    # codebooks strong enough for the selector to reorder candidates
    (dict(windows=[0, 5], no_rope=[], _strong=True), (0, 80), 0, 7, 1000),
    (dict(windows=[0, 0], no_rope=[], block=16, vocab=3000, mask_token=2999, _strong=True),
     (7, 120), 0, 15, 3000),
]


@pytest.mark.parametrize("case", BLOCK_CASES)
def test_block_parity(orc, case):
    over, (first, length), da, k, width = case
    over = dict(over)
    strong = over.pop("_strong", False)
    g = synth.small_geometry(**over)
    if strong:
        w = synth.make_weights(g, seed=2)
        strengthen_codebooks(w)
        d = pkg.Drafter(g, w, max_context=max(length, 1) + 8,
                        stream=torch.cuda.current_stream(_dev()).cuda_stream)
    else:
        w, d = make(g, seed=2, max_context=max(length, 1) + 8)
    try:
        from oracle.context import Context

        dev = _dev()
        m = orc.Model(g, w)
        ctx = Context(m)
        if length:
            taps = synth.make_taps(g, length, seed=3)
            d.settle(first, length, taps.to(dev).data_ptr())
            ctx.push(first, taps.numpy())
        same_state(d, ctx)
        a = first + length + da
        anchor = 123
        got = run_block(d, g, anchor, a, k, width)
        ref = ctx.block(anchor, a, k, width)
        tag = f"block {over} ctx {length}"
        close(got["hidden"], ref["hidden"], tag + " hidden")
        close(got["logits"], ref["logits"], tag + " logits")
        close(got["hp"], ref["hp"], tag + " hp")
        sel = m.select(ref["logits"], ref["hp"], anchor)
        check_selection(got, ref["logits"], sel, tag,
                        forced=forced_select(d, g, got, k, width, anchor))
        if strong:  # the selector must have reordered something
            assert np.any(sel["chosen"] != sel["plain"]), "codebooks too weak to reorder"
    finally:
        d.close()


def test_probe_peaks(small):
    """The peak probes run on a small sidecar (a head buffer far smaller than
    the probe's grid: most waves get an empty chunk) and return rates."""
    _, _, d = small
    read_gbs, mfma_tfs = d.probe_peaks(1)
    assert math.isfinite(read_gbs) and read_gbs > 0
    assert math.isfinite(mfma_tfs) and mfma_tfs > 0
    with pytest.raises(pkg.DflashError):
        d.probe_peaks(0)


def test_block_is_deterministic(small):
    g, w, d = small
    dev = _dev()
    taps = synth.make_taps(g, 50, seed=4)
    d.settle(0, 50, taps.to(dev).data_ptr())
    a = run_block(d, g, 9, 50, 7, 1000)
    b = run_block(d, g, 9, 50, 7, 1000)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# ----------------------------------------------------------------- select

# (top, rank): the staged codebook rows in 16-byte pieces (rank a multiple of
# 8), at the largest top and rank; and the element-wise path (rank 20)
@pytest.mark.parametrize("top,rank", [(16, 32), (32, 256), (7, 20)])
@pytest.mark.parametrize("strong", [False, True])
def test_select_parity(orc, strong, top, rank):
    g = synth.small_geometry(vocab=5000, mask_token=4999, selector_top=top, selector_rank=rank)
    w, d = make(g, seed=6, max_context=8)
    try:
        dev = _dev()
        if strong:  # codebooks large enough for the selector to reorder
            strengthen_codebooks(w)
            d.close()
            d = pkg.Drafter(g, w, max_context=8, stream=torch.cuda.current_stream(dev).cuda_stream)
        rng = np.random.default_rng(2)
        k, width = 7, 4093
        logits = rng.integers(-30, 30, (k, width)).astype(np.float32) / 4  # many exact ties
        hp = rng.standard_normal((k, g["selector_rank"])).astype(np.float32)
        top = g["selector_top"]
        ld, hd_ = torch.tensor(logits, device=dev), torch.tensor(hp, device=dev)
        cand = torch.empty(k, top, dtype=torch.int32, device=dev)
        unary = torch.empty(k, top, device=dev)
        score = torch.empty(k, top, device=dev)
        chosen = torch.empty(k, dtype=torch.int32, device=dev)
        d.debug_select(ld.data_ptr(), hd_.data_ptr(), k, width, 77, None, cand.data_ptr(),
                       unary.data_ptr(), score.data_ptr(), chosen.data_ptr())
        d.sync()
        ref = orc.Model(g, w).select(logits, hp, 77)
        assert np.array_equal(cand.cpu().numpy(), ref["cand"])       # same f32 inputs: exact
        assert np.array_equal(unary.cpu().numpy(), ref["unary"].astype(np.float32))
        got = dict(cand=cand.cpu().numpy(), score=score.cpu().numpy(),
                   chosen=chosen.cpu().numpy())
        check_selection(got, logits, ref, "select")
        # forced predecessors: every row scored against the oracle's chain
        fp = torch.tensor(np.concatenate([[77], ref["chosen"][:-1]]).astype(np.int32), device=dev)
        d.debug_select(ld.data_ptr(), hd_.data_ptr(), k, width, 77, fp.data_ptr(),
                       cand.data_ptr(), unary.data_ptr(), score.data_ptr(), chosen.data_ptr())
        d.sync()
        close(score.cpu().numpy(), ref["score"], "forced scores")
    finally:
        d.close()


def test_block_ties_everywhere(orc):
    """A zero head makes every logit exactly 0: the candidates are the first
    `top` token ids in order and every unary is 0 (exact tie-break path)."""
    g = synth.small_geometry(vocab=3000, mask_token=2999)
    w = synth.make_weights(g, seed=7)
    w["head"] = np.zeros_like(w["head"])
    stream = torch.cuda.current_stream(_dev()).cuda_stream
    d = pkg.Drafter(g, w, max_context=40, stream=stream)
    try:
        taps = synth.make_taps(g, 30, seed=1)
        d.settle(0, 30, taps.to(_dev()).data_ptr())
        got = run_block(d, g, 5, 30, 7, 3000)
        top = g["selector_top"]
        assert np.all(got["logits"] == 0)
        assert np.array_equal(got["cand"], np.tile(np.arange(top), (7, 1)))
        assert np.all(got["unary"] == 0)
        m = orc.Model(g, w)
        K, V = m.settle(taps.numpy(), 0)
        ref = m.block([(K[l], V[l]) for l in range(g["layers"])], 0, 30, 5, 30, 7, 3000)
        sel = m.select(ref["logits"], ref["hp"], 5)
        assert np.array_equal(sel["cand"], got["cand"])
        check_selection(got, np.ones_like(ref["logits"]), sel, "ties")
    finally:
        d.close()
