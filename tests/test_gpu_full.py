"""Parity at the full sidecar sizes, in the launch configuration the
benchmark times: whole blocks over a synthetic context store (loaded through
the debug entry, so no oracle input comes from the GPU), every row of 256-row
and 8-row settles, and the 27B stream's own composition end to end (a
library-settled context longer than the layers' windows, then the stream's
8-row settle and a block), the oracle settling its own context from the same
tap rows."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth

from test_gpu_parity import REL, check_selection, close, forced_select, run_block

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_cache = {}


def sidecar(name):
    """Weights drawn on the GPU (fast) and held as host arrays, once per session."""
    if name not in _cache:
        g = synth.geometry(name)
        w = synth.make_weights(g, seed=0, device=_dev())
        _cache.clear()
        _cache[name] = (g, w)
    return _cache[name]


def drafter(g, w, cap):
    return pkg.Drafter(g, w, max_context=cap, stream=torch.cuda.current_stream(_dev()).cuda_stream)


# width None: the full vocabulary; 65536: the shortlisted head (the first
# 65536 columns), which runs the head at four tiles a wave
@pytest.mark.parametrize("name,ctx,k,width", [("t27b", 32768, 15, None), ("t27b", 32768, 15, 65536),
                                              ("qwen3_4b", 4096, 15, None),
                                              ("t27b_long", 131072, 15, None)])
def test_full_block_over_synthetic_store(orc, name, ctx, k, width):
    g, w = sidecar(name)
    dev = _dev()
    store = synth.make_store(g, ctx, seed=1, device=dev)
    d = drafter(g, w, ctx + 16)
    try:
        first = 5
        d.debug_load_store(first, ctx, [s[0].data_ptr() for s in store],
                           [s[1].data_ptr() for s in store])
        a = first + ctx
        anchor = synth.uniform_tokens(g, 1, seed=3)[0]
        width = width or g["vocab"]
        tag = name if width == g["vocab"] else f"{name} width {width}"
        print(f"{tag}: block at a={a} over {ctx} positions, width {width}", flush=True)
        trace = torch.zeros(g["layers"], g["block"], g["hidden"], device=dev)
        d.debug_set_trace(trace.data_ptr())
        got = run_block(d, g, anchor, a, k, width)
        d.debug_set_trace(None)
        host_store = [(s[0].cpu().numpy(), s[1].cpu().numpy()) for s in store]
        del store
        m = orc.Model(g, w)
        ref = m.block(host_store, first, ctx, anchor, a, k, width, trace=True)
        tr = trace.cpu().numpy()
        for l in range(g["layers"]):
            e = np.abs(tr[l] - ref["trace"][l])
            print(f"{name} layer {l}: residual max|ref| {np.abs(ref['trace'][l]).max():.3e} "
                  f"max|err| {e.max():.3e} rows {np.round(e.max(axis=1) / np.abs(ref['trace'][l]).max(), 5).tolist()}",
                  flush=True)
        close(got["hidden"], ref["hidden"], f"{tag} hidden")
        close(got["logits"], ref["logits"], f"{tag} logits")
        close(got["hp"], ref["hp"], f"{tag} hp")
        sel = m.select(ref["logits"], ref["hp"], anchor)
        check_selection(got, ref["logits"], sel, tag,
                        forced=forced_select(d, g, got, k, width, anchor))
    finally:
        d.close()


def _store_rows(d, g, n, row0=0):
    dev = _dev()
    kd = g["kv_heads"] * g["head_dim"]
    ks = [torch.empty(n, kd, device=dev) for _ in range(g["layers"])]
    vs = [torch.empty(n, kd, device=dev) for _ in range(g["layers"])]
    for l in range(g["layers"]):
        d.debug_read_store(l, row0, n, ks[l].data_ptr(), vs[l].data_ptr())
    d.sync()
    return [k.cpu().numpy() for k in ks], [v.cpu().numpy() for v in vs]


@pytest.mark.parametrize("name", ["t27b", "qwen3_4b"])
def test_full_settle_every_row(orc, name):
    """Every row of a 256-row settle (the many-row kernels; tap rows with
    outlier channels) and of an 8-row settle (the stream's kernels)."""
    g, w = sidecar(name)
    dev = _dev()
    d = drafter(g, w, 300)
    try:
        m = orc.Model(g, w)
        for n, first, outl in ((256, 32768, True), (8, 40000, False)):
            taps = synth.make_taps(g, n, seed=n, outliers=outl, device=dev)
            d.settle(first, n, taps.data_ptr())
            ks, vs = _store_rows(d, g, n)
            print(f"{name}: settle of {n} rows at {first}, every row against the oracle",
                  flush=True)
            K, V = m.settle(taps.cpu().numpy(), first)
            for l in range(g["layers"]):
                close(ks[l], K[l], f"{name} settle {n} K layer {l}")
                close(vs[l], V[l], f"{name} settle {n} V layer {l}")
    finally:
        d.close()


def test_27b_repeat_bit_identical():
    """The same work twice gives the same bits: a 256-row settle (the fc and
    K/V kernels with their async-copy rings) re-settled at the same position,
    and a block over it. A missing wait between an async copy and its reader
    would show here as a difference between the two runs."""
    g, w = sidecar("t27b")
    dev = _dev()
    d = drafter(g, w, 600)
    try:
        taps = synth.make_taps(g, 512, seed=5, outliers=True, device=dev)
        anchor = synth.uniform_tokens(g, 1, seed=6)[0]
        runs = []
        for _ in range(2):
            d.settle(100, 512, taps.data_ptr())  # a rewind to 100 on the second run
            ks, vs = _store_rows(d, g, 512)
            got = run_block(d, g, anchor, 612, 15, g["vocab"])
            runs.append((ks, vs, got))
        (k0, v0, b0), (k1, v1, b1) = runs
        for l in range(g["layers"]):
            assert np.array_equal(k0[l], k1[l]) and np.array_equal(v0[l], v1[l]), l
        for n in ("logits", "hidden", "hp", "cand", "score", "chosen"):
            assert np.array_equal(b0[n], b1[n]), n
    finally:
        d.close()


def test_27b_stream_end_to_end(orc):
    """The 27B stream's composition: 2304 positions settled through the
    library (nine 256-row passes: longer than the 2048-position windows),
    then the next 8 rows (the stream's 8-row settle), then a block at the new
    end, width = vocabulary. The oracle settles the same tap rows itself; the
    store, the block's rows, logits, selector projections and selection are
    compared."""
    g, w = sidecar("t27b")
    dev = _dev()
    n0, n1, first = 2304, 8, 1000
    d = drafter(g, w, n0 + n1 + 16)
    try:
        taps = synth.make_taps(g, n0 + n1, seed=11, name="e2e", device=dev)
        d.settle(first, n0, taps.data_ptr())
        d.settle(first + n0, n1, taps[n0:].data_ptr())
        assert d.span() == (first, first + n0 + n1)
        a = first + n0 + n1
        anchor, k, width = synth.uniform_tokens(g, 1, seed=12)[0], g["block"] - 1, g["vocab"]
        got = run_block(d, g, anchor, a, k, width)
        ks, vs = _store_rows(d, g, n0 + n1)
        host_taps = taps.cpu().numpy()
        del taps
        m = orc.Model(g, w)
        print(f"t27b end to end: oracle settles {n0 + n1} rows", flush=True)
        K, V = m.settle(host_taps, first)
        for l in range(g["layers"]):
            close(ks[l], K[l], f"t27b e2e store K layer {l}")
            close(vs[l], V[l], f"t27b e2e store V layer {l}")
        print(f"t27b end to end: oracle block at a={a}", flush=True)
        ref = m.block([(K[l], V[l]) for l in range(g["layers"])], first, n0 + n1, anchor, a, k,
                      width)
        close(got["hidden"], ref["hidden"], "t27b e2e hidden")
        close(got["logits"], ref["logits"], "t27b e2e logits")
        close(got["hp"], ref["hp"], "t27b e2e hp")
        sel = m.select(ref["logits"], ref["hp"], anchor)
        check_selection(got, ref["logits"], sel, "t27b e2e",
                        forced=forced_select(d, g, got, k, width, anchor))
    finally:
        d.close()


def test_tiny_sidecar_end_to_end(orc):
    """The tiny fp32 sidecar: 128 settled positions then one block at 128,
    the oracle settling its own context."""
    g = synth.geometry("tiny")
    w = synth.make_weights(g, seed=0)
    d = drafter(g, w, 144)
    try:
        taps = synth.make_taps(g, 128, seed=0)
        d.settle(0, 128, taps.to(_dev()).data_ptr())
        m = orc.Model(g, w)
        K, V = m.settle(taps.numpy(), 0)
        anchor, k = 17, g["block"] - 1
        got = run_block(d, g, anchor, 128, k, g["vocab"])
        ref = m.block([(K[l], V[l]) for l in range(g["layers"])], 0, 128, anchor, 128, k,
                      g["vocab"])
        close(got["logits"], ref["logits"], "tiny logits")
        close(got["hp"], ref["hp"], "tiny hp")
        check_selection(got, ref["logits"], m.select(ref["logits"], ref["hp"], anchor), "tiny")
    finally:
        d.close()
