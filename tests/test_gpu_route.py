"""The router margin (dflash_route_margin) against the oracle's
`Route::margin` (oracle/router.py): rows near the block's subspace, near the
chain's and far from both, a zero row and one below the norm floor; ranks 0
to 256, 1 to 64 rows; the 5120-wide target row of the 27B-shaped sidecar.
Each call's margins are compared to the parity tolerance (2e-3 of the
largest |margin|), and the routing decision (the sign) wherever the
oracle's margin is farther than that from zero."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth

from test_gpu_parity import close

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _handle(hidden):
    g = synth.small_geometry(hidden=hidden, intermediate=256, conv_group=8, vocab=300,
                             mask_token=299)
    w = synth.make_weights(g, seed=3)
    return pkg.Drafter(g, w, max_context=16, stream=torch.cuda.current_stream(_dev()).cuda_stream)


def _run(d, rows, blk, chn):
    dev = _dev()
    x = rows.to(dev).contiguous()
    bm, bb = blk[0].to(dev), blk[1].to(dev).contiguous()
    cm, cb = chn[0].to(dev), chn[1].to(dev).contiguous()
    out = torch.full((rows.shape[0],), float("nan"), device=dev)
    d.route_margin(x.data_ptr(), rows.shape[0], (bm.data_ptr(), bb.data_ptr(), blk[2]),
                   (cm.data_ptr(), cb.data_ptr(), chn[2]), out.data_ptr())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _ref(rows, blk, chn):
    from oracle import router

    as_np = lambda s: (s[0].numpy(), s[1].numpy(), s[2])
    return router.margins(rows.numpy(), as_np(blk), as_np(chn))


def _rows(hidden, m, blk, chn, seed):
    """a third near the block's subspace, a third near the chain's, the rest
    N(0, 1); then a zero row and a row below the norm floor if there is room"""
    a = synth.make_route_rows(hidden, m, seed=seed, near=blk, share=1 / 3, name="route.a")
    b = synth.make_route_rows(hidden, m, seed=seed, near=chn, share=1 / 3, name="route.b")
    k = int(round(m / 3))
    rows = a.clone()
    rows[k:2 * k] = b[:k]
    if m >= 5:
        rows[-1] = 0.0
        rows[-2] = 0.0
        rows[-2, 3] = 1e-14
    return rows


@pytest.mark.parametrize("hidden,m,rb,rc", [(256, 1, 16, 16), (256, 7, 0, 5), (256, 64, 256, 3),
                                           (256, 12, 40, 40), (5120, 8, 64, 64),
                                           (5120, 3, 17, 200), (5120, 64, 256, 256)])
def test_route_margin_matches_oracle(hidden, m, rb, rc):
    d = _handle(hidden)
    try:
        blk = synth.make_subspace(hidden, rb, seed=hidden + rb, name="route.block")
        chn = synth.make_subspace(hidden, rc, seed=hidden + rc, name="route.chain")
        rows = _rows(hidden, m, blk, chn, seed=m)
        got = _run(d, rows, blk, chn)
        ref = _ref(rows, blk, chn)
        tag = f"route hidden {hidden} m {m} ranks {rb}/{rc}"
        close(got, ref, tag)
        tol = 2e-3 * np.max(np.abs(ref))
        sure = np.abs(ref) > tol
        assert np.array_equal(np.sign(got[sure]), np.sign(ref[sure])), tag
        # the same call again gives the same bits
        assert np.array_equal(_run(d, rows, blk, chn), got), tag
    finally:
        d.close()


def test_route_margin_rejections():
    d = _handle(256)
    dev = _dev()
    try:
        blk = synth.make_subspace(256, 4, seed=1)
        x = torch.zeros(65, 256, device=dev)
        bm, bb = blk[0].to(dev), blk[1].to(dev)
        out = torch.zeros(65, device=dev)
        good = (bm.data_ptr(), bb.data_ptr(), 4)
        for m, b, c in [(0, good, good), (65, good, good), (3, (bm.data_ptr(), bb.data_ptr(), 257), good),
                        (3, good, (bm.data_ptr(), 0, 2)), (3, good, (0, bb.data_ptr(), 4)),
                        (3, good, (bm.data_ptr(), bb.data_ptr(), -1))]:
            with pytest.raises(pkg.DflashError) as e:
                d.route_margin(x.data_ptr(), m, b, c, out.data_ptr())
            assert e.value.code == pkg.DFLASH_EINVAL
        # rank 0 with no basis is fine
        d.route_margin(x.data_ptr(), 2, (bm.data_ptr(), 0, 0), good, out.data_ptr())
        torch.cuda.synchronize()
    finally:
        d.close()
