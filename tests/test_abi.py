"""The C-ABI library loads on the CPU, exports every symbol the header
declares, and rejects invalid geometries before touching a device."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dflash_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = pkg.lib()
    declared = _declared()
    assert declared, "no declarations found"
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(pkg.EXPORTS)


def _try_create(**over):
    g = synth.small_geometry(hidden=128, intermediate=128, heads=2, kv_heads=1, head_dim=64,
                             vocab=64, mask_token=63, layers=1, windows=[0])
    w = synth.make_weights(g, seed=0)
    g.update(over)
    if "layers" in over:
        g["windows"] = [0] * max(1, over["layers"])
    try:
        pkg.Drafter(g, w, max_context=16)
    except pkg.DflashError as e:
        return e
    return None


@pytest.mark.parametrize("over", [
    dict(layers=0), dict(block=1), dict(block=17), dict(kv_heads=3), dict(head_dim=48),
    dict(conv_group=3), dict(hidden=96), dict(intermediate=200), dict(selector_top=0),
    dict(selector_top=33), dict(selector_rank=0), dict(mask_token=64), dict(conv_kernel=0),
    dict(n_taps=0), dict(hidden=5248),
])
def test_invalid_geometry_is_rejected_on_the_host(over):
    e = _try_create(**over)
    assert e is not None and e.code == pkg.DFLASH_EINVAL
    assert "geometry" in pkg.dflash_last_error(None)


def test_null_arguments():
    lib = pkg.lib()
    h = C.c_void_p()
    assert lib.dflash_create(None, None, None, C.byref(h)) == pkg.DFLASH_EINVAL
    assert h.value is None
    assert lib.dflash_settle(None, 0, 1, None) == pkg.DFLASH_EINVAL
    assert lib.dflash_block(None, 0, 0, 1, 8, None, None, None, None, None) == pkg.DFLASH_EINVAL
    lib.dflash_destroy(None)
