"""DFlash 2 drafter forward pass (context settle + block pass) on one MI355X.

A thin ctypes binding of libdflash.so, the C-ABI library declared in
include/dflash.h. Functions carry the C names; arguments are plain integers
and pointers (torch tensors' data_ptr() for device buffers). Every step of
the computation runs in the library's HIP kernels: nothing here computes.
`Drafter` wraps a handle for callers that hold a geometry dict and numpy
weights (as produced by `block_drafter_settle_amd.synth`).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdflash.so")

DFLASH_OK, DFLASH_EINVAL, DFLASH_ENOMEM, DFLASH_EHIP = 0, -1, -2, -3
(W_Q, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN, W_ATTN_KPROJ, W_MLP_KPROJ, W_FC, W_HEAD,
 W_SEL) = range(12)


class DflashError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


class I4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p)]


class LayerW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("in_norm", "post_norm", "q_norm", "k_norm",
                                          "attn_base", "mlp_base", "attn_kproj", "mlp_kproj")]
    _fields_ += [(n, I4) for n in ("q", "k", "v", "o", "gate", "up", "down")]


class Geometry(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("hidden", "intermediate", "layers", "heads", "kv_heads",
                                         "head_dim", "vocab", "block", "mask_token", "conv_group",
                                         "conv_kernel", "selector_rank", "selector_top",
                                         "n_taps")]
    _fields_ += [("windows", C.c_void_p), ("rotary", C.c_void_p), ("rope_theta", C.c_double),
                 ("eps", C.c_double), ("max_context", C.c_int64)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("fc", "hidden_norm", "norm", "sel_proj", "pred_book",
                                          "succ_book", "embed", "head", "layer")]


_lib = None

_SIGS = {
    "dflash_create": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_settle": ([C.c_void_p, C.c_int64, C.c_int32, C.c_void_p], C.c_int),
    "dflash_block": ([C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_block_noalloc": ([C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_create_context": ([C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_block_batch": ([C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                            C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_route_margin": ([C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                             C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p], C.c_int),
    "dflash_queue": ([C.c_void_p, C.c_int64, C.c_int32, C.c_void_p], C.c_int),
    "dflash_flush": ([C.c_void_p], C.c_int),
    "dflash_reserve": ([C.c_void_p, C.c_int64], C.c_int),
    "dflash_state": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_truncate": ([C.c_void_p, C.c_int64], C.c_int),
    "dflash_span": ([C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_sync": ([C.c_void_p], C.c_int),
    "dflash_destroy": ([C.c_void_p], None),
    "dflash_last_error": ([C.c_void_p], C.c_char_p),
    "dflash_set_timing": ([C.c_void_p, C.c_int], C.c_int),
    "dflash_stage_times": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_probe_peaks": ([C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_debug_dequant": ([C.c_void_p, C.c_int32, C.c_int32, C.c_void_p], C.c_int),
    "dflash_debug_matvec": ([C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32,
                             C.c_void_p], C.c_int),
    "dflash_debug_read_store": ([C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_void_p,
                                 C.c_void_p], C.c_int),
    "dflash_debug_load_store": ([C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p],
                                C.c_int),
    "dflash_debug_last_block": ([C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "dflash_debug_set_trace": ([C.c_void_p, C.c_void_p], C.c_int),
    "dflash_debug_select": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
}

EXPORTS = tuple(_SIGS)

# stage order of the library's timers (include/dflash.h, DFLASH_ST_*)
STAGES = ("kproj", "conv_norm", "qkv", "qk_post", "attention", "o", "gate_up", "down", "head",
          "select", "settle_taps", "settle_fc", "settle_norm", "settle_kv", "settle_store")


def lib():
    """Load libdflash.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_drafter_settle_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc, handle=None):
    if rc != DFLASH_OK:
        msg = lib().dflash_last_error(handle)
        raise DflashError(rc, msg.decode() if msg else "")


def dflash_create(geometry_p, weights_p, stream, out_p):
    return lib().dflash_create(geometry_p, weights_p, stream, out_p)


def dflash_settle(h, first_pos, n, taps):
    return lib().dflash_settle(h, first_pos, n, taps)


def dflash_block(h, anchor, a, k, width, logits, cand, unary, score, chosen):
    return lib().dflash_block(h, anchor, a, k, width, logits, cand, unary, score, chosen)


def dflash_block_noalloc(h, anchor, a, k, width, logits, cand, unary, score, chosen):
    return lib().dflash_block_noalloc(h, anchor, a, k, width, logits, cand, unary, score, chosen)


def dflash_create_context(model, max_context, stream, out_p):
    return lib().dflash_create_context(model, max_context, stream, out_p)


def dflash_block_batch(hs_p, nseq, anchors_p, a_p, k, width, logits, cand, unary, score, chosen):
    return lib().dflash_block_batch(hs_p, nseq, anchors_p, a_p, k, width, logits, cand, unary,
                                    score, chosen)


def block_batch(drafters, anchors, a, k, width, logits_ptr, cand_ptr, unary_ptr, score_ptr,
                chosen_ptr):
    """dflash_block_batch over Drafter handles that share weights (the first
    leads); outputs are sequence-major device buffers."""
    n = len(drafters)
    hs = (C.c_void_p * n)(*[x.h.value for x in drafters])
    an = (C.c_int32 * n)(*[int(x) for x in anchors])
    ap = (C.c_int64 * n)(*[int(x) for x in a])
    _check(lib().dflash_block_batch(hs, n, an, ap, k, width, logits_ptr, cand_ptr, unary_ptr,
                                    score_ptr, chosen_ptr), drafters[0].h)


def dflash_queue(h, first_pos, n, taps):
    return lib().dflash_queue(h, first_pos, n, taps)


def dflash_flush(h):
    return lib().dflash_flush(h)


def dflash_reserve(h, rows):
    return lib().dflash_reserve(h, rows)


def dflash_state(h, first_p, settled_p, waiting_p, dropped_p):
    return lib().dflash_state(h, first_p, settled_p, waiting_p, dropped_p)


def dflash_truncate(h, pos):
    return lib().dflash_truncate(h, pos)


def dflash_sync(h):
    return lib().dflash_sync(h)


def dflash_destroy(h):
    lib().dflash_destroy(h)


def dflash_last_error(h):
    msg = lib().dflash_last_error(h)
    return msg.decode() if msg else ""


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p).value


class Drafter:
    """One library handle built from a geometry dict and numpy weights."""

    def __init__(self, g: dict, w: dict, max_context: int, stream: int = 0):
        self.g = g
        self.h = None
        keep = []

        def arr(a, dt):
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            return _ptr(a)

        geo = Geometry()
        for n in ("hidden", "intermediate", "layers", "heads", "kv_heads", "head_dim", "vocab",
                  "block", "mask_token", "conv_group", "conv_kernel", "selector_rank",
                  "selector_top", "n_taps"):
            setattr(geo, n, int(g[n]))
        geo.windows = arr(np.array(g["windows"]), np.int32)
        geo.rotary = arr(np.array([0 if l in g["no_rope"] else 1 for l in range(g["layers"])]),
                         np.uint8)
        geo.rope_theta, geo.eps = float(g["rope_theta"]), float(g["eps"])
        geo.max_context = int(max_context)
        wt = Weights()
        for n in ("fc", "sel_proj", "pred_book", "succ_book", "embed", "head"):
            setattr(wt, n, arr(w[n], np.uint16))
        wt.hidden_norm = arr(w["hidden_norm"], np.float32)
        wt.norm = arr(w["norm"], np.float32)
        layers = (LayerW * max(1, len(w["layers"])))()
        for l, lw in enumerate(w["layers"]):
            L = layers[l]
            for n in ("in_norm", "post_norm", "q_norm", "k_norm", "attn_base", "mlp_base"):
                setattr(L, n, arr(lw[n], np.float32))
            L.attn_kproj = arr(lw["attn_kproj"], np.uint16)
            L.mlp_kproj = arr(lw["mlp_kproj"], np.uint16)
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                codes, scale = lw[n]
                getattr(L, n).q = arr(codes, np.uint8)
                getattr(L, n).scale = arr(scale, np.uint16)
        wt.layer = C.cast(layers, C.c_void_p).value
        h = C.c_void_p()
        rc = lib().dflash_create(C.byref(geo), C.byref(wt), stream, C.byref(h))
        _check(rc, None)
        self.h = h
        del keep

    @classmethod
    def context_of(cls, model: "Drafter", max_context: int, stream: int = 0) -> "Drafter":
        """A handle sharing `model`'s weights with a context of its own
        (dflash_create_context)."""
        self = cls.__new__(cls)
        self.g = model.g
        self.h = None
        h = C.c_void_p()
        _check(lib().dflash_create_context(model.h, int(max_context), stream, C.byref(h)), None)
        self.h = h
        return self

    def close(self):
        if self.h:
            lib().dflash_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # The calls, with pointers to device buffers (torch data_ptr()).
    def settle(self, first_pos: int, n: int, taps_ptr: int):
        _check(lib().dflash_settle(self.h, first_pos, n, taps_ptr), self.h)

    def block(self, anchor: int, a: int, k: int, width: int, logits_ptr, cand_ptr, unary_ptr,
              score_ptr, chosen_ptr):
        _check(lib().dflash_block(self.h, anchor, a, k, width, logits_ptr, cand_ptr, unary_ptr,
                                  score_ptr, chosen_ptr), self.h)

    def block_noalloc(self, anchor: int, a: int, k: int, width: int, logits_ptr, cand_ptr,
                      unary_ptr, score_ptr, chosen_ptr):
        _check(lib().dflash_block_noalloc(self.h, anchor, a, k, width, logits_ptr, cand_ptr,
                                          unary_ptr, score_ptr, chosen_ptr), self.h)

    def route_margin(self, rows_ptr, m: int, block, chain, margin_ptr):
        """dflash_route_margin: block and chain are (mean_ptr, basis_ptr,
        rank) of device f16 buffers; rows and margin device f32."""
        _check(lib().dflash_route_margin(self.h, rows_ptr, m, block[0], block[1], block[2],
                                         chain[0], chain[1], chain[2], margin_ptr), self.h)

    def queue(self, first_pos: int, n: int, taps_ptr: int):
        _check(lib().dflash_queue(self.h, first_pos, n, taps_ptr), self.h)

    def flush(self):
        _check(lib().dflash_flush(self.h), self.h)

    def reserve(self, rows: int):
        _check(lib().dflash_reserve(self.h, rows), self.h)

    def state(self):
        """(first, settled rows, waiting rows, [dropped rows of each layer])."""
        f, s, w = C.c_int64(), C.c_int64(), C.c_int64()
        dr = (C.c_int64 * self.g["layers"])()
        _check(lib().dflash_state(self.h, C.byref(f), C.byref(s), C.byref(w), dr), self.h)
        return f.value, s.value, w.value, list(dr)

    def truncate(self, pos: int):
        _check(lib().dflash_truncate(self.h, pos), self.h)

    def span(self):
        f, e = C.c_int64(), C.c_int64()
        _check(lib().dflash_span(self.h, C.byref(f), C.byref(e)), self.h)
        return f.value, e.value

    def sync(self):
        _check(lib().dflash_sync(self.h), self.h)

    def set_timing(self, on: bool):
        _check(lib().dflash_set_timing(self.h, 1 if on else 0), self.h)

    def stage_times(self):
        us = (C.c_double * len(STAGES))()
        n = (C.c_int64 * len(STAGES))()
        b, s = C.c_int64(), C.c_int64()
        _check(lib().dflash_stage_times(self.h, us, n, C.byref(b), C.byref(s)), self.h)
        return {name: (us[i], n[i]) for i, name in enumerate(STAGES)}, b.value, s.value

    def probe_peaks(self, reps: int = 5):
        """(streaming read GB/s, back-to-back f16 MFMA TFLOP/s) as measured on this GPU."""
        r, m = C.c_double(), C.c_double()
        _check(lib().dflash_probe_peaks(self.h, reps, C.byref(r), C.byref(m)), self.h)
        return r.value, m.value

    def debug_dequant(self, layer, which, out_ptr):
        _check(lib().dflash_debug_dequant(self.h, layer, which, out_ptr), self.h)

    def debug_matvec(self, layer, which, x_ptr, m, y_ptr):
        _check(lib().dflash_debug_matvec(self.h, layer, which, x_ptr, m, y_ptr), self.h)

    def debug_read_store(self, layer, row0, n, k_ptr, v_ptr):
        _check(lib().dflash_debug_read_store(self.h, layer, row0, n, k_ptr, v_ptr), self.h)

    def debug_load_store(self, first, length, k_ptrs, v_ptrs):
        kp = (C.c_void_p * len(k_ptrs))(*k_ptrs)
        vp = (C.c_void_p * len(v_ptrs))(*v_ptrs)
        _check(lib().dflash_debug_load_store(self.h, first, length, kp, vp), self.h)

    def debug_last_block(self, hidden_ptr, hp_ptr):
        _check(lib().dflash_debug_last_block(self.h, hidden_ptr, hp_ptr), self.h)

    def debug_set_trace(self, trace_ptr):
        _check(lib().dflash_debug_set_trace(self.h, trace_ptr), self.h)

    def debug_select(self, logits_ptr, hp_ptr, k, width, anchor, forced_ptr, cand_ptr, unary_ptr,
                     score_ptr, chosen_ptr):
        _check(lib().dflash_debug_select(self.h, logits_ptr, hp_ptr, k, width, anchor, forced_ptr,
                                         cand_ptr, unary_ptr, score_ptr, chosen_ptr), self.h)
