"""ctypes front of the CPU oracle (liboracle.so) — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this module. It marshals numpy arrays into the oracle's C structs; every
step of the arithmetic is in dflash_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "dflash_oracle.c")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent outputs)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Q4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("in_norm", "post_norm", "q_norm", "k_norm",
                                          "attn_base", "mlp_base", "attn_kproj", "mlp_kproj")]
    _fields_ += [(n, _Q4) for n in ("q", "k", "v", "o", "gate", "up", "down")]


class _Model(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("hidden", "intermediate", "layers", "heads", "kv_heads",
                                       "head_dim", "vocab", "block", "mask_token", "conv_group",
                                       "conv_kernel", "selector_rank", "selector_top", "n_taps")]
    _fields_ += [("windows", C.c_void_p), ("rotary", C.c_void_p), ("rope_theta", C.c_double),
                 ("eps", C.c_double)]
    _fields_ += [(n, C.c_void_p) for n in ("fc", "hidden_norm", "norm", "sel_proj", "pred_book",
                                           "succ_book", "embed", "head", "layer")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        vp, i, l, d = C.c_void_p, C.c_int, C.c_long, C.c_double
        L.orc_f16.restype = d
        L.orc_f16.argtypes = [C.c_uint16]
        L.orc_dequant_q4.argtypes = [vp, i, i, vp]
        L.orc_inv_freq.argtypes = [d, i, vp]
        L.orc_rms.argtypes = [vp, l, i, vp, d, vp]
        L.orc_rotate.argtypes = [vp, l, i, i, vp, vp]
        L.orc_conv.argtypes = [i, i, i, i, i, vp, vp, vp, vp]
        L.orc_apply_f16.argtypes = [vp, i, i, vp, i, vp]
        L.orc_apply_q4.argtypes = [vp, i, i, vp, i, vp]
        L.orc_attention.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, l, l, l, l, i, vp]
        L.orc_settle.argtypes = [vp, vp, i, l, vp, vp]
        L.orc_settle.restype = i
        L.orc_block.argtypes = [vp, vp, vp, l, l, vp, i, l, i, i, vp, vp, vp, vp]
        L.orc_block.restype = i
        L.orc_top_k.argtypes = [vp, l, i, vp, vp]
        L.orc_select.argtypes = [vp, vp, i, vp, i, i, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f64(a):
    return _c(a, np.float64)


class Model:
    """The oracle's view of a sidecar (geometry dict + weight dict of numpy arrays)."""

    def __init__(self, g: dict, w: dict):
        self.g, self.w = g, w
        self._keep = []
        keep = self._keep.append

        def arr(a, dt):
            a = _c(a, dt)
            keep(a)
            return _p(a)

        m = _Model()
        for n in ("hidden", "intermediate", "layers", "heads", "kv_heads", "head_dim", "vocab",
                  "block", "mask_token", "conv_group", "conv_kernel", "selector_rank",
                  "selector_top", "n_taps"):
            setattr(m, n, int(g[n]))
        m.windows = arr(np.array(g["windows"]), np.int32)
        m.rotary = arr(np.array([0 if l in g["no_rope"] else 1 for l in range(g["layers"])]),
                       np.uint8)
        m.rope_theta, m.eps = float(g["rope_theta"]), float(g["eps"])
        for n in ("fc", "sel_proj", "pred_book", "succ_book", "embed", "head"):
            setattr(m, n, arr(w[n], np.uint16))
        m.hidden_norm = arr(w["hidden_norm"], np.float32)
        m.norm = arr(w["norm"], np.float32)
        layers = (_Layer * g["layers"])()
        for l, lw in enumerate(w["layers"]):
            L = layers[l]
            for n in ("in_norm", "post_norm", "q_norm", "k_norm", "attn_base", "mlp_base"):
                setattr(L, n, arr(lw[n], np.float32))
            L.attn_kproj = arr(lw["attn_kproj"], np.uint16)
            L.mlp_kproj = arr(lw["mlp_kproj"], np.uint16)
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                codes, scale = lw[n]
                getattr(L, n).q = arr(codes, np.uint8)
                getattr(L, n).s = arr(scale, np.uint16)
        keep(layers)
        m.layer = C.cast(layers, C.c_void_p)
        self.m = m

    @property
    def ptr(self):
        return C.byref(self.m)

    # -- settle / block / select -------------------------------------------------

    def settle(self, taps: np.ndarray, pos0: int):
        """K, V of each layer for the tap rows: f32 [layers][n][kv*hd] each."""
        g = self.g
        taps = _c(taps, np.float32)
        n = taps.shape[0]
        kd = g["kv_heads"] * g["head_dim"]
        k = np.zeros((g["layers"], n, kd), np.float32)
        v = np.zeros_like(k)
        rc = lib().orc_settle(self.ptr, _p(taps), n, pos0, _p(k), _p(v))
        assert rc == 0
        return k, v

    def block(self, store, first: int, length: int, anchor: int, a: int, k: int, width: int,
              trace: bool = False, dropped=None):
        """store: per layer (K, V) f32 [rows][kv*hd], row i = position
        first + dropped[l] + i (dropped None: all zero). Returns dict of
        logits [k][width], hp [k][rank], hidden [block][hidden] (float64)."""
        g = self.g
        ks = [_c(s[0], np.float32) for s in store]
        vs = [_c(s[1], np.float32) for s in store]
        kp = (C.c_void_p * g["layers"])(*[_p(x) for x in ks])
        vp = (C.c_void_p * g["layers"])(*[_p(x) for x in vs])
        logits = np.zeros((k, width))
        hp = np.zeros((k, g["selector_rank"]))
        hidden = np.zeros((g["block"], g["hidden"]))
        tr = np.zeros((g["layers"], g["block"], g["hidden"])) if trace else None
        dr = None if dropped is None else _c(dropped, np.int64)
        rc = lib().orc_block(self.ptr, kp, vp, first, length, _p(dr) if dr is not None else None,
                             anchor, a, k, width, _p(logits), _p(hp), _p(hidden),
                             _p(tr) if trace else None)
        assert rc == 0, rc
        out = dict(logits=logits, hp=hp, hidden=hidden)
        if trace:
            out["trace"] = tr
        return out

    def select(self, logits: np.ndarray, hp: np.ndarray, anchor: int, forced_prev=None):
        g = self.g
        logits, hp = f64(logits), f64(hp)
        k, width = logits.shape
        top = g["selector_top"]
        cand = np.zeros((k, top), np.int32)
        unary = np.zeros((k, top))
        score = np.zeros((k, top))
        chosen = np.zeros(k, np.int32)
        plain = np.zeros(k, np.int32)
        fp = None
        if forced_prev is not None:
            fp = _c(forced_prev, np.int32)
        lib().orc_select(self.ptr, _p(logits), width, _p(hp), k, anchor,
                         _p(fp) if fp is not None else None, _p(cand), _p(unary), _p(score),
                         _p(chosen), _p(plain))
        return dict(cand=cand, unary=unary, score=score, chosen=chosen, plain=plain)


# -- the pieces, on their own -------------------------------------------------------

def f16(bits: int) -> float:
    return lib().orc_f16(bits)


def dequant_q4(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    codes, scale = _c(codes, np.uint8), _c(scale, np.uint16)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    w = _Q4(_p(codes).value, _p(scale).value)
    out = np.zeros((rows, cols))
    lib().orc_dequant_q4(C.byref(w), rows, cols, _p(out))
    return out


def inv_freq(theta: float, hd: int) -> np.ndarray:
    out = np.zeros(hd // 2, np.float32)
    lib().orc_inv_freq(theta, hd, _p(out))
    return out


def rms(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = f64(x)
    w = _c(w, np.float32)
    y = np.zeros_like(x)
    lib().orc_rms(_p(x), x.size // w.size, w.size, _p(w), eps, _p(y))
    return y


def rotate(x: np.ndarray, heads: int, hd: int, pos, theta: float) -> np.ndarray:
    """x [rows][heads*hd], pos [rows]."""
    x = f64(x).copy()
    pos = _c(pos, np.int64)
    inv = inv_freq(theta, hd)
    lib().orc_rotate(_p(x), x.shape[0], heads, hd, _p(pos), _p(inv))
    return x


def conv(x: np.ndarray, d: np.ndarray, base: np.ndarray, conv_group: int, conv_kernel: int,
         stage: int) -> np.ndarray:
    x, d = f64(x), f64(d)
    base = _c(base, np.float32)
    rows, hs = x.shape
    y = np.zeros_like(x)
    lib().orc_conv(rows, hs, conv_group, conv_kernel, stage, _p(base), _p(d), _p(x), _p(y))
    return y


def apply_f16(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    w = _c(w, np.uint16)
    x = f64(x)
    y = np.zeros((x.shape[0], w.shape[0]))
    lib().orc_apply_f16(_p(w), w.shape[0], w.shape[1], _p(x), x.shape[0], _p(y))
    return y


def apply_q4(codes: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    codes, scale = _c(codes, np.uint8), _c(scale, np.uint16)
    x = f64(x)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    w = _Q4(_p(codes).value, _p(scale).value)
    y = np.zeros((x.shape[0], rows))
    lib().orc_apply_q4(C.byref(w), rows, cols, _p(x), x.shape[0], _p(y))
    return y


def attention(q, k, v, store_k, store_v, first, length, a, window, heads, kv_heads, hd,
              dropped=0):
    """q [rows][heads*hd], k/v [rows][kv*hd], store [rows][kv*hd] f32 (row i
    = position first + dropped + i)."""
    q, k, v = f64(q), f64(k), f64(v)
    sk, sv = _c(store_k, np.float32), _c(store_v, np.float32)
    rows = q.shape[0]
    y = np.zeros_like(q)
    lib().orc_attention(rows, heads, kv_heads, hd, _p(q), _p(k), _p(v), _p(sk), _p(sv), first,
                        length, dropped, a, window, _p(y))
    return y


def top_k(x, k: int):
    x = f64(x)
    val = np.zeros(k)
    idx = np.zeros(k, np.int32)
    lib().orc_top_k(_p(x), x.size, k, _p(val), _p(idx))
    return val, idx
