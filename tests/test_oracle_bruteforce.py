"""The C oracle against an independent float64 NumPy restatement on tiny
geometries (explicit visibility predicate, explicit zero-padded convolution,
per-head loops), written from the same definitions on the docs.rs page
"cortiq_engine/dflash.rs" (cortiq-engine 0.8.78): `Drafter::block`,
`settle_rows`, `rms`, `rotate`, `conv`, `mlp`."""
import math

import numpy as np
import pytest

from block_drafter_settle_amd import synth


def _unpack(codes, scale):
    q = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    q = np.where(q > 7, q - 16, q)
    s = scale.view(np.float16).astype(np.float64)
    return q * np.repeat(s, 32, axis=1)


def _h(a):
    return a.view(np.float16).astype(np.float64)


class Brute:
    def __init__(self, g, w):
        self.g, self.w = g, w
        self.eps = float(np.float32(g["eps"]))
        hd = g["head_dim"]
        self.inv = np.array([g["rope_theta"] ** (-(2.0 * i) / hd) for i in range(hd // 2)],
                            np.float32)

    def rms(self, x, w):
        out = np.empty_like(x)
        for i in range(x.shape[0]):
            out[i] = x[i] / math.sqrt(np.mean(x[i] ** 2) + self.eps) * w.astype(np.float64)
        return out

    def rope(self, x, pos):  # x [heads][hd]
        hd = x.shape[1]
        half = hd // 2
        out = x.copy()
        for i in range(half):
            ang = float(np.float32(pos) * self.inv[i])
            c, s = math.cos(ang), math.sin(ang)
            out[:, i] = x[:, i] * c - x[:, i + half] * s
            out[:, i + half] = x[:, i + half] * c + x[:, i] * s
        return out

    def conv(self, x, d, base, stage):
        g = self.g
        B, hs = x.shape
        kn, gs = g["conv_kernel"], g["conv_group"]
        G = hs // gs
        d = d.reshape(B, 2, kn, G)
        base = base.reshape(2, kn, hs).astype(np.float64)
        y = np.zeros_like(x)
        for r in range(B):
            for o in range(kn):
                src = x[r - o] if r - o >= 0 else np.zeros(hs)  # zero rows before row 0
                for i in range(hs):
                    y[r, i] += (base[stage, o, i] + d[r, stage, o, i // gs]) * src[i]
        return y

    def block(self, store, first, length, anchor, a, k, width):
        g, w = self.g, self.w
        B, hs, nh, kv, hd = g["block"], g["hidden"], g["heads"], g["kv_heads"], g["head_dim"]
        rep = nh // kv
        E = _h(w["embed"])
        h = np.stack([E[anchor]] + [E[g["mask_token"]]] * (B - 1))
        for l, L in enumerate(w["layers"]):
            win = g["windows"][l]
            rot = l not in g["no_rope"]
            x = self.rms(h, L["in_norm"])
            d = x @ _h(L["attn_kproj"]).T
            xc = self.conv(x, d, L["attn_base"], 0)
            q = xc @ _unpack(*L["q"]).T
            kk = xc @ _unpack(*L["k"]).T
            vv = xc @ _unpack(*L["v"]).T
            q = q.reshape(B, nh, hd)
            kk = kk.reshape(B, kv, hd)
            vv = vv.reshape(B, kv, hd)
            for r in range(B):
                q[r] = self.rms(q[r], L["q_norm"])
                kk[r] = self.rms(kk[r], L["k_norm"])
                if rot:
                    q[r] = self.rope(q[r], a + r)
                    kk[r] = self.rope(kk[r], a + r)
            sk = store[l][0].reshape(-1, kv, hd).astype(np.float64)
            sv = store[l][1].reshape(-1, kv, hd).astype(np.float64)
            y = np.zeros((B, nh, hd))
            for r in range(B):
                for hq in range(nh):
                    gi = hq // rep
                    keys, vals = [], []
                    for p in range(first, first + length):
                        visible = p < a  # only positions before the anchor
                        if win > 0 and p < a + 1 - win:
                            visible = False  # before the layer's first row's reach
                        if win > 0 and p < a + r + 1 - win:
                            visible = False  # before this row's reach
                        if visible:
                            keys.append(sk[p - first, gi])
                            vals.append(sv[p - first, gi])
                    for b in range(B):
                        keys.append(kk[b, gi])
                        vals.append(vv[b, gi])
                    s = np.array([q[r, hq] @ kq for kq in keys]) / math.sqrt(hd)
                    p_ = np.exp(s - s.max())
                    p_ /= p_.sum()
                    y[r, hq] = p_ @ np.array(vals)
            o = y.reshape(B, nh * hd) @ _unpack(*L["o"]).T
            h = h + self.conv(o, d, L["attn_base"], 1)
            x = self.rms(h, L["post_norm"])
            d2 = x @ _h(L["mlp_kproj"]).T
            xc = self.conv(x, d2, L["mlp_base"], 0)
            gt = xc @ _unpack(*L["gate"]).T
            up = xc @ _unpack(*L["up"]).T
            m = gt / (1 + np.exp(-gt)) * up
            dn = m @ _unpack(*L["down"]).T
            h = h + self.conv(dn, d2, L["mlp_base"], 1)
        x = self.rms(h, w["norm"])
        logits = x[1:k + 1] @ _h(w["head"])[:width].T
        hp = x[1:k + 1] @ _h(w["sel_proj"]).T
        return logits, hp

    def settle(self, taps, pos0):
        g, w = self.g, self.w
        kv, hd = g["kv_heads"], g["head_dim"]
        t = taps.astype(np.float64) @ _h(w["fc"]).T
        t = self.rms(t, w["hidden_norm"])
        K, V = [], []
        for l, L in enumerate(w["layers"]):
            kk = (t @ _unpack(*L["k"]).T).reshape(-1, kv, hd)
            vv = t @ _unpack(*L["v"]).T
            for r in range(kk.shape[0]):
                kk[r] = self.rms(kk[r], L["k_norm"])
                if l not in g["no_rope"]:
                    kk[r] = self.rope(kk[r], pos0 + r)
            K.append(kk.reshape(kk.shape[0], -1))
            V.append(vv)
        return np.array(K), np.array(V)


CASES = [
    dict(windows=[0], no_rope=[], kv_heads=2, length=0, first=0),
    dict(windows=[1], no_rope=[], kv_heads=1, length=9, first=0),
    dict(windows=[3], no_rope=[0], kv_heads=2, length=23, first=5),
    dict(windows=[40], no_rope=[], kv_heads=2, length=31, first=2),
    dict(windows=[0, 4], no_rope=[1], kv_heads=2, length=40, first=0),
]


@pytest.mark.parametrize("case", CASES)
def test_block_matches_bruteforce(orc, case):
    layers = len(case["windows"])
    g = dict(hidden=32, intermediate=64, layers=layers, heads=2, kv_heads=case["kv_heads"],
             head_dim=16, vocab=64, block=4, mask_token=63, conv_group=4, conv_kernel=3,
             selector_rank=8, selector_top=4, n_taps=2, windows=case["windows"],
             no_rope=case["no_rope"], rope_theta=1e4, eps=1e-6)
    w = synth.make_weights(g, seed=21)
    # larger weights so the layers change the rows noticeably
    rows = max(case["length"], 1)
    store = [(k.numpy(), v.numpy()) for k, v in synth.make_store(g, rows, seed=4)]
    first, length = case["first"], case["length"]
    for a in (first + length, first + length + 3, max(first, first + length - 2)):
        ref = orc.Model(g, w).block(store, first, length, 7, a, 3, 60)
        bl, bh = Brute(g, w).block(store, first, length, 7, a, 3, 60)
        np.testing.assert_allclose(ref["logits"], bl, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(ref["hp"], bh, rtol=1e-9, atol=1e-12)


def test_settle_matches_bruteforce(orc):
    g = dict(hidden=32, intermediate=64, layers=2, heads=2, kv_heads=2, head_dim=16, vocab=64,
             block=4, mask_token=63, conv_group=4, conv_kernel=3, selector_rank=8,
             selector_top=4, n_taps=3, windows=[0, 0], no_rope=[1], rope_theta=1e4, eps=1e-6)
    w = synth.make_weights(g, seed=22)
    taps = synth.make_taps(g, 6, seed=3).numpy()
    K, V = orc.Model(g, w).settle(taps, 77)
    bK, bV = Brute(g, w).settle(taps, 77)
    np.testing.assert_allclose(K, bK.astype(np.float32), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(V, bV.astype(np.float32), rtol=1e-6, atol=1e-7)
