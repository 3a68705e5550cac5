"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the definition it pins (docs.rs page "cortiq_engine/dflash.rs",
cortiq-engine 0.8.78) and is chosen so that a plausible slip in the oracle — a
dropped term, a wrong sign, a swapped index, a transposed operand — fails it.
"""
import math
import os

import numpy as np
import pytest
import torch

from block_drafter_settle_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_top_k_golden():
    x, cases = None, {}
    with open(os.path.join(GOLDEN, "top_k_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            if key == "x":
                x = [float(t) for t in rest.split()]
            else:
                k = int(key[2:])
                cases[k] = [(float(p.split(",")[0]), int(p.split(",")[1])) for p in rest.split()]
    return x, cases


# ------------------------------------------------------------------ T1 top_k

def test_top_k_printed_example(orc):
    """`top_k` unit test on the page: values and the tie order are exact."""
    x, cases = _read_top_k_golden()
    for k, want in cases.items():
        val, idx = orc.top_k(x, k)
        assert [(float(v), int(i)) for v, i in zip(val, idx)] == want


def test_top_k_ties_and_order(orc):
    x = np.array([1.0, 3.0, 3.0, 3.0, -2.0, 3.0, 0.0])
    val, idx = orc.top_k(x, 4)
    assert idx.tolist() == [1, 2, 3, 5] and val.tolist() == [3.0] * 4
    rng = np.random.default_rng(1)
    y = rng.integers(-5, 5, 200).astype(float)
    val, idx = orc.top_k(y, 30)
    want = sorted(range(200), key=lambda i: (-y[i], i))[:30]
    assert idx.tolist() == want


# ------------------------------------------------------------------- T2 int4

def _pack(q):
    q = np.asarray(q, np.int64) & 15
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def test_int4_dequant_nibble_order_and_sign(orc):
    """Low nibble = even column; two's complement; one f16 scale per 32 columns."""
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x8F   # col0 = 0xF → −1, col1 = 0x8 → −8
    codes[0, 1] = 0x71   # col2 = 1, col3 = 7
    codes[0, 16] = 0x20  # col32 = 0, col33 = 2
    scale = np.array([[0x3800, 0x4200]], np.uint16)  # 0.5, 3.0
    w = orc.dequant_q4(codes, scale)
    assert w[0, :4].tolist() == [-0.5, -4.0, 0.5, 3.5]
    assert w[0, 32:34].tolist() == [0.0, 6.0]
    assert np.count_nonzero(w) == 5


def test_int4_round_trip_and_error_bound(orc):
    rng = np.random.default_rng(0)
    rows, cols = 40, 256
    # codes and normal-range scales survive dequant → quantise exactly
    q = rng.integers(-7, 8, (rows, cols))
    q[:, ::32] = 7  # each group's largest |q| is 7, so the scale is recovered
    s = (rng.uniform(0.001, 0.05, (rows, cols // 32))).astype(np.float16)
    codes, bits = _pack(q), s.view(np.uint16)
    w = orc.dequant_q4(codes, bits)
    c2, b2 = synth.quantize_int4(torch.tensor(w, dtype=torch.float32))
    assert np.array_equal(c2, codes) and np.array_equal(b2, bits)
    # quantise → dequantise stays within half a step of the weight
    wr = torch.randn(rows, cols) * 0.02
    wr[3, 64:96] = 0.0
    c3, b3 = synth.quantize_int4(wr)
    back = orc.dequant_q4(c3, b3)
    step = np.repeat(b3.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(back - wr.double().numpy()) <= step / 2 * (1 + 2 ** -10) + 1e-12)
    assert np.all(b3[3, 2] == 0) and np.all(back[3, 64:96] == 0)


def test_matvec_against_numpy(orc):
    """The oracle's loops agree with numpy's matmul on the dequantised matrix."""
    rng = np.random.default_rng(2)
    wf = (rng.standard_normal((48, 96)) * 0.1).astype(np.float16)
    x = rng.standard_normal((5, 96))
    y = orc.apply_f16(wf.view(np.uint16), x)
    np.testing.assert_allclose(y, x @ wf.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    codes, sc = synth.quantize_int4(torch.randn(48, 128))
    # an unpack written independently of the oracle's
    lo = (codes & 15).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    qq = np.empty((48, 128), np.int64)
    qq[:, 0::2], qq[:, 1::2] = lo, hi
    qq = np.where(qq >= 8, qq - 16, qq)
    dense = qq * np.repeat(sc.view(np.float16).astype(np.float64), 32, axis=1)
    x2 = rng.standard_normal((3, 128))
    np.testing.assert_allclose(orc.apply_q4(codes, sc, x2), x2 @ dense.T, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------------- T3 rms

def test_rms_constant_row_closed_form(orc):
    w = (1 + np.random.default_rng(3).standard_normal(64) * 0.02).astype(np.float32)
    eps = 1e-6
    for c in (0.25, -3.0, 1e-4):
        y = orc.rms(np.full((1, 64), c), w, eps)
        want = c / math.sqrt(c * c + eps) * w.astype(np.float64)
        np.testing.assert_allclose(y[0], want, rtol=1e-14)


def test_rms_scale_invariance(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 100)) * 10
    w = np.ones(100, np.float32)
    np.testing.assert_allclose(orc.rms(x, w, 1e-6), orc.rms(7.5 * x, w, 1e-6), rtol=1e-8)
    y = orc.rms(x, w, 0.0)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-12)


# ----------------------------------------------------------------- T4 rotary

def test_rotary_position_zero_is_identity(orc):
    x = np.random.default_rng(5).standard_normal((3, 4 * 64))
    y = orc.rotate(x, 4, 64, [0, 0, 0], 1e6)
    assert np.array_equal(x, y)


def test_rotary_sign_and_half_split_pairing(orc):
    """hd = 4: pairs are (x0, x2) and (x1, x3); (1, 0) turns to (cos, sin)."""
    theta = 1e4
    p = 3
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    y = orc.rotate(x, 1, 4, [p], theta)
    a0 = float(np.float32(p) * np.float32(1.0))
    a1 = float(np.float32(p) * np.float32(theta ** -0.5))
    np.testing.assert_allclose(y[0], [math.cos(a0), -math.sin(a1), math.sin(a0), math.cos(a1)],
                               rtol=0, atol=1e-15)


def test_rotary_angle_is_binary32_product(orc):
    """At large positions the angle is the f32 product, not the exact one."""
    hd, theta, p = 128, 1e6, 131071
    inv = orc.inv_freq(theta, hd)
    assert inv.dtype == np.float32
    np.testing.assert_array_equal(inv, np.array([theta ** (-(2.0 * i) / hd) for i in range(64)],
                                                 np.float32))
    x = np.zeros((1, hd))
    x[0, 0] = 1.0
    y = orc.rotate(x, 1, hd, [p], theta)
    ang = float(np.float32(p) * inv[0])
    assert y[0, 0] == math.cos(ang) and y[0, 64] == math.sin(ang)


def test_rotary_norm_and_relative_position(orc):
    rng = np.random.default_rng(6)
    hd, theta = 64, 1e6
    q = rng.standard_normal((1, hd))
    k = rng.standard_normal((1, hd))
    qr = orc.rotate(q, 1, hd, [37], theta)
    np.testing.assert_allclose(np.linalg.norm(qr), np.linalg.norm(q), rtol=1e-14)
    for p, pp, d in ((5, 9, 100), (1000, 17, 2000), (0, 4000, 50)):
        s1 = (orc.rotate(q, 1, hd, [p], theta) * orc.rotate(k, 1, hd, [pp], theta)).sum()
        s2 = (orc.rotate(q, 1, hd, [p + d], theta) * orc.rotate(k, 1, hd, [pp + d], theta)).sum()
        assert abs(s1 - s2) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)


# ------------------------------------------------------------------- T5 conv

def _conv_case(rows=7, hs=16, gs=4, kn=3, seed=7):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, hs))
    d = rng.standard_normal((rows, 2 * kn * (hs // gs)))
    base = rng.standard_normal(2 * kn * hs).astype(np.float32)
    return x, d, base, gs, kn


def test_conv_is_causal(orc):
    x, d, base, gs, kn = _conv_case()
    for stage in (0, 1):
        y = orc.conv(x, d, base, gs, kn, stage)
        for j in range(x.shape[0]):
            x2, d2 = x.copy(), d.copy()
            x2[j] += 1.0
            d2[j] += 1.0
            y2 = orc.conv(x2, d2, base, gs, kn, stage)
            assert np.array_equal(y[:j], y2[:j])
            assert not np.array_equal(y[j], y2[j])


def test_conv_identity_and_shift(orc):
    x, d, base, gs, kn = _conv_case()
    d0 = np.zeros_like(d)
    hs = x.shape[1]
    for stage in (0, 1):
        b = np.zeros((2, kn, hs), np.float32)
        b[stage, 0] = 1.0
        b[1 - stage, :] = 5.0  # the other stage's kernel must not be read
        assert np.array_equal(orc.conv(x, d0, b.ravel(), gs, kn, stage), x)
        b = np.zeros((2, kn, hs), np.float32)
        b[stage, 1] = 1.0
        y = orc.conv(x, d0, b.ravel(), gs, kn, stage)
        assert np.array_equal(y[1:], x[:-1]) and np.all(y[0] == 0)


def test_conv_dynamic_kernel_group_index(orc):
    """d[r][stage][o][g] multiplies channels g·gs … g·gs+gs−1 of row r−o."""
    rows, hs, gs, kn = 5, 12, 3, 2
    G = hs // gs
    x = np.arange(1, rows * hs + 1, dtype=float).reshape(rows, hs)
    d = np.zeros((rows, 2, kn, G))
    d[3, 1, 1, 2] = 2.0   # row 3, stage 1, offset 1, group 2 (channels 6..8)
    d[4, 1, 0, 0] = -1.0  # row 4, stage 1, offset 0, group 0 (channels 0..2)
    y = orc.conv(x, d.reshape(rows, -1), np.zeros(2 * kn * hs, np.float32), gs, kn, 1)
    want = np.zeros_like(x)
    want[3, 6:9] = 2.0 * x[2, 6:9]
    want[4, 0:3] = -1.0 * x[4, 0:3]
    assert np.array_equal(y, want)
    assert np.all(orc.conv(x, d.reshape(rows, -1), np.zeros(2 * kn * hs, np.float32), gs, kn,
                           0) == 0)


# ------------------------------------------------------------- T6/T7 attention

def _attn_case(rows=4, heads=4, kv=2, hd=8, length=30, seed=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, heads * hd))
    k = rng.standard_normal((rows, kv * hd))
    v = rng.standard_normal((rows, kv * hd))
    sk = rng.standard_normal((length, kv * hd)).astype(np.float32)
    sv = rng.standard_normal((length, kv * hd)).astype(np.float32)
    return q, k, v, sk, sv


def test_attention_wide_window_equals_full(orc):
    rows, heads, kv, hd, length, first = 4, 4, 2, 8, 30, 100
    q, k, v, sk, sv = _attn_case(rows, heads, kv, hd, length)
    a = first + length
    full = orc.attention(q, k, v, sk, sv, first, length, a, 0, heads, kv, hd)
    wide = orc.attention(q, k, v, sk, sv, first, length, a, (a - first) + rows, heads, kv, hd)
    assert np.array_equal(full, wide)
    # w = a − first + 1: row 0 (position a) still reaches `first`, row 1 does not
    narrow = orc.attention(q, k, v, sk, sv, first, length, a, a - first + 1, heads, kv, hd)
    assert np.array_equal(narrow[0], full[0])
    assert not np.array_equal(narrow[1], full[1])  # row 1 loses position `first`


@pytest.mark.parametrize("window", [0, 1, 3, 7, 25, 60])
def test_attention_uniform_scores_give_mean_of_visible(orc, window):
    """q = 0 makes every score 0, so each row's output is the plain mean of
    the values it sees: context positions in [max(lo, a+r+1−w), hi) and all
    block rows. This pins the visibility rule and the range arithmetic."""
    rows, heads, kv, hd, length, first = 4, 4, 2, 8, 30, 11
    _, k, v, sk, sv = _attn_case(rows, heads, kv, hd, length)
    q = np.zeros((rows, heads * hd))
    for a in (first + length, first + 20, first + 3, first):
        y = orc.attention(q, k, v, sk, sv, first, length, a, window, heads, kv, hd)
        hi = min(a, first + length)
        for r in range(rows):
            lo_r = first if window == 0 else max(first, a + r + 1 - window)
            ctx = list(range(max(lo_r, first), hi))
            for h in range(heads):
                g = h // (heads // kv)
                vals = [sv[p - first, g * hd:(g + 1) * hd].astype(float) for p in ctx]
                vals += [v[b, g * hd:(g + 1) * hd] for b in range(rows)]
                np.testing.assert_allclose(y[r, h * hd:(h + 1) * hd], np.mean(vals, axis=0),
                                           rtol=1e-13, atol=1e-13)


def test_attention_gqa_head_mapping_and_single_key(orc):
    """q head h reads kv head h // (heads/kv); one visible key returns its value."""
    rows, heads, kv, hd = 1, 4, 2, 4
    q = np.zeros((rows, heads * hd))
    k = np.zeros((rows, kv * hd))
    v = np.concatenate([np.full(hd, 1.0), np.full(hd, 2.0)])[None]
    y = orc.attention(q, k, v, np.zeros((0, kv * hd), np.float32),
                      np.zeros((0, kv * hd), np.float32), 0, 0, 0, 0, heads, kv, hd)
    np.testing.assert_array_equal(y[0].reshape(heads, hd)[:, 0], [1.0, 1.0, 2.0, 2.0])


def test_attention_softmax_two_keys(orc):
    """scale·q·k with scale = hd^−½; a two-key softmax in closed form."""
    hd = 4
    q = np.array([[2.0, 0, 0, 0]])
    k = np.array([[1.0, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0]])
    sk = np.array([[3.0, 0, 0, 0]], np.float32)
    sv = np.array([[0.0, 5.0, 0, 0]], np.float32)
    y = orc.attention(q, k, v, sk, sv, 0, 1, 1, 0, 1, 1, hd)
    s_ctx, s_blk = 2 * 3 / 2.0, 2 * 1 / 2.0
    p_ctx = math.exp(s_ctx) / (math.exp(s_ctx) + math.exp(s_blk))
    np.testing.assert_allclose(y[0], [1 - p_ctx, 5 * p_ctx, 0, 0], rtol=1e-14)


def test_attention_is_not_causal(orc):
    rows, heads, kv, hd, length = 4, 4, 2, 8, 10
    q, k, v, sk, sv = _attn_case(rows, heads, kv, hd, length)
    y = orc.attention(q, k, v, sk, sv, 0, length, length, 0, heads, kv, hd)
    v2 = v.copy()
    v2[rows - 1] += 1.0
    y2 = orc.attention(q, k, v2, sk, sv, 0, length, length, 0, heads, kv, hd)
    assert not np.array_equal(y[0], y2[0])


def test_attention_mha_equals_expanded_gqa(orc):
    rows, heads, kv, hd, length = 3, 4, 2, 8, 12
    q, k, v, sk, sv = _attn_case(rows, heads, kv, hd, length)
    rep = heads // kv

    def expand(a):
        a = a.reshape(a.shape[0], kv, hd)
        return np.repeat(a, rep, axis=1).reshape(a.shape[0], heads * hd)

    g = orc.attention(q, k, v, sk, sv, 0, length, length, 5, heads, kv, hd)
    m = orc.attention(q, expand(k), expand(v), expand(sk).astype(np.float32),
                      expand(sv).astype(np.float32), 0, length, length, 5, heads, heads, hd)
    np.testing.assert_allclose(g, m, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------ whole block and settle

@pytest.fixture(scope="module")
def tiny():
    g = synth.small_geometry(windows=[0, 5], vocab=600, mask_token=599)
    w = synth.make_weights(g, seed=3)
    return g, w


def _store(g, rows, seed=1):
    return [(k.numpy(), v.numpy()) for k, v in synth.make_store(g, rows, seed=seed)]


def test_block_zero_attention_and_mlp_is_head_of_embedding(orc, tiny):
    """With o_proj and down at zero the residual stays the embedding rows, so
    logits = Head · rms(E[mask], norm) for every draft row, hp = S · the same."""
    g, w = tiny
    w = dict(w)
    w["layers"] = [dict(l) for l in w["layers"]]
    for l in w["layers"]:
        for n in ("o", "down"):
            c, s = l[n]
            l[n] = (np.zeros_like(c), np.zeros_like(s))
    m = orc.Model(g, w)
    k, width, anchor = g["block"] - 1, g["vocab"], 17
    out = m.block(_store(g, 20), 0, 20, anchor, 20, k, width)
    E = w["embed"].view(np.float16).astype(np.float64)
    H = w["head"].view(np.float16).astype(np.float64)
    S = w["sel_proj"].view(np.float16).astype(np.float64)
    e = E[g["mask_token"]]
    x = e / math.sqrt((e * e).mean() + float(np.float32(g["eps"]))) * w["norm"].astype(np.float64)
    np.testing.assert_allclose(out["logits"], np.tile(H @ x, (k, 1)), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["hp"], np.tile(S @ x, (k, 1)), rtol=1e-10, atol=1e-12)
    e0 = E[anchor]
    x0 = e0 / math.sqrt((e0 * e0).mean() + float(np.float32(g["eps"]))) * w["norm"]
    np.testing.assert_allclose(out["hidden"][0], x0, rtol=1e-10)


def test_block_no_rope_shift_invariance(orc):
    """Every layer without rotary: moving the context and the anchor by Δ
    changes nothing, bit for bit (positions only enter through rotary and
    the window masks, which move together)."""
    g = synth.small_geometry(windows=[0, 6], no_rope=[0, 1], vocab=300, mask_token=299)
    w = synth.make_weights(g, seed=4)
    m = orc.Model(g, w)
    st = _store(g, 25)
    a = m.block(st, 10, 25, 5, 35, 3, 300)
    b = m.block(st, 10 + 1000, 25, 5, 35 + 1000, 3, 300)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["hp"], b["hp"])
    g2 = synth.small_geometry(windows=[0, 6], no_rope=[], vocab=300, mask_token=299)
    m2 = orc.Model(g2, w)
    c = m2.block(st, 10, 25, 5, 35, 3, 300)
    assert not np.array_equal(a["logits"], c["logits"])  # rotary does enter otherwise


def test_block_window_at_least_context_equals_full(orc):
    g0 = synth.small_geometry(windows=[0, 0], vocab=300, mask_token=299)
    w = synth.make_weights(g0, seed=5)
    st = _store(g0, 40)
    first, length = 3, 40
    a = first + length
    full = orc.Model(g0, w).block(st, first, length, 9, a, 4, 300)
    wide = (a - first) + g0["block"]
    g1 = synth.small_geometry(windows=[wide, wide + 7], vocab=300, mask_token=299)
    win = orc.Model(g1, w).block(st, first, length, 9, a, 4, 300)
    assert np.array_equal(full["logits"], win["logits"])
    g2 = synth.small_geometry(windows=[a - first, 0], vocab=300, mask_token=299)
    narrow = orc.Model(g2, w).block(st, first, length, 9, a, 4, 300)
    assert not np.array_equal(full["logits"], narrow["logits"])


def test_settle_chunking_and_row_independence(orc, tiny):
    g, w = tiny
    m = orc.Model(g, w)
    taps = synth.make_taps(g, 9, seed=2).numpy()
    k_all, v_all = m.settle(taps, 50)
    k_a, v_a = m.settle(taps[:4], 50)
    k_b, v_b = m.settle(taps[4:], 54)
    assert np.array_equal(k_all, np.concatenate([k_a, k_b], axis=1))
    assert np.array_equal(v_all, np.concatenate([v_a, v_b], axis=1))
    k_1, v_1 = m.settle(taps[6:7], 56)
    assert np.array_equal(k_all[:, 6:7], k_1) and np.array_equal(v_all[:, 6:7], v_1)


def test_settle_closed_form_identity_projections(orc):
    """fc picking tap 0, identity-coded Wk/Wv: t = rms(tap0, hidden_norm),
    K = rot(rms(t per head, k_norm), pos), V = t."""
    g = synth.small_geometry(hidden=128, intermediate=128, heads=2, kv_heads=2, head_dim=64,
                             n_taps=2, layers=1, windows=[0])
    w = synth.make_weights(g, seed=6)
    hs, tw = g["hidden"], synth.tap_width(g)
    fc = np.zeros((hs, tw), np.float16)
    fc[np.arange(hs), np.arange(hs)] = 1.0
    w["fc"] = fc.view(np.uint16)
    eye_codes = _pack(np.eye(hs, dtype=np.int64))
    one = np.full((hs, hs // 32), 0x3C00, np.uint16)
    w["layers"][0]["k"] = (eye_codes, one)
    w["layers"][0]["v"] = (eye_codes, one)
    m = orc.Model(g, w)
    taps = synth.make_taps(g, 3, seed=9).numpy()
    K, V = m.settle(taps, 1000)
    eps = float(np.float32(g["eps"]))
    for r in range(3):
        x = taps[r, :hs].astype(np.float64)
        t = x / math.sqrt((x * x).mean() + eps) * w["hidden_norm"]
        np.testing.assert_allclose(V[0, r], t.astype(np.float32), rtol=1e-6)
        kh = t.reshape(2, 64)
        kh = kh / np.sqrt((kh * kh).mean(axis=1, keepdims=True) + eps) * w["layers"][0]["k_norm"]
        inv = np.array([1e6 ** (-(2.0 * i) / 64) for i in range(32)], np.float32)
        ang = (np.float32(1000 + r) * inv).astype(np.float64)
        c, s = np.cos(ang), np.sin(ang)
        rot = np.concatenate([kh[:, :32] * c - kh[:, 32:] * s, kh[:, 32:] * c + kh[:, :32] * s],
                             axis=1)
        np.testing.assert_allclose(K[0, r], rot.ravel().astype(np.float32), rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------- T10 select

def test_select_zero_codebooks_pick_plain_argmax(orc, tiny):
    g, w = tiny
    w = dict(w)
    w["pred_book"] = np.zeros_like(w["pred_book"])
    m = orc.Model(g, w)
    rng = np.random.default_rng(10)
    logits = rng.integers(0, 4, (5, 600)).astype(float)  # many ties
    hp = rng.standard_normal((5, g["selector_rank"]))
    out = m.select(logits, hp, anchor=3)
    want = [int(np.argmax(r)) for r in logits]  # argmax returns the first maximum
    assert out["chosen"].tolist() == want and out["plain"].tolist() == want
    np.testing.assert_array_equal(out["score"], out["unary"])


def test_select_top_one_is_plain(orc):
    g = synth.small_geometry(selector_top=1, vocab=300, mask_token=299)
    w = synth.make_weights(g, seed=11)
    m = orc.Model(g, w)
    rng = np.random.default_rng(11)
    out = m.select(rng.standard_normal((4, 300)), rng.standard_normal((4, 16)) * 50, anchor=1)
    assert np.array_equal(out["chosen"], out["plain"])


def test_select_chain_closed_form(orc):
    """Two rows, rank 2: the predecessor row of the anchor, then of the
    token chosen for row 0, scales the successor rows of the candidates."""
    g = synth.small_geometry(vocab=8, mask_token=7, selector_rank=2, selector_top=2)
    w = synth.make_weights(g, seed=12)
    P = np.zeros((8, 2), np.float16)
    C = np.zeros((8, 2), np.float16)
    P[5] = [1.0, 0.0]     # anchor
    P[2] = [0.0, 2.0]
    C[2] = [3.0, 0.0]
    C[4] = [0.0, 1.0]
    C[6] = [0.0, -1.0]
    w["pred_book"], w["succ_book"] = P.view(np.uint16), C.view(np.uint16)
    m = orc.Model(g, w)
    logits = np.full((2, 8), -5.0)
    logits[0, 4], logits[0, 2] = 1.0, 0.5   # row 0 candidates: 4 (1.0), 2 (0.5)
    logits[1, 6], logits[1, 4] = 2.0, 1.9   # row 1 candidates: 6, 4
    hp = np.array([[1.0, 1.0], [1.0, 0.25]])
    out = m.select(logits, hp, anchor=5)
    # row 0: pc = P[5]⊙hp0 = (1, 0); s(4) = 1 + 0 = 1; s(2) = 0.5 + 3 = 3.5 → 2
    # row 1: pc = P[2]⊙hp1 = (0, 0.5); s(6) = 2 − 0.5 = 1.5; s(4) = 1.9 + 0.5 = 2.4 → 4
    assert out["cand"].tolist() == [[4, 2], [6, 4]]
    np.testing.assert_allclose(out["score"], [[1.0, 3.5], [1.5, 2.4]], rtol=1e-15)
    assert out["chosen"].tolist() == [2, 4] and out["plain"].tolist() == [4, 6]
    forced = m.select(logits, hp, anchor=5, forced_prev=[5, 5])
    # row 1 with prev forced to 5: pc = (1, 0) → s(6) = 2, s(4) = 1.9 → 6
    assert forced["chosen"].tolist() == [2, 6]
