"""Seeded synthetic sidecars, tap rows and context stores.

This module only draws inputs: it holds none of the drafter's arithmetic and
is shared by the tests, the benchmark and the oracle's callers alike. Every
tensor comes from its own generator, seeded from (seed, tensor name), so a
tensor does not change when another one is added.

Recipe (the pages give only the shapes, so the values follow the usual
initialisation of such a drafter):
  - every matrix, base kernel, codebook, embedding and head: N(0, 0.02);
  - norm gains: 1 + N(0, 0.02), a unit gain with a jitter that shows a
    misindexed gain;
  - q, k, v, o, gate, up, down: quantised to symmetric int4 with one f16
    scale per 32 columns (`quantize_int4`); fc, the kernel projections, the
    selector projection, the embedding, the head and both codebooks: f16;
    norm gains and base kernels: f32;
  - tap rows: N(0, 1) f32, optionally with a fixed set of channels scaled
    (1 % of the tap width, x20, for the settle-bound workload);
  - context stores for block-only tests: N(0, 1) f32 keys and values;
  - router subspaces (`make_subspace`): an orthonormal basis of `rank` rows
    (the Q factor of an N(0, 1) [hidden][rank] matrix, rows of its
    transpose) and a mean of N(0, 0.25/hidden) values (norm about 0.5), both
    rounded to f16 as a sidecar holds them; target rows (`make_route_rows`):
    N(0, 1), or, for a share of them, a point of a given subspace near the
    unit sphere (its mean plus N(0, 0.75/rank) coordinates along its basis
    rows) plus N(0, noise) jitter.

Weight preparation (`quantize_int4`) is the offline conversion the pages
leave to their converter: scale = f16(max|w| / 7) per 32-column group,
code = clamp(round_half_even(w / scale), -8, 7), an all-zero group (or one
whose scale rounds to zero) giving scale 0 and codes 0. Codes are packed two
per byte, the even column in the low nibble.
"""
from __future__ import annotations

import copy
import math
import zlib

import numpy as np
import torch

# --------------------------------------------------------------- geometries

_BASE = dict(conv_group=8, conv_kernel=4, selector_rank=64, selector_top=16,
             rope_theta=1e6, eps=1e-6)

# Sidecar shapes: a tiny fp32 sidecar, a Qwen3-4B-shaped one, the 27B-target
# shape the pages' comments describe (5 taps of hidden 5120 = 100 KB f32 a
# row), and its long-context variant.
GEOMETRIES = {
    "tiny": dict(hidden=256, intermediate=768, layers=2, heads=4, kv_heads=2, head_dim=64,
                 vocab=4096, block=8, mask_token=4095, conv_group=4, conv_kernel=4,
                 selector_rank=16, selector_top=8, n_taps=3, windows=[0, 0], no_rope=[],
                 rope_theta=1e6, eps=1e-6),
    "qwen3_4b": dict(_BASE, hidden=2560, intermediate=9728, layers=5, heads=32, kv_heads=8,
                     head_dim=128, vocab=151936, block=16, mask_token=151935, n_taps=5,
                     windows=[0] * 5, no_rope=[]),
    "t27b": dict(_BASE, hidden=5120, intermediate=17408, layers=5, heads=32, kv_heads=8,
                 head_dim=128, vocab=248320, block=16, mask_token=248319, n_taps=5,
                 windows=[2048, 2048, 2048, 2048, 0], no_rope=[4]),
    "t27b_long": dict(_BASE, hidden=5120, intermediate=17408, layers=5, heads=32, kv_heads=8,
                      head_dim=128, vocab=262144, block=16, mask_token=262143, n_taps=5,
                      windows=[0] * 5, no_rope=[4], selector_rank=128, selector_top=32),
}


def geometry(name: str, **over) -> dict:
    g = copy.deepcopy(GEOMETRIES[name])
    g.update(over)
    return g


def small_geometry(**over) -> dict:
    """A few-tile geometry with a ragged head (vocab not a multiple of 16·4)."""
    g = dict(hidden=256, intermediate=384, layers=2, heads=4, kv_heads=2, head_dim=64,
             vocab=1000, block=8, mask_token=999, conv_group=4, conv_kernel=4,
             selector_rank=16, selector_top=8, n_taps=2, windows=[0, 0], no_rope=[],
             rope_theta=1e6, eps=1e-6)
    g.update(over)
    return g


def tap_width(g: dict) -> int:
    return g["n_taps"] * g["hidden"]


def rotary_flags(g: dict) -> list:
    return [0 if l in g["no_rope"] else 1 for l in range(g["layers"])]


# ------------------------------------------------------------------ drawing

def _seed(seed: int, name: str) -> int:
    return (seed * 1_000_003 + zlib.crc32(name.encode())) % (2 ** 62)


def _normal(seed: int, name: str, shape, std: float, device) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed(seed, name))
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std


def _f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float16).view(torch.int16).cpu().numpy().view(np.uint16)


def quantize_int4(w: torch.Tensor):
    """Symmetric int4 per 32 columns (module docstring). Returns
    (codes uint8 [rows][cols/2], scales f16 bits uint16 [rows][cols/32])."""
    rows, cols = w.shape
    assert cols % 32 == 0
    grp = w.reshape(rows, cols // 32, 32)
    scale = (grp.abs().amax(dim=2) / 7.0).to(torch.float16)
    sf = scale.float().unsqueeze(2)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.where(sf > 0, torch.round(grp / safe), torch.zeros_like(grp)).clamp_(-8, 7)
    q = q.to(torch.int16).reshape(rows, cols // 2, 2) & 15
    packed = (q[..., 0] | (q[..., 1] << 4)).to(torch.uint8)
    return packed.cpu().numpy(), scale.view(torch.int16).cpu().numpy().view(np.uint16)


def make_weights(g: dict, seed: int = 0, device="cpu") -> dict:
    """A synthetic sidecar of geometry g: numpy arrays on the host."""
    hs, ffn = g["hidden"], g["intermediate"]
    qd, kd = g["heads"] * g["head_dim"], g["kv_heads"] * g["head_dim"]
    hd, kn, gs = g["head_dim"], g["conv_kernel"], g["conv_group"]
    P = 2 * kn * (hs // gs)
    V, rank, tw = g["vocab"], g["selector_rank"], tap_width(g)
    std = 0.02

    def mat16(name, rows, cols):
        return _f16_bits(_normal(seed, name, (rows, cols), std, device))

    def gain(name, n):
        return (1.0 + _normal(seed, name, (n,), std, device)).cpu().numpy()

    def vec(name, n):
        return _normal(seed, name, (n,), std, device).cpu().numpy()

    def q4(name, rows, cols):
        return quantize_int4(_normal(seed, name, (rows, cols), std, device))

    w = {
        "fc": mat16("fc.weight", hs, tw),
        "hidden_norm": gain("hidden_norm.weight", hs),
        "norm": gain("norm.weight", hs),
        "sel_proj": mat16("candidate_selector.hidden_projection.weight", rank, hs),
        "pred_book": mat16("candidate_selector.predecessor_codebook", V, rank),
        "succ_book": mat16("candidate_selector.successor_codebook", V, rank),
        "embed": mat16("embed_tokens.weight", V, hs),
        "head": mat16("lm_head.weight", V, hs),
        "layers": [],
    }
    for l in range(g["layers"]):
        p = f"layers.{l}."
        w["layers"].append({
            "in_norm": gain(p + "input_layernorm.weight", hs),
            "post_norm": gain(p + "post_attention_layernorm.weight", hs),
            "q_norm": gain(p + "self_attn.q_norm.weight", hd),
            "k_norm": gain(p + "self_attn.k_norm.weight", hd),
            "attn_base": vec(p + "attention_conv.base_kernel", 2 * kn * hs),
            "mlp_base": vec(p + "mlp_conv.base_kernel", 2 * kn * hs),
            "attn_kproj": mat16(p + "attention_conv.kernel_projection.weight", P, hs),
            "mlp_kproj": mat16(p + "mlp_conv.kernel_projection.weight", P, hs),
            "q": q4(p + "self_attn.q_proj.weight", qd, hs),
            "k": q4(p + "self_attn.k_proj.weight", kd, hs),
            "v": q4(p + "self_attn.v_proj.weight", kd, hs),
            "o": q4(p + "self_attn.o_proj.weight", hs, qd),
            "gate": q4(p + "mlp.gate_proj.weight", ffn, hs),
            "up": q4(p + "mlp.up_proj.weight", ffn, hs),
            "down": q4(p + "mlp.down_proj.weight", hs, ffn),
        })
    return w


def make_taps(g: dict, n: int, seed: int = 0, name: str = "taps", outliers: bool = False,
              device="cpu") -> torch.Tensor:
    """n joined tap rows, f32 [n][tap width] on `device`."""
    tw = tap_width(g)
    x = _normal(seed, name, (n, tw), 1.0, device)
    if outliers:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(_seed(seed, "outlier_channels"))
        chans = torch.randperm(tw, generator=gen)[: math.ceil(0.01 * tw)].to(x.device)
        x[:, chans] *= 20.0
    return x


def make_store(g: dict, rows: int, seed: int = 0, device="cpu"):
    """A synthetic context store: per layer (K, V) f32 [rows][kv][hd]."""
    kd = g["kv_heads"] * g["head_dim"]
    out = []
    for l in range(g["layers"]):
        k = _normal(seed, f"store.{l}.k", (rows, kd), 1.0, device)
        v = _normal(seed, f"store.{l}.v", (rows, kd), 1.0, device)
        out.append((k, v))
    return out


def uniform_tokens(g: dict, n: int, seed: int = 0, name: str = "anchors") -> list:
    gen = torch.Generator(device="cpu")
    gen.manual_seed(_seed(seed, name))
    return torch.randint(0, g["vocab"], (n,), generator=gen).tolist()


def make_subspace(hidden: int, rank: int, seed: int = 0, name: str = "route.block"):
    """A router subspace as a sidecar holds it: (mean f16 [hidden], basis f16
    [rank][hidden], rank), torch float16 on the CPU."""
    mean = _normal(seed, name + ".mean", (hidden,), 0.5 / math.sqrt(hidden), "cpu")
    if rank:
        a = _normal(seed, name + ".basis", (hidden, rank), 1.0, "cpu").double()
        q, _ = torch.linalg.qr(a)
        basis = q.T.contiguous().float()
    else:
        basis = torch.zeros(0, hidden)
    return mean.to(torch.float16), basis.to(torch.float16), rank


def make_route_rows(hidden: int, m: int, seed: int = 0, near=None, share: float = 0.0,
                    noise: float = 0.01, name: str = "route.rows") -> torch.Tensor:
    """m target rows f32 [m][hidden]: N(0, 1); the first round(share·m) of
    them instead a point of subspace `near` (its mean plus N(0, 0.75/rank)
    coordinates along its basis rows) plus N(0, noise) jitter."""
    x = _normal(seed, name, (m, hidden), 1.0, "cpu")
    k = int(round(share * m))
    if near is not None and k:
        mean, basis, rank = near
        coef = _normal(seed, name + ".coef", (k, rank), math.sqrt(0.75 / max(rank, 1)), "cpu")
        jit = _normal(seed, name + ".jitter", (k, hidden), noise, "cpu")
        x[:k] = mean.float() + coef @ basis.float() + jit
    return x

