"""The router margin, as the pages define it — TEST INFRASTRUCTURE ONLY.

From the docs.rs page "cortiq_engine/dflash.rs" (cortiq-engine 0.8.78),
items `Route`, `Route::margin`, `Subspace` and `RouteFit`: a sidecar keeps
two subspaces of the target's rows at the tip, one for the rounds the block
drafter won and one for the rounds the target's own chain won, each a mean
and `rank` basis rows of `hidden` values, both held as f16 and decoded to
f32. For a target row, the margin normalises the row (its norm floored at
1e-12), takes each subspace's reconstruction error of that unit row, and
returns the chain's error minus the block's: above zero the round is the
block's.

The pages name the reconstruction error but do not print it. Reading taken
here (the plainest one the rest supports, "recon-argmin routing" over
fitted subspaces): the Euclidean norm of what is left of u − mean after
removing its components along the basis rows,

    err(u) = ‖ d − Σ_r ⟨d, b_r⟩ b_r ‖₂,   d = u − mean,

which is the distance from u to the affine subspace when the rows are
orthonormal. Whether the norm is squared does not change the margin's sign.

Arithmetic is binary64 on the f16 values decoded exactly.
"""
from __future__ import annotations

import numpy as np


def decode_f16(x) -> np.ndarray:
    """f16 bits (uint16) or f16 values → f64, exactly."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def unit(row) -> np.ndarray:
    """The row over its Euclidean norm, the norm floored at 1e-12."""
    r = np.asarray(row, dtype=np.float64)
    n = max(float(np.sqrt(np.sum(r * r))), 1e-12)
    return r / n


def recon_error(u, mean, basis, rank: int) -> float:
    """‖ d − Bᵀ(B d) ‖₂ with d = u − mean and B the first `rank` rows of
    basis ([rank][hidden], row-major)."""
    u = np.asarray(u, dtype=np.float64)
    d = u - decode_f16(mean)
    if rank == 0:
        return float(np.sqrt(np.sum(d * d)))
    B = decode_f16(basis).reshape(-1, u.shape[0])[:rank]
    c = B @ d
    e = d - B.T @ c
    return float(np.sqrt(np.sum(e * e)))


def margin(row, block, chain) -> float:
    """`Route::margin`: err(chain) − err(block) of the unit row; block and
    chain are (mean, basis, rank) with f16 mean [hidden] and basis
    [rank][hidden]."""
    u = unit(row)
    return recon_error(u, *chain) - recon_error(u, *block)


def margins(rows, block, chain) -> np.ndarray:
    """margin of each row of rows [m][hidden]."""
    return np.array([margin(r, block, chain) for r in np.asarray(rows)], dtype=np.float64)
