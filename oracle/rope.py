"""Rotary position embedding at the episode DAG's positions (oracle; test
infrastructure only).

Sources: Octopus project page, card "02 · Memory": a mounted key keeps the position it
was written at (mounts are rotation-free) and a reader's positions jump to
max(p_B, e_A + 1), so positions only move forward; ia.com.br article, section "Memória
associativa versus memória de trabalho": the same rule.  ``oracle.dag.positions``
computes those positions; this module applies them.

Reading (the pages name no RoPE variant): rotate-half pairs ``(x_i, x_{i+D/2})`` turn by
the angle ``p * base^(-2i/D)``, base 10000, in float64.  The rotation is orthogonal, so
the gradient with respect to an unrotated input is the gradient with respect to the
rotated one turned back by the same angle.
"""

from __future__ import annotations

import numpy as np

from . import attention as att
from . import dag as dagmod


def rotate(x, pos, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """``x [T, H, D]`` turned pairwise at integer positions ``pos [T]`` (float64); with
    ``inverse`` by the opposite angle."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attn_fwd(q, k, v, branches, mounts, base: float = 10000.0, **kw):
    """Packed forward with Q and K given unrotated: each is turned at its token's DAG
    position first."""
    pos = dagmod.positions(branches, mounts)
    return att.attn_fwd(rotate(q, pos, base), rotate(k, pos, base), v, branches, mounts, **kw)


def attn_bwd(q, k, v, do, branches, mounts, base: float = 10000.0, **kw):
    """Gradients with respect to the unrotated Q and K (and V)."""
    pos = dagmod.positions(branches, mounts)
    dq, dk, dv = att.attn_bwd(rotate(q, pos, base), rotate(k, pos, base), v, do, branches,
                              mounts, **kw)
    return rotate(dq, pos, base, inverse=True), rotate(dk, pos, base, inverse=True), dv
