"""Seeded tensor draws for the attention and decode workloads.

Values are drawn in float32 from the caller's generator, optionally rotated with
rotate-half RoPE (base 10000, computed in float64) at positions the caller supplies,
then rounded once to the storage precision.  bfloat16 values are returned as float32
arrays holding exactly representable bf16 numbers, so every consumer (the float64
oracle and the GPU path) sees identical inputs.
"""

from __future__ import annotations

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and return the
    16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array of the bfloat16 values nearest to ``x`` (ties to even)."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
                chunk: int = 8192) -> np.ndarray:
    """Rotate-half RoPE over the last axis of ``x [T, H, D]`` at integer positions
    ``pos [T]``: pairs ``(x_i, x_{i+D/2})`` turn by ``pos * base^(-2i/D)``.  Done in
    float64 in row chunks; returns float32."""
    T, H, D = x.shape
    half = D // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / D)
    out = np.empty((T, H, D), dtype=np.float32)
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        ang = pos[a:b].astype(np.float64)[:, None] * inv[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        x1 = x[a:b, :, :half].astype(np.float64)
        x2 = x[a:b, :, half:].astype(np.float64)
        out[a:b, :, :half] = x1 * c - x2 * s
        out[a:b, :, half:] = x2 * c + x1 * s
    return out


def _normal(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def draw_attention_inputs(rng: np.random.Generator, T: int, Hq: int, Hkv: int, D: int,
                          pos: np.ndarray | None, dtype: str = "bf16", std: float = 0.5,
                          with_dout: bool = False, dout_std: float = 1.0):
    """Q ``[T,Hq,D]``, K and V ``[T,Hkv,D]`` ~ N(0, std^2) in that draw order, then dO
    ``[T,Hq,D]`` ~ N(0, dout_std^2) if asked.  Q and K are RoPE-rotated at ``pos``
    when it is given.  Values are rounded to ``dtype`` ("bf16" or "fp32")."""
    q = _normal(rng, (T, Hq, D), std)
    k = _normal(rng, (T, Hkv, D), std)
    v = _normal(rng, (T, Hkv, D), std)
    do = _normal(rng, (T, Hq, D), dout_std) if with_dout else None
    if pos is not None:
        q = rope_rotate(q, pos)
        k = rope_rotate(k, pos)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
        if do is not None:
            do = round_bf16(do)
    elif dtype != "fp32":
        raise ValueError(dtype)
    out = {"q": q, "k": k, "v": v}
    if do is not None:
        out["do"] = do
    return out


def draw_decode_inputs(rng: np.random.Generator, B: int, Hq: int, Hkv: int, D: int,
                       n_pages: int, page_size: int, std: float = 0.5,
                       dtype: str = "bf16"):
    """Decode queries ``[B,Hq,D]`` and K/V pools ``[n_pages,Hkv,page_size,D]``, i.i.d.
    N(0, std^2), rounded to ``dtype``."""
    q = _normal(rng, (B, Hq, D), std)
    kp = _normal(rng, (n_pages, Hkv, page_size, D), std)
    vp = _normal(rng, (n_pages, Hkv, page_size, D), std)
    if dtype == "bf16":
        q, kp, vp = round_bf16(q), round_bf16(kp), round_bf16(vp)
    return {"q": q, "k_pool": kp, "v_pool": vp}


def draw_extend_inputs(rng: np.random.Generator, n_rows: int, Hq: int, Hkv: int, D: int,
                       n_pages: int, page_size: int, std: float = 0.5,
                       dtype: str = "bf16"):
    """Extend queries ``[n_rows,Hq,D]`` (the new tokens of all cursors, cursor by cursor)
    and K/V pools ``[n_pages,Hkv,page_size,D]``, i.i.d. N(0, std^2), rounded to
    ``dtype``."""
    q = _normal(rng, (n_rows, Hq, D), std)
    kp = _normal(rng, (n_pages, Hkv, page_size, D), std)
    vp = _normal(rng, (n_pages, Hkv, page_size, D), std)
    if dtype == "bf16":
        q, kp, vp = round_bf16(q), round_bf16(kp), round_bf16(vp)
    return {"q": q, "k_pool": kp, "v_pool": vp}


def draw_scan_inputs(rng: np.random.Generator, T: int, H: int, D: int = 128,
                     dtype: str = "bf16"):
    """Recurrent-layer inputs: q and k unit vectors per (token, head) (the layer
    normalises them before the scan), v ~ N(0, 0.25), gates alpha in [0.9, 1) and step
    sizes beta in [0.05, 0.95), float32."""
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, H, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = 0.5 * rng.standard_normal((T, H, D))
    alpha = rng.uniform(0.9, 1.0, size=(T, H)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, size=(T, H)).astype(np.float32)
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}
