"""Dense masked softmax attention over the explicit DAG visibility mask, float64
(oracle; test infrastructure only).

The packed block-sparse pass of the Octopus trainer (project page, card
"03 · Training": one unpadded 1-D forward-backward pass per tree; ia.com.br
article, section "Crédito contrafactual ...": a single block-sparse attention pass
structured as a prefix tree, with mount edges differentiable end to end) computes
exactly ordinary softmax attention in which query ``i`` attends to the keys of
``Ctx(i)``.  This module writes that definition out:

    S_ij   = scale * <Q_ih, K_jk>            for j in Ctx(i),  k = h // (Hq / Hkv)
    LSE_ih = log sum_j exp(S_ij)
    P_ij   = exp(S_ij - LSE_ih)
    O_ih   = sum_j P_ij V_jk

and, for ``L = sum <dO, O>``,

    Delta_ih = <dO_ih, O_ih>,   dP_ij = <dO_ih, V_jk>,   dS_ij = P_ij (dP_ij - Delta_ih)
    dQ_ih = scale sum_j dS_ij K_jk
    dK_jk = scale sum_{h -> k} sum_i dS_ij Q_ih
    dV_jk = sum_{h -> k} sum_i P_ij dO_ih

In packed indices a shared-prefix key has one dK/dV row that sums the queries of
every branch that sees it, and a mounted key's row also sums its readers' queries:
the prefix is owned once and reader gradients land in the producer's tokens.

Scale defaults to ``1/sqrt(D)`` and the query-head to KV-head map is contiguous
groups (the pages fix neither).  Rows are processed in blocks; for each block the
dense mask rows come from ``dag.mask_rows`` and only the columns some row of the
block sees are gathered.  Blocks run on a thread pool (NumPy releases the GIL) with
BLAS limited to one thread per worker.
"""

from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import dag as dagmod

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover
    threadpool_limits = None


def n_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _blocks(T, rows, block):
    if rows is None:
        return [(lo, min(T, lo + block)) for lo in range(0, T, block)]
    out = []
    for lo, hi in rows:
        for a in range(lo, hi, block):
            out.append((a, min(hi, a + block)))
    return out


def _run(fn, blocks, workers):
    workers = workers or n_workers()
    if workers == 1 or len(blocks) == 1:
        return [fn(b) for b in blocks]
    if threadpool_limits is None:  # pragma: no cover
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, blocks))
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, blocks))


def _block_inputs(branches, mounts, T, lo, hi, k, v):
    M = dagmod.mask_rows(branches, mounts, T, lo, hi)
    cols = np.flatnonzero(M.any(axis=0))
    Mb = M[:, cols]
    kc = np.ascontiguousarray(k[cols].astype(np.float64).transpose(1, 0, 2))  # [Hkv, nk, D]
    kt = np.ascontiguousarray(kc.transpose(0, 2, 1))  # [Hkv, D, nk]
    vc = np.ascontiguousarray(v[cols].astype(np.float64).transpose(1, 0, 2))  # [Hkv, nk, D]
    return Mb, cols, kc, kt, vc


def _probs(qh, kt_k, Mb, scale):
    """Masked softmax of one head over one row block: returns (P, LSE)."""
    S = qh @ kt_k
    S *= scale
    S[~Mb] = -np.inf
    m = S.max(axis=1)
    np.subtract(S, m[:, None], out=S)
    np.exp(S, out=S)
    l = S.sum(axis=1)
    S /= l[:, None]
    return S, m + np.log(l)


def attn_fwd(q, k, v, branches, mounts, scale=None, rows=None, block=256, workers=None):
    """Forward over the rows in ``rows`` (a list of ``(lo, hi)`` ranges; all rows if
    ``None``).  Inputs ``q [T,Hq,D]``, ``k, v [T,Hkv,D]`` of any float dtype.
    Returns ``O`` (float64 ``[T,Hq,D]``, zero outside the requested rows) and ``LSE``
    (float64 ``[Hq,T]``, NaN outside them)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    O = np.zeros((T, Hq, D), dtype=np.float64)
    LSE = np.full((Hq, T), np.nan, dtype=np.float64)

    def one(bl):
        lo, hi = bl
        Mb, cols, kc, kt, vc = _block_inputs(branches, mounts, T, lo, hi, k, v)
        Q = q[lo:hi].astype(np.float64)
        for h in range(Hq):
            kk = h // G
            P, lse = _probs(Q[:, h, :], kt[kk], Mb, scale)
            O[lo:hi, h, :] = P @ vc[kk]
            LSE[h, lo:hi] = lse
        return None

    _run(one, _blocks(T, rows, block), workers)
    return O, LSE


def attn_bwd(q, k, v, do, branches, mounts, scale=None, rows=None, block=256,
             workers=None):
    """Backward of ``L = sum <dO, O>`` restricted to the queries in ``rows`` (all if
    ``None``).  Recomputes the forward of those rows itself (its own float64 ``O``
    gives ``Delta``).  Returns ``dQ`` (float64 ``[T,Hq,D]``, zero outside ``rows``),
    ``dK``, ``dV`` (float64 ``[T,Hkv,D]``: the contributions of the requested
    queries, i.e. the full gradient when ``rows`` is ``None``)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    dQ = np.zeros((T, Hq, D), dtype=np.float64)
    dK = np.zeros((T, Hkv, D), dtype=np.float64)
    dV = np.zeros((T, Hkv, D), dtype=np.float64)
    lock = threading.Lock()

    def one(bl):
        lo, hi = bl
        Mb, cols, kc, kt, vc = _block_inputs(branches, mounts, T, lo, hi, k, v)
        Q = q[lo:hi].astype(np.float64)
        dO = do[lo:hi].astype(np.float64)
        dk = np.zeros((Hkv, cols.size, D))
        dv = np.zeros((Hkv, cols.size, D))
        for h in range(Hq):
            kk = h // G
            P, _ = _probs(Q[:, h, :], kt[kk], Mb, scale)
            Oh = P @ vc[kk]
            delta = np.einsum("id,id->i", dO[:, h, :], Oh)
            dP = dO[:, h, :] @ vc[kk].T
            dS = P * (dP - delta[:, None])
            dQ[lo:hi, h, :] = scale * (dS @ kc[kk])
            dk[kk] += scale * (dS.T @ Q[:, h, :])
            dv[kk] += P.T @ dO[:, h, :]
        with lock:
            dK[cols] += dk.transpose(1, 0, 2)
            dV[cols] += dv.transpose(1, 0, 2)
        return None

    _run(one, _blocks(T, rows, block), workers)
    return dQ, dK, dV


def useful_pairs(branches, mounts, T, rows=None, block=2048) -> int:
    """Number of visible (query, key) pairs among the requested rows (nnz)."""
    total = 0
    for lo, hi in _blocks(T, rows, block):
        total += int(dagmod.mask_rows(branches, mounts, T, lo, hi).sum())
    return total
