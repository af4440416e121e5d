"""Paged mounted decode, float64 (oracle; test infrastructure only).

Serving side of the same DAG (project page, primitives table: ``fork`` shares the
parent's radix KV pages by reference counting, ``read_thread`` mounts a sibling's
pages ``c_A[s_A:e_A)`` zero-copy, ``done`` pins a finished branch's pages so others
can mount them; card "02 · Memory": mounts allocate no new KV pages).  A decode
cursor is a branch whose last own token is the current query.  It attends to
``Ctx`` of that token (dag visibility), each visible token read in place from the
physical page of the branch that owns it:

    token r of branch b  ->  page pages[page_ptr[b] + r // page_size],
                             slot r % page_size

Pools are ``[n_pages, Hkv, page_size, D]``; queries ``[B, Hq, D]`` are the current
tokens' (already rotated) queries.

Extend (prefill of several new tokens per cursor, the step that appends a turn's delta
to a cursor whose earlier context is already in pages): cursor ``c`` adds its branch's
last ``m_c`` own tokens, already written to its pages; each of them attends to ``Ctx``
of its own packed index, so the new tokens see each other causally, and a span mounted
at a reader offset inside the new tokens is seen from that offset on.
"""

from __future__ import annotations

import numpy as np

from . import dag as dagmod


def cursor_tokens(branches, mounts, cursor_branch: int) -> np.ndarray:
    """Packed indices visible to the last own token of ``cursor_branch``."""
    br = np.asarray(branches).reshape(-1, 4)
    T = int(br[:, 3].sum())
    i = int(br[cursor_branch, 2] + br[cursor_branch, 3] - 1)
    row = dagmod.mask_rows(branches, mounts, T, i, i + 1)[0]
    return np.flatnonzero(row)


def physical_slots(branches, page_ptr, pages, page_size, idx, owner=None):
    """Physical ``(page, slot)`` of packed indices ``idx`` through the page table."""
    br = np.asarray(branches).reshape(-1, 4)
    if owner is None:
        owner = dagmod.branch_of(br, int(br[:, 3].sum()))
    b = owner[idx]
    r = idx - br[b, 2]
    page = np.asarray(pages)[np.asarray(page_ptr)[b] + r // page_size]
    return page.astype(np.int64), (r % page_size).astype(np.int64)


def decode(q, k_pool, v_pool, branches, mounts, page_ptr, pages, page_size, cursors,
           scale=None):
    """One-query attention for every cursor.  Returns ``O`` float64 ``[B, Hq, D]`` and
    ``LSE`` float64 ``[B, Hq]``."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    br = np.asarray(branches).reshape(-1, 4)
    owner = dagmod.branch_of(br, int(br[:, 3].sum()))
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for c, b in enumerate(np.asarray(cursors)):
        idx = cursor_tokens(branches, mounts, int(b))
        page, slot = physical_slots(br, page_ptr, pages, page_size, idx, owner)
        K = k_pool[page, :, slot, :].astype(np.float64)  # [n, Hkv, D]
        V = v_pool[page, :, slot, :].astype(np.float64)
        for h in range(Hq):
            kk = h // G
            s = scale * (K[:, kk, :] @ q[c, h].astype(np.float64))
            m = s.max()
            p = np.exp(s - m)
            l = p.sum()
            O[c, h] = (p @ V[:, kk, :]) / l
            LSE[c, h] = m + np.log(l)
    return O, LSE


def unique_tokens(branches, mounts, cursors) -> int:
    """Number of distinct packed tokens any cursor sees (each physical KV token
    counted once however many cursors read it)."""
    br = np.asarray(branches).reshape(-1, 4)
    T = int(br[:, 3].sum())
    seen = np.zeros(T, dtype=bool)
    for b in np.asarray(cursors):
        seen[cursor_tokens(branches, mounts, int(b))] = True
    return int(seen.sum())


def extend(q, k_pool, v_pool, branches, mounts, page_ptr, pages, page_size, cursors, q_ptr,
           scale=None, only=None):
    """Attention of the new tokens of every cursor.  ``q_ptr`` (``[B+1]``) delimits the
    rows of ``q`` (``[n_rows, Hq, D]``) that belong to each cursor: rows
    ``q_ptr[c] .. q_ptr[c+1]-1`` are the last ``m_c = q_ptr[c+1] - q_ptr[c]`` own tokens
    of branch ``cursors[c]``, in order.  Returns ``O`` float64 ``[n_rows, Hq, D]`` and
    ``LSE`` float64 ``[n_rows, Hq]``.  With ``only`` (a set of row indices), only those
    rows are computed; the others are left zero."""
    n_rows, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    br = np.asarray(branches).reshape(-1, 4)
    T = int(br[:, 3].sum())
    owner = dagmod.branch_of(br, T)
    O = np.zeros((n_rows, Hq, D))
    LSE = np.zeros((n_rows, Hq))
    for c, b in enumerate(np.asarray(cursors)):
        r0, r1 = int(q_ptr[c]), int(q_ptr[c + 1])
        m = r1 - r0
        if m == 0:
            continue
        start, L = int(br[b, 2]), int(br[b, 3])
        for j in range(m):
            if only is not None and r0 + j not in only:
                continue
            i = start + L - m + j  # packed index of this new token
            idx = np.flatnonzero(dagmod.mask_rows(branches, mounts, T, i, i + 1)[0])
            page, slot = physical_slots(br, page_ptr, pages, page_size, idx, owner)
            K = k_pool[page, :, slot, :].astype(np.float64)
            V = v_pool[page, :, slot, :].astype(np.float64)
            for h in range(Hq):
                kk = h // G
                s_ = scale * (K[:, kk, :] @ q[r0 + j, h].astype(np.float64))
                mx = s_.max()
                p = np.exp(s_ - mx)
                l = p.sum()
                O[r0 + j, h] = (p @ V[:, kk, :]) / l
                LSE[r0 + j, h] = mx + np.log(l)
    return O, LSE
