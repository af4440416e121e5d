"""Branch-aware gated delta-rule scan over the packed episode DAG (oracle; test
infrastructure only).

Sources: Octopus project page, primitives table: `fork` clones the parent's recurrent
checkpoint at the fork point, and `read_thread` mounts a span into the attention layers
only (recurrent layers skip mounted spans); section "Architecture & Co-Design": the
hybrid backbone interleaves Gated DeltaNet recurrent layers with full-attention layers,
and the packed trainer compiles the recurrent boundary checkpoints of the tree into the
same pass; ia.com.br article: the recurrent layers hold mutable working memory h_B.

The recurrence is the published gated delta rule (Gated Delta Networks, Yang, Kautz and
Hatamizadeh, 2024), per head, with state S (Dv x Dk):

    S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

Readings (the pages give no formulas): a root starts from S = 0; a child starts from its
parent's state just before the parent's own token `fork` (after tokens 0 .. fork-1); a
branch processes only its own tokens, in order; mounts change nothing.  Float64.

The backward (``scan_bwd``) is the gradient of L = sum_t <dO_t, o_t> through the same
recurrence, token by token in reverse (back-propagation through time): the gradient of a
child's initial state is added to its parent's state gradient at the fork offset, since
the child's first state is the parent's state there.  States are recomputed from saved
ones every ``segment`` tokens to bound memory; the arithmetic of every step is the
forward's, so the recomputed states are the forward's bit for bit.
"""

from __future__ import annotations

import numpy as np


def _step(S, q, k, v, a, b):
    """One token for all heads: S [H, Dv, Dk], q, k [H, Dk], v [H, Dv], a, b [H]."""
    Sk = np.einsum("hij,hj->hi", S, k)
    S = a[:, None, None] * (S - b[:, None, None] * Sk[:, :, None] * k[:, None, :]) \
        + b[:, None, None] * v[:, :, None] * k[:, None, :]
    return S, np.einsum("hij,hj->hi", S, q)


def scan(q, k, v, alpha, beta, branches, mounts=None):
    """Outputs ``o [T, H, Dv]`` (float64) and the final state of every branch
    ``[NB, H, Dv, Dk]``.  ``q, k [T, H, Dk]``, ``v [T, H, Dv]``, ``alpha, beta [T, H]``;
    ``mounts`` is accepted and ignored (recurrent layers skip mounted spans)."""
    br = np.asarray(branches).reshape(-1, 4)
    T, H, Dk = q.shape
    Dv = v.shape[2]
    o = np.zeros((T, H, Dv))
    final = np.zeros((br.shape[0], H, Dv, Dk))
    # states[b][r]: state of branch b before its own token r, kept for the offsets its
    # children fork at (parents have lower indices, so they are done first)
    need = [set() for _ in range(br.shape[0])]
    for b, (parent, fork, _, _) in enumerate(br):
        if parent >= 0:
            need[parent].add(int(fork))
    saved = [dict() for _ in range(br.shape[0])]
    for b, (parent, fork, start, L) in enumerate(br):
        S = np.zeros((H, Dv, Dk)) if parent < 0 else saved[parent][int(fork)].copy()
        for r in range(int(L)):
            if r in need[b]:
                saved[b][r] = S.copy()
            t = int(start) + r
            S, o[t] = _step(S, q[t].astype(np.float64), k[t].astype(np.float64),
                            v[t].astype(np.float64), alpha[t].astype(np.float64),
                            beta[t].astype(np.float64))
        if int(L) in need[b]:
            saved[b][int(L)] = S.copy()
        final[b] = S
    return o, final


def path_tokens(branches, b):
    """Packed indices of the tokens a branch's recurrent state has consumed before and
    including its own: the ancestors' own tokens up to each fork, then b's own tokens."""
    br = np.asarray(branches).reshape(-1, 4)
    parent, fork, start, L = (int(x) for x in br[b])
    head = [] if parent < 0 else path_prefix(branches, parent, fork)
    return head + list(range(start, start + L))


def path_prefix(branches, b, upto):
    br = np.asarray(branches).reshape(-1, 4)
    parent, fork, start, L = (int(x) for x in br[b])
    head = [] if parent < 0 else path_prefix(branches, parent, fork)
    return head + list(range(start, start + upto))


def _step_bwd(S_prev, q, k, v, a, b, dS, do):
    """Backward of one token for all heads.  ``S_prev`` is the state before the token,
    ``dS`` the gradient with respect to the state after it from everything later (not
    this token's own output), ``do`` the gradient of this token's output.  Returns the
    gradient with respect to ``S_prev`` and those of ``q, k, v, a, b``.

    With X = S_prev - b (S_prev k) k^T and S = a X + b v k^T, o = S q:
        dq = S^T do,  dS += do q^T,  dv = b dS k,  da = <dS, X>,
        db = <(v - a S_prev k), dS k>,
        dk = b dS^T v - a b (S_prev^T (dS k) + dS^T (S_prev k)),
        dS_prev = a (dS - b (dS k) k^T)."""
    Sk = np.einsum("hij,hj->hi", S_prev, k)
    X = S_prev - b[:, None, None] * Sk[:, :, None] * k[:, None, :]
    S = a[:, None, None] * X + b[:, None, None] * v[:, :, None] * k[:, None, :]
    dq = np.einsum("hij,hi->hj", S, do)
    dS = dS + do[:, :, None] * q[:, None, :]
    dSk = np.einsum("hij,hj->hi", dS, k)
    dv = b[:, None] * dSk
    da = np.einsum("hij,hij->h", dS, X)
    db = np.einsum("hi,hi->h", v - a[:, None] * Sk, dSk)
    dk = b[:, None] * np.einsum("hij,hi->hj", dS, v) - (a * b)[:, None] * (
        np.einsum("hij,hi->hj", S_prev, dSk) + np.einsum("hij,hi->hj", dS, Sk))
    dS_prev = a[:, None, None] * (dS - b[:, None, None] * dSk[:, :, None] * k[:, None, :])
    return dS_prev, dq, dk, dv, da, db


def scan_bwd(q, k, v, alpha, beta, do, branches, mounts=None, segment=256):
    """Gradients ``(dq, dk, dv, dalpha, dbeta)`` (float64, shapes of the inputs) of
    L = sum_t <do_t, o_t> for the outputs of ``scan``; ``mounts`` is ignored."""
    br = np.asarray(branches).reshape(-1, 4)
    T, H, Dk = q.shape
    Dv = v.shape[2]
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, alpha, beta, do = f64(q), f64(k), f64(v), f64(alpha), f64(beta), f64(do)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    da, db = np.zeros_like(alpha), np.zeros_like(beta)
    nb = br.shape[0]
    need = [set() for _ in range(nb)]
    for b, (parent, fork, _, _) in enumerate(br):
        if parent >= 0:
            need[parent].add(int(fork))
    # forward: every branch's initial state and its state at the start of each segment
    init = [None] * nb
    seg_start = [dict() for _ in range(nb)]
    saved = [dict() for _ in range(nb)]
    for b, (parent, fork, start, L) in enumerate(br):
        S = np.zeros((H, Dv, Dk)) if parent < 0 else saved[parent][int(fork)].copy()
        init[b] = S.copy()
        for r in range(int(L)):
            if r % segment == 0:
                seg_start[b][r] = S.copy()
            if r in need[b]:
                saved[b][r] = S.copy()
            t = int(start) + r
            S, _ = _step(S, q[t], k[t], v[t], alpha[t], beta[t])
        if int(L) in need[b]:
            saved[b][int(L)] = S.copy()
    # backward, children (higher indices) before their parents
    handed = [dict() for _ in range(nb)]  # gradient of a child's initial state, by fork
    for b in range(nb - 1, -1, -1):
        parent, fork, start, L = (int(x) for x in br[b])
        dS = handed[b].get(L, np.zeros((H, Dv, Dk)))
        for r0 in range(((L - 1) // segment) * segment if L > 0 else 0, -1, -segment):
            r1 = min(L, r0 + segment)
            states = [seg_start[b][r0]]
            for r in range(r0, r1 - 1):
                t = start + r
                states.append(_step(states[-1], q[t], k[t], v[t], alpha[t], beta[t])[0])
            for r in range(r1 - 1, r0 - 1, -1):
                t = start + r
                dS, dq[t], dk[t], dv[t], da[t], db[t] = _step_bwd(
                    states[r - r0], q[t], k[t], v[t], alpha[t], beta[t], dS, do[t])
                if r in handed[b]:
                    dS = dS + handed[b][r]
        if parent >= 0:
            handed[parent][fork] = handed[parent].get(fork, 0.0) + dS
    return dq, dk, dv, da, db
