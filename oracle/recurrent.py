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
