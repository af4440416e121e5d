"""Episode DAG semantics for one packed tree (oracle; test infrastructure only).

Sources (the Octopus pages):

* project page shatianming5.github.io/octopus, section "Architecture & Co-Design":
  the episode is a cursor-addressed DAG ``G = (V, E_tree, E_mount)``; the primitives
  table says ``fork`` shares the parent's radix KV prefix and ``read_thread`` mounts
  a sibling span ``c_A[s_A:e_A)`` into the attention layers; card "02 · Memory"
  gives the rotation-free monotonic position rule ``s(c'_B) = max(p_B, e_A + 1)``;
  card "03 · Training" packs every branch of a tree into one unpadded 1-D pass in
  which a shared prefix is owned once.
* ia.com.br article, section "Memória associativa versus memória de trabalho": the
  same position rule; section "Anatomia de um pensamento ramificado ...": a child
  branch is an O(1) view over the parent's pages.
* rit.work blog, section on branches sharing the prefix: a branch uses the prefix
  pages until it appends its own history; mounted positions only move forward.

Readings where the pages are silent (each one is listed in the design notes):

* ``fork`` is an offset into the parent's own tokens; the child sees the parent's
  tokens before it plus everything the parent saw at that offset.
* ``s, e`` of a mount are producer-local, half-open; ``rpos`` is reader-local: the
  reader's own tokens at offsets ``>= rpos`` see the span.
* visibility is a set: a key mounted twice, or mounted while already visible, is one
  key.  A query always sees itself.
* ``e_A`` in the jump rule is the span's exclusive end expressed in positions; the
  literal ``+1`` is kept (one position is left unused).  ``p_B`` is the position the
  reader's token would have had without this mount.  Parity unpinned for this
  ``+1``: positions only feed the RoPE pre-rotation of the inputs, never the mask.

Tables: ``branches int[NB,4] (parent, fork, start, len)``, ``mounts int[NM,5]
(reader, rpos, producer, s, e)``; ``g(b, r) = start_b + r`` is the packed index of
branch ``b``'s own token ``r``.
"""

from __future__ import annotations

import numpy as np


class DagError(ValueError):
    """``code`` is ``"EINVAL"`` for a malformed table, ``"ECYCLE"`` for a position
    dependency cycle."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _rows(branches, mounts):
    br = [tuple(int(x) for x in row) for row in np.asarray(branches).reshape(-1, 4)]
    mt = [tuple(int(x) for x in row) for row in np.asarray(mounts).reshape(-1, 5)]
    return br, mt


def validate(branches, mounts, T: int) -> None:
    """Reject malformed tables (``DagError('EINVAL')``): row 0 is a root
    (``parent = -1``, ``fork = 0``); any later row is a root too or has a parent of
    lower index with ``0 <= fork <= len(parent)``; ``len >= 1``; the branch spans
    tile ``[0, T)`` without gap or overlap; every mount has ``reader != producer``,
    both in the same tree, ``0 <= rpos <= len(reader)`` and
    ``0 <= s < e <= len(producer)``.

    Several roots are a forest: independent trees packed into one stream (a training
    step batches several episodes, card "03 · Training").  Reading: nothing in one
    tree sees another, so a mount across trees is rejected."""
    br, mt = _rows(branches, mounts)
    if len(br) < 1:
        raise DagError("EINVAL", "no branches")
    tree = []
    for b, (parent, fork, start, length) in enumerate(br):
        if length < 1:
            raise DagError("EINVAL", f"branch {b}: len < 1")
        if parent == -1:
            if fork != 0:
                raise DagError("EINVAL", f"branch {b}: a root must have fork 0")
            tree.append(b)
        else:
            if not 0 <= parent < b:
                raise DagError("EINVAL", f"branch {b}: parent must be -1 or a lower index")
            if not 0 <= fork <= br[parent][3]:
                raise DagError("EINVAL", f"branch {b}: fork outside the parent")
            tree.append(tree[parent])
    covered = np.zeros(T, dtype=np.int64)
    for b, (_, _, start, length) in enumerate(br):
        if start < 0 or start + length > T:
            raise DagError("EINVAL", f"branch {b}: span outside [0, T)")
        covered[start:start + length] += 1
    if T < 1 or not np.all(covered == 1):
        raise DagError("EINVAL", "branch spans do not tile [0, T) exactly")
    for i, (reader, rpos, producer, s, e) in enumerate(mt):
        if not (0 <= reader < len(br) and 0 <= producer < len(br)):
            raise DagError("EINVAL", f"mount {i}: branch index out of range")
        if reader == producer:
            raise DagError("EINVAL", f"mount {i}: reader == producer")
        if not 0 <= rpos <= br[reader][3]:
            raise DagError("EINVAL", f"mount {i}: rpos outside the reader")
        if not 0 <= s < e <= br[producer][3]:
            raise DagError("EINVAL", f"mount {i}: span outside the producer")
        if tree[reader] != tree[producer]:
            raise DagError("EINVAL", f"mount {i}: producer belongs to another tree")


# --------------------------------------------------------------------------------------
# Positions.
# --------------------------------------------------------------------------------------

def branch_positions(branches, mounts) -> list:
    """``[x_b(0), ..., x_b(len_b)]`` for every branch ``b``, where

        x_b(r) = max( {base_b if r == 0 else x_b(r-1) + 1}
                      ∪ {E_m + 1 : reader_m = b, rpos_m = r} )
        base_root = 0,  base_b = x_parent(fork_b),
        E_m = x_producer(e_m - 1) + 1   (the span's exclusive end, in positions)

    i.e. a token is one past its predecessor unless a mount issued just before it
    pushes it to ``max(p_B, e_A + 1)``; ``x_b(len_b)`` is the branch's next
    position.  Evaluated by memoised recursion over (branch, offset); a request for
    an offset of a branch that is itself being extended is a dependency cycle
    (``DagError('ECYCLE')``).  Parity of the ``+1`` gap is unpinned (see the module
    docstring)."""
    br, mt = _rows(branches, mounts)
    at = [dict() for _ in br]
    for (reader, rpos, producer, s, e) in mt:
        at[reader].setdefault(rpos, []).append((producer, e))
    xs = [[] for _ in br]
    busy = [False] * len(br)

    def get(b, r):
        if r < len(xs[b]):
            return xs[b][r]
        if busy[b]:
            raise DagError("ECYCLE", f"position of branch {b} offset {r} depends on itself")
        busy[b] = True
        parent, fork, _, _ = br[b]
        while len(xs[b]) <= r:
            k = len(xs[b])
            if k == 0:
                cands = [0 if parent < 0 else get(parent, fork)]
            else:
                cands = [xs[b][k - 1] + 1]
            for producer, e in at[b].get(k, []):
                E = get(producer, e - 1) + 1
                cands.append(E + 1)
            xs[b].append(max(cands))
        busy[b] = False
        return xs[b][r]

    for b in range(len(br)):
        get(b, br[b][3])
    return xs


def positions(branches, mounts) -> np.ndarray:
    """Position of every packed token: ``pos(g(b, r)) = x_b(r)`` (see
    ``branch_positions``)."""
    br, _ = _rows(branches, mounts)
    xs = branch_positions(branches, mounts)
    T = sum(row[3] for row in br)
    pos = np.zeros(T, dtype=np.int64)
    for b, (_, _, start, length) in enumerate(br):
        pos[start:start + length] = xs[b][:length]
    return pos


# --------------------------------------------------------------------------------------
# Visibility: recursive set definition (tiny inputs) and dense mask rows.
# --------------------------------------------------------------------------------------

def context(branches, mounts, b: int, r: int) -> set:
    """``A(b, r)``, the packed indices visible to anything branch ``b`` emits at own
    offset ``r`` (``0 <= r <= len_b``), excluding that token itself:

        A(b, r) = H(b) ∪ {g(b, r') : r' < r}
                  ∪ ⋃_{m: reader_m = b, rpos_m <= r} {g(producer_m, t) : s_m <= t < e_m}
        H(root) = ∅,  H(b) = A(parent_b, fork_b).

    Python sets; meant for small DAGs."""
    br, mt = _rows(branches, mounts)
    parent, fork, start, _ = br[b]
    out = set() if parent < 0 else context(branches, mounts, parent, fork)
    out |= set(range(start, start + r))
    for (reader, rpos, producer, s, e) in mt:
        if reader == b and rpos <= r:
            ps = br[producer][2]
            out |= set(range(ps + s, ps + e))
    return out


def visible(branches, mounts, i: int) -> set:
    """``Ctx(i) = A(b, r) ∪ {i}`` for the packed token ``i = g(b, r)``."""
    br, _ = _rows(branches, mounts)
    for b, (_, _, start, length) in enumerate(br):
        if start <= i < start + length:
            return context(branches, mounts, b, i - start) | {i}
    raise IndexError(i)


def _ancestor_vector(br, mt, b: int, T: int) -> np.ndarray:
    """Boolean vector of ``H(b)`` (what branch ``b`` inherits at its fork)."""
    parent, fork, _, _ = br[b]
    h = np.zeros(T, dtype=bool)
    if parent < 0:
        return h
    h |= _ancestor_vector(br, mt, parent, T)
    ps = br[parent][2]
    h[ps:ps + fork] = True
    for (reader, rpos, producer, s, e) in mt:
        if reader == parent and rpos <= fork:
            qs = br[producer][2]
            h[qs + s:qs + e] = True
    return h


def mask_rows(branches, mounts, T: int, row_lo: int, row_hi: int) -> np.ndarray:
    """Dense boolean rows ``M[i, j] = [j ∈ Ctx(i)]`` for ``row_lo <= i < row_hi``,
    built straight from the definition of ``Ctx``: the inherited set ``H(b)``, the
    branch's own tokens up to and including the query, and every span mounted by the
    branch at an offset not after the query's."""
    br, mt = _rows(branches, mounts)
    M = np.zeros((row_hi - row_lo, T), dtype=bool)
    for b, (_, _, start, length) in enumerate(br):
        lo = max(row_lo, start)
        hi = min(row_hi, start + length)
        if lo >= hi:
            continue
        rows = np.arange(lo, hi)
        r = rows - start
        blk = M[lo - row_lo:hi - row_lo]
        blk |= _ancestor_vector(br, mt, b, T)[None, :]
        own = np.arange(start, start + length)
        blk[:, start:start + length] |= own[None, :] <= rows[:, None]
        for (reader, rpos, producer, s, e) in mt:
            if reader == b:
                qs = br[producer][2]
                blk[r >= rpos, qs + s:qs + e] = True
    return M


def mask(branches, mounts, T: int) -> np.ndarray:
    """The whole ``T x T`` visibility matrix (small ``T`` only)."""
    return mask_rows(branches, mounts, T, 0, T)


def row_counts(branches, mounts, T: int, block: int = 2048) -> np.ndarray:
    """``|Ctx(i)|`` for every row, from the dense rows in blocks."""
    out = np.zeros(T, dtype=np.int64)
    for lo in range(0, T, block):
        hi = min(T, lo + block)
        out[lo:hi] = mask_rows(branches, mounts, T, lo, hi).sum(axis=1)
    return out


# --------------------------------------------------------------------------------------
# Second formulation: flattened root-to-branch paths.
# --------------------------------------------------------------------------------------

def flatten_path(branches, mounts, b: int) -> list:
    """``Seq(b)``: the packed indices a single flat transcript of branch ``b`` would
    hold, in order.  For each own offset ``r = 0 .. len_b`` first the spans of the
    mounts the branch issued at ``rpos = r`` (table order), then, if ``r < len_b``,
    the branch's own token ``g(b, r)``.  A child's sequence starts with the part of
    its parent's sequence emitted before the parent's own token ``fork`` (including
    spans mounted at ``rpos = fork``).  May repeat an index when a span overlaps keys
    that are already present."""
    br, mt = _rows(branches, mounts)

    def emit(b, upto):
        parent, fork, start, _ = br[b]
        seq = [] if parent < 0 else emit(parent, fork)
        for r in range(upto + 1):
            for (reader, rpos, producer, s, e) in mt:
                if reader == b and rpos == r:
                    ps = br[producer][2]
                    seq.extend(range(ps + s, ps + e))
            if r < upto:
                seq.append(start + r)
        return seq

    return emit(b, br[b][3])


def dedup_first(seq) -> list:
    """Keep the first occurrence of every index (set semantics of the context)."""
    seen = set()
    out = []
    for x in seq:
        if x not in seen:
            seen.add(x)
            out.append(x)
    return out


def branch_of(branches, T: int) -> np.ndarray:
    """Owning branch of every packed token."""
    br, _ = _rows(branches, np.zeros((0, 5)))
    out = np.full(T, -1, dtype=np.int64)
    for b, (_, _, start, length) in enumerate(br):
        out[start:start + length] = b
    return out
