"""Seeded episode structures: branch tables, mount tables, page tables, cursors.

Table formats (shared by every consumer):

* ``branches``: ``int32[NB, 4]`` rows ``(parent, fork, start, len)``.  Row 0 is the
  root with ``parent = -1``.  ``fork`` is the offset into the parent's own tokens at
  which the child was forked (a ``fork`` call of the project page's primitives
  table); ``start`` is where the branch's own tokens sit in the packed stream.
* ``mounts``: ``int32[NM, 5]`` rows ``(reader, rpos, producer, s, e)``: the reader,
  when its own length was ``rpos``, issued ``read(producer, [s, e))`` over the
  producer's own tokens (the ``read_thread`` row of that table).

Only structure is drawn here; nothing in this module decides what a token sees.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Dag:
    name: str
    branches: np.ndarray  # int32 [NB, 4]
    mounts: np.ndarray  # int32 [NM, 5]
    T: int
    meta: dict = field(default_factory=dict)

    @property
    def nb(self) -> int:
        return int(self.branches.shape[0])

    @property
    def nm(self) -> int:
        return int(self.mounts.shape[0])


def _tables(rows_b, rows_m):
    b = np.asarray(rows_b, dtype=np.int32).reshape(-1, 4)
    m = np.asarray(rows_m, dtype=np.int32).reshape(-1, 5)
    return b, m


# --------------------------------------------------------------------------------------
# The named workloads.
# --------------------------------------------------------------------------------------

def tiny() -> Dag:
    """Tiny fixed DAG: a 256-token root forks two 128-token branches; branch 2 mounts
    the span [32, 96) of branch 1 when its own length is 64.  512 packed tokens."""
    b, m = _tables(
        [[-1, 0, 0, 256], [0, 256, 256, 128], [0, 256, 384, 128]],
        [[2, 64, 1, 32, 96]],
    )
    return Dag("tiny", b, m, 512)


def forked(rng: np.random.Generator, prefix=4096, n_children=4, child_len=4096,
           n_mounts=2, span=1024) -> Dag:
    """A root prefix forks ``n_children`` equal siblings; ``n_mounts`` read_thread
    mounts, each between two distinct siblings (reader and producer drawn without
    repetition), over the producer's terminal ``span`` tokens, issued at a reader
    offset drawn uniformly in [0, child_len)."""
    perm = rng.permutation(n_children)
    rpos = rng.integers(0, child_len, size=n_mounts)
    rows_b = [[-1, 0, 0, prefix]]
    for c in range(n_children):
        rows_b.append([0, prefix, prefix + c * child_len, child_len])
    rows_m = []
    for i in range(n_mounts):
        reader = 1 + int(perm[(2 * i) % n_children])
        producer = 1 + int(perm[(2 * i + 1) % n_children])
        rows_m.append([reader, int(rpos[i]), producer, child_len - span, child_len])
    b, m = _tables(rows_b, rows_m)
    return Dag("forked", b, m, prefix + n_children * child_len)


def water_fill(lengths, total, cap, floor=1):
    """Adjust ``lengths`` until they sum to ``total``.  Short of the total: equal
    integer increments to every entry still below ``cap``; when the remainder is
    smaller than the number of such entries, one token each to the shortest, lowest
    index first.  Over the total: the mirror image (equal decrements to entries above
    ``floor``, the remainder from the longest, lowest index first)."""
    L = [int(x) for x in lengths]
    if not floor * len(L) <= total <= cap * len(L):
        raise ValueError("water_fill: target not reachable")
    deficit = total - sum(L)
    while deficit > 0:
        open_ = [i for i in range(len(L)) if L[i] < cap]
        inc = deficit // len(open_)
        if inc > 0:
            for i in open_:
                add = min(inc, cap - L[i])
                L[i] += add
                deficit -= add
        else:
            for i in sorted(open_, key=lambda j: (L[j], j))[:deficit]:
                L[i] += 1
            deficit = 0
    while deficit < 0:
        open_ = [i for i in range(len(L)) if L[i] > floor]
        dec = (-deficit) // len(open_)
        if dec > 0:
            for i in open_:
                sub = min(dec, L[i] - floor)
                L[i] -= sub
                deficit += sub
        else:
            for i in sorted(open_, key=lambda j: (-L[j], j))[:-deficit]:
                L[i] -= 1
            deficit = 0
    return L


def episode(rng: np.random.Generator, total=262144, prefix=8192, n_workers=8,
            wmin=16384, wmax=32768, cont=4096, n_mounts=3, smin=1024, smax=8192,
            name="episode") -> Dag:
    """Orchestrator/worker episode: a ``prefix``-token orchestrator root forks
    ``n_workers`` workers at its end; worker lengths are drawn in [wmin, wmax] then
    water-filled (cap ``wmax``) so the packed total is exactly ``total``.  The
    orchestrator continues in a separate branch of ``cont`` tokens (forked from the
    root at its end, packed last) that mounts the terminal spans of ``n_mounts``
    distinct workers, span lengths in [smin, smax], at sorted reader offsets drawn in
    [0, cont)."""
    lens = rng.integers(wmin, wmax + 1, size=n_workers)
    producers = rng.choice(n_workers, size=n_mounts, replace=False)
    spans = rng.integers(smin, smax + 1, size=n_mounts)
    rpos = np.sort(rng.integers(0, cont, size=n_mounts))
    lens = water_fill(lens, total - prefix - cont, wmax, floor=wmin)
    rows_b = [[-1, 0, 0, prefix]]
    start = prefix
    for w in range(n_workers):
        rows_b.append([0, prefix, start, lens[w]])
        start += lens[w]
    reader = len(rows_b)
    rows_b.append([0, prefix, start, cont])
    rows_m = []
    for i in range(n_mounts):
        p = 1 + int(producers[i])
        Lp = lens[p - 1]
        ell = min(int(spans[i]), Lp)
        rows_m.append([reader, int(rpos[i]), p, Lp - ell, Lp])
    b, m = _tables(rows_b, rows_m)
    assert start + cont == total
    return Dag(name, b, m, total)


def forest(trees, rng: np.random.Generator | None = None, name="forest") -> Dag:
    """Several trees in one packed stream: the rows of every tree, parents and mount
    branch indices shifted by the rows before it.  Without ``rng`` the trees are
    packed one after another, each in its own order; with ``rng`` the branch spans of
    all trees are packed in one random interleaved order."""
    rows_b, rows_m, base = [], [], 0
    for t in trees:
        for (parent, fork, start, L) in t.branches:
            rows_b.append([int(parent) + base if parent >= 0 else -1, int(fork), int(start),
                           int(L)])
        for (reader, rpos, producer, s, e) in t.mounts:
            rows_m.append([int(reader) + base, int(rpos), int(producer) + base, int(s),
                           int(e)])
        base += t.nb
    if rng is None:
        off = 0
        i = 0
        for t in trees:
            for _ in range(t.nb):
                rows_b[i][2] += off
                i += 1
            off += t.T
    else:
        s = 0
        for b in rng.permutation(len(rows_b)):
            rows_b[int(b)][2] = s
            s += rows_b[int(b)][3]
    b, m = _tables(rows_b, rows_m)
    return Dag(name, b, m, int(sum(t.T for t in trees)))


def build(name: str, seed: int | None = None):
    """Return ``(dag, rng)`` for a named workload; ``rng`` is left positioned after
    the structure draws so the tensors can be drawn from it next (structure, then Q,
    K, V, then dO)."""
    defaults = {"tiny": 1, "forked": 2, "episode262k": 3, "episode131k": 3,
                "episode_small": 7, "episode_mid": 11, "forest_small": 13, "forest1m": 17}
    if seed is None:
        seed = defaults[name]
    rng = np.random.default_rng(seed)
    if name == "tiny":
        return tiny(), rng
    if name == "forked":
        return forked(rng), rng
    if name == "episode262k":
        return episode(rng, name=name), rng
    if name == "episode131k":
        return episode(rng, total=131072, prefix=4096, wmin=8192, wmax=16384, cont=2048,
                       smin=512, smax=4096, name=name), rng
    if name == "episode_small":
        # Same shape family, lengths not multiples of any tile size.
        return episode(rng, total=3000, prefix=300, n_workers=5, wmin=200, wmax=600,
                       cont=229, n_mounts=3, smin=20, smax=150, name=name), rng
    if name == "episode_mid":
        return episode(rng, total=12345, prefix=1037, n_workers=6, wmin=900, wmax=2048,
                       cont=611, n_mounts=3, smin=100, smax=700, name=name), rng
    if name == "forest_small":
        # Three small episodes of different totals, branch spans interleaved.
        trees = [episode(rng, total=tot, prefix=pre, n_workers=nw, wmin=150, wmax=700,
                         cont=cont, n_mounts=2, smin=20, smax=150, name=name)
                 for tot, pre, nw, cont in ((3000, 300, 5, 229), (2077, 129, 3, 301),
                                            (1111, 65, 2, 97))]
        return forest(trees, rng, name=name), rng
    if name == "forest1m":
        # Four 262,144-token episodes of the headline shape, packed one after another
        # (the trainer's step holds about a million owned tokens).
        trees = [episode(rng, name=name) for _ in range(4)]
        return forest(trees, name=name), rng
    raise KeyError(name)


# --------------------------------------------------------------------------------------
# Small random DAGs for property tests.
# --------------------------------------------------------------------------------------

def fuzz_dag(rng: np.random.Generator, max_branches=6, max_len=40, max_mounts=4,
             acyclic=True, name="fuzz") -> Dag:
    """A random small DAG.  Forks and reader offsets favour the edge values 0 and the
    full length; spans may have length 1, overlap each other, or come from an
    ancestor.  Branches are packed in a random order.  With ``acyclic`` every
    producer has a lower table index than its reader (parents always do), which rules
    out dependency cycles by construction; without it cycles may occur."""
    nb = int(rng.integers(1, max_branches + 1))
    lens = [int(rng.integers(1, max_len + 1)) for _ in range(nb)]
    parents = [-1] + [int(rng.integers(0, b)) for b in range(1, nb)]

    def edge_pick(n):
        u = rng.random()
        if u < 0.2:
            return 0
        if u < 0.4:
            return n
        return int(rng.integers(0, n + 1))

    forks = [0] + [edge_pick(lens[parents[b]]) for b in range(1, nb)]
    order = rng.permutation(nb)
    starts = [0] * nb
    s = 0
    for b in order:
        starts[int(b)] = s
        s += lens[int(b)]
    rows_b = [[parents[b], forks[b], starts[b], lens[b]] for b in range(nb)]
    rows_m = []
    if nb >= 2:
        nm = int(rng.integers(0, max_mounts + 1))
        for _ in range(nm):
            reader = int(rng.integers(1 if acyclic else 0, nb))
            if acyclic:
                producer = int(rng.integers(0, reader))
            else:
                producer = int(rng.integers(0, nb - 1))
                if producer >= reader:
                    producer += 1
            Lp = lens[producer]
            if rng.random() < 0.25:
                a = int(rng.integers(0, Lp))
                e = a + 1
            else:
                a = int(rng.integers(0, Lp))
                e = int(rng.integers(a + 1, Lp + 1))
            rows_m.append([reader, edge_pick(lens[reader]), producer, a, e])
    b, m = _tables(rows_b, rows_m)
    return Dag(name, b, m, s)


# --------------------------------------------------------------------------------------
# Paged decode workloads.
# --------------------------------------------------------------------------------------

@dataclass
class DecodeWorkload:
    """A paged decode batch.  ``dag`` holds one root (the shared prefix) and one branch
    per cursor; ``page_ptr``/``pages`` is the page table (CSR over branches: physical
    page ids holding each branch's own tokens in order, ``page_size`` tokens per page,
    each branch starting on a fresh page); ``cursors`` lists the branch of each
    cursor, whose current token is that branch's last token."""
    dag: Dag
    page_size: int
    n_pages: int
    page_ptr: np.ndarray  # int32 [NB+1]
    pages: np.ndarray  # int32 [sum pages]
    cursors: np.ndarray  # int32 [B]


def assign_pages(dag: Dag, page_size: int, rng: np.random.Generator, n_pages=None,
                 shuffle=True):
    """Give every branch ``ceil(len/page_size)`` pages of its own, from a seeded
    permutation of the pool (or consecutive ids when ``shuffle`` is false)."""
    need = [-(-int(L) // page_size) for L in dag.branches[:, 3]]
    total = int(sum(need))
    if n_pages is None:
        n_pages = total
    if n_pages < total:
        raise ValueError("pool too small")
    ids = rng.permutation(n_pages) if shuffle else np.arange(n_pages)
    ptr = np.zeros(len(need) + 1, dtype=np.int32)
    ptr[1:] = np.cumsum(need)
    pages = ids[:total].astype(np.int32)
    return n_pages, ptr, pages


def decode_workload(seed=5, n_cursors=64, prefix=16384, own_max=32768, max_mounts=3,
                    span_max=8192, page_size=64, name="decode64") -> DecodeWorkload:
    """Paged mounted decode: ``n_cursors`` cursors share a ``prefix``-token radix
    prefix; each has its own branch of ``L ~ U{1..own_max}`` tokens (the last one is
    the current token) and ``min(U{0..max_mounts}, c)`` mounts of terminal spans of
    distinct earlier cursors' branches, span length ``U{1..min(span_max, L_producer)}``, issued
    at a reader offset ``U{0..L-1}``.  Physical page ids are a seeded permutation of
    a pool just large enough for every branch's own pages."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1, own_max + 1, size=n_cursors)
    rows_b = [[-1, 0, 0, prefix]]
    start = prefix
    for c in range(n_cursors):
        rows_b.append([0, prefix, start, int(L[c])])
        start += int(L[c])
    rows_m = []
    for c in range(n_cursors):
        # Producers are earlier cursors (lower index): a mounted span then never
        # depends, through positions, on the reader itself.
        k = min(int(rng.integers(0, max_mounts + 1)), c)
        prods = rng.choice(c, size=k, replace=False) if k else []
        for p in prods:
            Lp = int(L[p])
            ell = int(rng.integers(1, min(span_max, Lp) + 1))
            rpos = int(rng.integers(0, int(L[c])))
            rows_m.append([c + 1, rpos, int(p) + 1, Lp - ell, Lp])
    b, m = _tables(rows_b, rows_m)
    dag = Dag(name, b, m, start)
    n_pages, ptr, pages = assign_pages(dag, page_size, rng)
    cursors = np.arange(1, n_cursors + 1, dtype=np.int32)
    return DecodeWorkload(dag, page_size, n_pages, ptr, pages, cursors)


def extend_workload(seed=5, new_min=256, new_max=2048, **kw):
    """The paged decode batch of ``decode_workload`` with every cursor appending a turn:
    its branch's last ``min(L, U{new_min..new_max})`` tokens are new.  Returns
    ``(workload, n_new)``."""
    wl = decode_workload(seed=seed, **kw)
    rng = np.random.default_rng(seed + 1000)
    L = wl.dag.branches[wl.cursors, 3]
    n_new = np.minimum(L, rng.integers(new_min, new_max + 1, size=len(L))).astype(np.int32)
    return wl, n_new
