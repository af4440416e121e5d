"""Pins of the oracle's DAG semantics: hand-derived values, closed forms, a second
independent formulation, brute force and invariants."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import dag as D
from conftest import read_golden


def _fuzz(seed, acyclic=True, **kw):
    return synth.fuzz_dag(np.random.default_rng(seed), acyclic=acyclic, **kw)


# ---------------------------------------------------------------------------- positions

def test_tiny_positions_hand_derived():
    dag, _ = synth.build("tiny")
    pos = D.positions(dag.branches, dag.mounts)
    vals = read_golden("tiny_positions.txt")
    expect = np.full(dag.T, -1)
    for lo, hi, p0 in zip(vals[0::3], vals[1::3], vals[2::3]):
        expect[lo:hi] = np.arange(p0, p0 + hi - lo)
    assert np.array_equal(pos, expect)


def _closed_form_x(dag, xs):
    """x_b(r) = max(base_b + r, max over mounts of b issued at rpos <= r of
    E_m + 1 + (r - rpos)): unrolling the one-step recursion by hand."""
    out = []
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        base = 0 if parent < 0 else xs[parent][fork]
        row = []
        for r in range(L + 1):
            best = base + r
            for (reader, rpos, producer, s, e) in dag.mounts:
                if reader == b and rpos <= r:
                    E = xs[producer][e - 1] + 1
                    best = max(best, E + 1 + r - rpos)
            row.append(best)
        out.append(row)
    return out


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 10**9))
def test_positions_closed_form(seed):
    dag = _fuzz(seed)
    xs = D.branch_positions(dag.branches, dag.mounts)
    assert _closed_form_x(dag, xs) == xs


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 10**9))
def test_positions_invariants(seed):
    dag = _fuzz(seed)
    xs = D.branch_positions(dag.branches, dag.mounts)
    pos = D.positions(dag.branches, dag.mounts)
    M = D.mask(dag.branches, dag.mounts, dag.T)
    jumps_at = {}
    for (reader, rpos, producer, s, e) in dag.mounts:
        jumps_at.setdefault(int(reader), set()).add(int(rpos))
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        x = np.array(xs[b])
        d = np.diff(x)
        # strictly increasing; steps larger than one only where a mount was issued
        assert np.all(d >= 1)
        for r in np.flatnonzero(d > 1) + 1:
            assert r in jumps_at.get(b, set())
        if parent >= 0:
            assert x[0] >= xs[parent][fork]
            if 0 not in jumps_at.get(b, set()):
                assert x[0] == xs[parent][fork]
    # no RoPE flip: every visible key other than the query sits at a lower position
    ii, jj = np.nonzero(M)
    off = ii != jj
    assert np.all(pos[jj[off]] < pos[ii[off]])


def test_positions_cycle_detection():
    # b1 mounts b2[0:5) before its first token and b2 mounts b1[0:5) before its first
    # token: each first position needs the other's fifth.
    br = np.array([[-1, 0, 0, 4], [0, 4, 4, 6], [0, 4, 10, 6]])
    mt = np.array([[1, 0, 2, 0, 5], [2, 0, 1, 0, 5]])
    with pytest.raises(D.DagError) as ei:
        D.positions(br, mt)
    assert ei.value.code == "ECYCLE"
    # Mutual reads at the branch level are fine when the tokens do not depend on
    # each other: spans [0,3) read at offset 4.
    mt2 = np.array([[1, 4, 2, 0, 3], [2, 4, 1, 0, 3]])
    pos = D.positions(br, mt2)
    # b1: 4,5,6,7 then the mount of b2[0:3) (positions 4..6, E=7) -> max(8, 8) = 8
    assert list(pos[4:10]) == [4, 5, 6, 7, 8, 9]
    # A root that mounts a descendant's span that forked after the mount point.
    br3 = np.array([[-1, 0, 0, 10], [0, 8, 10, 4]])
    with pytest.raises(D.DagError):
        D.positions(br3, np.array([[0, 5, 1, 0, 2]]))
    pos3 = D.positions(br3, np.array([[0, 9, 1, 0, 2]]))
    # child: base x_root(8) = 8 -> 8, 9; E = 10; root offset 9 -> max(9, 11) = 11
    assert list(pos3[:10]) == list(range(9)) + [11]
    assert list(pos3[10:]) == [8, 9, 10, 11]


def test_validate_errors():
    ok_b = np.array([[-1, 0, 0, 4], [0, 2, 4, 3]])
    ok_m = np.array([[1, 1, 0, 0, 2]])
    D.validate(ok_b, ok_m, 7)
    bad = [
        (np.array([[0, 0, 0, 4], [0, 2, 4, 3]]), ok_m, 7),  # root with a parent
        (np.array([[-1, 0, 0, 4], [1, 2, 4, 3]]), ok_m, 7),  # parent not lower
        (np.array([[-1, 0, 0, 4], [0, 5, 4, 3]]), ok_m, 7),  # fork past the parent
        (np.array([[-1, 0, 0, 4], [0, 2, 4, 0]]), ok_m, 4),  # empty branch
        (np.array([[-1, 0, 0, 4], [0, 2, 5, 3]]), ok_m, 8),  # gap in the packing
        (np.array([[-1, 0, 0, 4], [0, 2, 3, 3]]), ok_m, 6),  # overlap
        (ok_b, np.array([[1, 1, 1, 0, 2]]), 7),  # reader == producer
        (ok_b, np.array([[1, 4, 0, 0, 2]]), 7),  # rpos past the reader
        (ok_b, np.array([[1, 1, 0, 2, 2]]), 7),  # empty span
        (ok_b, np.array([[1, 1, 0, 0, 5]]), 7),  # span past the producer
        (ok_b, np.array([[1, 1, 2, 0, 1]]), 7),  # producer index out of range
        (np.array([[-1, 0, 0, 4], [-1, 2, 4, 3]]), ok_m, 7),  # second root forked
        (np.array([[-1, 0, 0, 4], [-1, 0, 4, 3]]), ok_m, 7),  # mount across trees
    ]
    for b, m, T in bad:
        with pytest.raises(D.DagError) as ei:
            D.validate(b, m, T)
        assert ei.value.code == "EINVAL"


# ---------------------------------------------------------------------------- visibility

def test_tiny_nnz_hand_derived():
    dag, _ = synth.build("tiny")
    nnz, ctx448 = read_golden("tiny_nnz.txt")
    M = D.mask(dag.branches, dag.mounts, dag.T)
    assert int(M.sum()) == nnz
    assert int(M[448].sum()) == ctx448
    assert len(D.visible(dag.branches, dag.mounts, 448)) == ctx448


def test_forked_nnz_closed_form():
    dag, _ = synth.build("forked")
    # root causal + 4 children each seeing the 4096 prefix and themselves causally,
    # plus (4096 - rpos) reader rows times 1024 mounted keys per mount.
    base = 4096 * 4097 // 2 + 4 * (4096 * 4096 + 4096 * 4097 // 2)
    assert base == 109_062_144
    extra = sum(1024 * (4096 - int(m[1])) for m in dag.mounts)
    from oracle.attention import useful_pairs
    assert useful_pairs(dag.branches, dag.mounts, dag.T) == base + extra


@pytest.mark.parametrize("name", ["episode_small", "episode_mid"])
def test_episode_nnz_closed_form(name):
    dag, _ = synth.build(name)
    br, mt = dag.branches, dag.mounts
    # Without overlaps: sum over branches of len*|H(b)| + causal + mounted rows*span.
    total = 0
    for b, (parent, fork, start, L) in enumerate(br):
        H = 0 if parent < 0 else int(fork)  # every non-root branch forks from the root
        total += L * H + L * (L + 1) // 2
        for (reader, rpos, producer, s, e) in mt:
            if reader == b:
                total += (L - rpos) * (e - s)
    from oracle.attention import useful_pairs
    assert useful_pairs(br, mt, dag.T) == total


@settings(max_examples=200, deadline=None)
@given(st.integers(0, 10**9), st.booleans())
def test_mask_three_formulations(seed, acyclic):
    """Dense rows == recursive sets == prefixes of the flattened paths.  The path
    formulation needs a DAG whose positions exist: with a dependency cycle a token can
    be mounted into its own past, so only the first two are compared then."""
    dag = _fuzz(seed, acyclic=acyclic)
    M = D.mask(dag.branches, dag.mounts, dag.T)
    try:
        D.positions(dag.branches, dag.mounts)
        has_paths = True
    except D.DagError as e:
        assert e.code == "ECYCLE" and not acyclic
        has_paths = False
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        seq = D.flatten_path(dag.branches, dag.mounts, b)
        for r in range(L):
            i = start + r
            s_set = D.visible(dag.branches, dag.mounts, i)
            assert set(np.flatnonzero(M[i])) == s_set
            if has_paths:
                upto = seq[: seq.index(i) + 1]
                assert set(upto) == s_set


@settings(max_examples=100, deadline=None)
@given(st.integers(0, 10**9))
def test_mask_prefix_tree_without_mounts(seed):
    """No mounts: a query sees exactly the tokens on its root-to-branch path before
    it, found here by walking parent links."""
    dag = _fuzz(seed)
    br = dag.branches
    M = D.mask(br, np.zeros((0, 5), dtype=np.int32), dag.T)
    for b, (parent, fork, start, L) in enumerate(br):
        for r in range(L):
            want = set(range(start, start + r + 1))
            cur, cut = b, None
            while br[cur][0] >= 0:
                cut = br[cur][1]
                cur = br[cur][0]
                want |= set(range(br[cur][2], br[cur][2] + cut))
            assert set(np.flatnonzero(M[start + r])) == want


def test_single_branch_is_lower_triangular():
    br = np.array([[-1, 0, 0, 37]])
    M = D.mask(br, np.zeros((0, 5)), 37)
    assert np.array_equal(M, np.tril(np.ones((37, 37), dtype=bool)))


def test_overlapping_mount_counts_once():
    # A child mounts a span of its own parent that it already sees.
    br = np.array([[-1, 0, 0, 10], [0, 8, 10, 5]])
    mt = np.array([[1, 0, 0, 2, 6], [1, 2, 0, 4, 10]])
    M = D.mask(br, mt, 15)
    # row of child offset 3 (packed 13): root [0,8) + root [4,10) + own [10,14)
    assert set(np.flatnonzero(M[13])) == set(range(0, 10)) | set(range(10, 14))
    seq = D.flatten_path(br, mt, 1)
    assert len(D.dedup_first(seq)) < len(seq)
