"""Forest batching on the CPU: several episode trees packed into one stream and one
plan (a training step batches several episodes, card "03 · Training" of the Octopus
project page).

Pins: a forest is block diagonal.  Every tree's positions, mask rows, attention
outputs and gradients equal those of the same tree packed alone (which the
single-tree pins fix), and no token sees another tree.  The planner's mask, expanded
from its tile lists, equals the oracle's bit for bit, and its nnz is the sum of the
trees' nnz."""

import numpy as np
import pytest

import synth
import tree_packed_block_amd as tpb
from oracle import attention as A
from oracle import dag as D
from test_planner import _check_plan


def split_trees(dag):
    """``[(sub_dag, idx)]``: every tree of ``dag`` as a DAG of its own, and the packed
    indices of its tokens in the forest (ascending; the sub-DAG packs them in the same
    relative order)."""
    br = dag.branches
    tree = np.zeros(dag.nb, dtype=np.int64)
    for b, (parent, _, _, _) in enumerate(br):
        tree[b] = b if parent < 0 else tree[parent]
    out = []
    for root in np.flatnonzero(br[:, 0] < 0):
        rows = np.flatnonzero(tree == root)
        new = {int(b): i for i, b in enumerate(rows)}
        idx = np.sort(np.concatenate([np.arange(br[b, 2], br[b, 2] + br[b, 3])
                                      for b in rows]))
        sb = [[new[int(br[b, 0])] if br[b, 0] >= 0 else -1, int(br[b, 1]),
               int(np.searchsorted(idx, br[b, 2])), int(br[b, 3])] for b in rows]
        sm = [[new[int(m[0])], int(m[1]), new[int(m[2])], int(m[3]), int(m[4])]
              for m in dag.mounts if tree[m[0]] == root]
        b_, m_ = synth.dags._tables(sb, sm)
        out.append((synth.dags.Dag(f"tree{root}", b_, m_, len(idx)), idx))
    return out


def fuzz_forest(seed, n_trees=3, **kw):
    rng = np.random.default_rng(seed)
    trees = [synth.fuzz_dag(rng, **kw) for _ in range(n_trees)]
    return synth.dags.forest(trees, rng if seed % 2 else None)


FORESTS = [("forest_small", None)] + [("fuzz", s) for s in range(6)]


def _forest(name, seed):
    if name == "fuzz":
        return fuzz_forest(seed, n_trees=2 + seed % 3, max_len=60, max_branches=5,
                           max_mounts=3)
    return synth.build(name)[0]


@pytest.mark.parametrize("name,seed", FORESTS)
def test_forest_positions_and_mask_are_block_diagonal(name, seed):
    dag = _forest(name, seed)
    D.validate(dag.branches, dag.mounts, dag.T)
    pos = D.positions(dag.branches, dag.mounts)
    M = D.mask(dag.branches, dag.mounts, dag.T)
    parts = split_trees(dag)
    assert len(parts) == int((dag.branches[:, 0] < 0).sum()) >= 2
    covered = np.zeros(dag.T, dtype=bool)
    for sub, idx in parts:
        assert np.array_equal(pos[idx], D.positions(sub.branches, sub.mounts))
        rows = M[idx]
        assert np.array_equal(rows[:, idx], D.mask(sub.branches, sub.mounts, sub.T))
        rows[:, idx] = False
        assert not rows.any()
        covered[idx] = True
    assert covered.all()


@pytest.mark.parametrize("seed", [1, 4])
def test_forest_attention_equals_each_tree_alone(seed):
    dag = fuzz_forest(seed, n_trees=3, max_len=50, max_branches=4, max_mounts=3)
    rng = np.random.default_rng(100 + seed)
    x = synth.draw_attention_inputs(rng, dag.T, 4, 2, 16,
                                    D.positions(dag.branches, dag.mounts), dtype="fp32",
                                    std=1.0, with_dout=True)
    o, lse = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts)
    for sub, idx in split_trees(dag):
        so, sl = A.attn_fwd(x["q"][idx], x["k"][idx], x["v"][idx], sub.branches,
                            sub.mounts)
        np.testing.assert_allclose(o[idx], so, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, idx], sl, rtol=0, atol=1e-12)
        sg = A.attn_bwd(x["q"][idx], x["k"][idx], x["v"][idx], x["do"][idx], sub.branches,
                        sub.mounts)
        for a, b in zip(g, sg):
            np.testing.assert_allclose(a[idx], b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,seed", FORESTS)
def test_forest_plan_bit_exact(name, seed):
    dag = _forest(name, seed)
    p = _check_plan(dag)
    nnz = sum(int(D.mask(s.branches, s.mounts, s.T).sum()) for s, _ in split_trees(dag))
    assert p.stats()["nnz"] == nnz


def test_forest1m_plan_matches_its_trees():
    """Four 262,144-token trees: positions equal each tree's alone, nnz is the sum of
    the trees' nnz (each from its own plan)."""
    dag, _ = synth.build("forest1m")
    p = tpb.Plan(dag.branches, dag.mounts, dag.T)
    pos = p.positions()
    total = 0
    for sub, idx in split_trees(dag):
        ps = tpb.Plan(sub.branches, sub.mounts, sub.T)
        assert np.array_equal(pos[idx], ps.positions())
        total += ps.stats()["nnz"]
    assert p.stats()["nnz"] == total


def test_cross_tree_mount_rejected():
    b = np.array([[-1, 0, 0, 4], [0, 2, 4, 3], [-1, 0, 7, 5]])
    D.validate(b, np.array([[1, 1, 0, 0, 2]]), 12)
    for m in ([[2, 1, 0, 0, 2]], [[1, 0, 2, 0, 3]]):
        with pytest.raises(D.DagError):
            D.validate(b, np.array(m), 12)
        with pytest.raises(tpb.OctopusError) as ei:
            tpb.Plan(b, np.array(m), 12)
        assert ei.value.name == "EINVAL"
