"""GPU parity of forward and backward on small DAGs built for the degenerate cases of
the packing: a single token, tile-aligned and one-past-aligned streams, a fork at
offset 0 (the child sees none of its parent) and at the parent's full length, a child
packed before its parent, one-token mounted spans at reader offset 0 and at the
reader's full length, a span mounted twice, a reader that mounts from an ancestor, and
readers that mount spans of their own descendants (a child and a great-grandchild,
read after the fork the descendant's line starts from, so no position depends on
itself); then fuzzed DAGs whose producers may be any branch of the tree."""

import pytest

from oracle import attention as A
from parity import TOL, check_close, check_grad, dev, host, say, table_workload

pytestmark = pytest.mark.gpu

EDGE_DAGS = {
    "one_token": ([[-1, 0, 0, 1]], []),
    "aligned_256": ([[-1, 0, 0, 256]], []),
    "one_past_128": ([[-1, 0, 0, 129]], []),
    "fork_at_zero": ([[-1, 0, 0, 64], [0, 0, 64, 65]], []),
    "fork_at_end": ([[-1, 0, 0, 130], [0, 130, 130, 1]], []),
    "child_first": ([[-1, 0, 129, 127], [0, 50, 0, 129]], []),
    "span_len1_rpos0": ([[-1, 0, 0, 70], [0, 70, 70, 40], [0, 33, 110, 90]],
                        [[2, 0, 1, 5, 6]]),
    "span_at_reader_end": ([[-1, 0, 0, 70], [0, 70, 70, 40], [0, 33, 110, 90]],
                           [[2, 90, 1, 0, 40]]),
    "span_twice": ([[-1, 0, 0, 200], [0, 100, 200, 150], [0, 150, 350, 100]],
                   [[2, 10, 1, 20, 90], [2, 10, 1, 20, 90]]),
    "span_from_ancestor": ([[-1, 0, 0, 100], [0, 60, 100, 80], [1, 80, 180, 120]],
                           [[2, 30, 0, 70, 100]]),
    # branch 1 forks branch 2 at its offset 40 and mounts [10, 110) of it at offset 90
    "span_from_child": ([[-1, 0, 0, 100], [0, 100, 100, 150], [1, 40, 250, 120]],
                        [[1, 90, 2, 10, 110]]),
    # branch 1 mounts all of its great-grandchild 3 (line 1 -> 2 at 30 -> 3 at 50) at
    # offset 60, and branch 2 mounts a span of branch 3 too
    "span_from_descendants": ([[-1, 0, 0, 80], [0, 80, 80, 100], [1, 30, 180, 90],
                               [2, 50, 270, 70]],
                              [[1, 60, 3, 0, 70], [2, 70, 3, 20, 45]]),
}


@pytest.mark.parametrize("name", sorted(EDGE_DAGS))
@pytest.mark.parametrize("Hq,Hkv,Dh", [(4, 2, 128), (3, 1, 64)])
def test_edge_fwd_bwd_bf16(name, Hq, Hkv, Dh):
    import torch
    import tree_packed_block_amd as tpb
    say(f"case edge {name} Hq={Hq} Hkv={Hkv} D={Dh}")
    rows_b, rows_m = EDGE_DAGS[name]
    dag, x = table_workload(name, rows_b, rows_m, Hq, Hkv, Dh)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "bf16") for k, v in x.items()}
    o, lse = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(host(o), ro, TOL["bf16"], "O")
    check_close(host(lse), rl, TOL["bf16"], "LSE")
    gq, gk, gv = A.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts)
    check_grad(host(dq), gq, "dQ")
    check_grad(host(dk), gk, "dK")
    check_grad(host(dv), gv, "dV")


def _any_producer_dag(seed):
    """A fuzzed DAG whose mounts may name any other branch as producer (ancestors,
    descendants, siblings), redrawn until it has a mount and the oracle finds no position
    cycle."""
    import numpy as np
    import synth
    from oracle import dag as D
    rng = np.random.default_rng(seed)
    while True:
        dag = synth.fuzz_dag(rng, max_len=300, max_branches=7, max_mounts=5, acyclic=False)
        if len(dag.mounts) == 0:
            continue
        try:
            D.positions(dag.branches, dag.mounts)
        except D.DagError as e:
            assert e.code == "ECYCLE"
            continue
        return dag, rng


def _descends(br, a, b):
    """True if branch a descends from branch b."""
    while a >= 0:
        a = int(br[a][0])
        if a == b:
            return True
    return False


@pytest.mark.parametrize("seed", range(8))
def test_fuzz_any_producer_fwd_bwd_bf16(seed):
    import torch
    import synth
    import tree_packed_block_amd as tpb
    from oracle import dag as D
    dag, rng = _any_producer_dag(1000 + seed)
    desc = sum(_descends(dag.branches, int(p), int(r)) for (r, rp, p, s, e) in dag.mounts)
    say(f"case edge fuzz any-producer seed={seed} T={dag.T} mounts={len(dag.mounts)} "
        f"from descendants={desc}")
    pos = D.positions(dag.branches, dag.mounts)
    x = synth.draw_attention_inputs(rng, dag.T, 4, 2, 128, pos, dtype="bf16", std=0.5,
                                    with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "bf16") for k, v in x.items()}
    o, lse = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(host(o), ro, TOL["bf16"], "O")
    gq, gk, gv = A.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts)
    check_grad(host(dq), gq, "dQ")
    check_grad(host(dk), gk, "dK")
    check_grad(host(dv), gv, "dV")

