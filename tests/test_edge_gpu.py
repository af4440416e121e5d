"""GPU parity of forward and backward on small DAGs built for the degenerate cases of
the packing: a single token, tile-aligned and one-past-aligned streams, a fork at
offset 0 (the child sees none of its parent) and at the parent's full length, a child
packed before its parent, one-token mounted spans at reader offset 0 and at the
reader's full length, a span mounted twice, and a reader that mounts from an
ancestor."""

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
