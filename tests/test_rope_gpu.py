"""GPU parity of attention with RoPE applied on the device at the DAG positions, against
the float64 oracle (``oracle.rope``), through the C-ABI library: the rotation itself at
large positions, forward and backward with unrotated Q and K (gradients with respect to
the unrotated inputs), and decode / extend queries rotated at their cursor positions
over pages holding keys rotated at their producers' positions."""

import numpy as np
import pytest

import synth
from oracle import decode as DEC
from oracle import rope as R
from parity import TOL, check_close, check_grad, dev, host, say

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [128, 64])
def test_rope_kernel(dtype, D):
    import torch
    import tree_packed_block_amd as tpb
    say(f"case rope kernel {dtype} D={D}")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((777, 5, D)).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    pos = rng.integers(0, 300000, size=777)
    pos[:3] = [0, 1, 299999]
    got = host(tpb.rope(dev(x, dtype), _i32(pos)))
    ref = R.rotate(x, pos)
    check_close(got, ref, TOL[dtype], "rotated")
    back = host(tpb.rope(dev(got.astype(np.float32), dtype), _i32(pos), inverse=True))
    check_close(back, x, 2 * TOL[dtype], "rotated back")
    torch.cuda.synchronize()


def _rope_case(dag, Hq, Hkv, Dh, dtype, seed):
    import torch
    import tree_packed_block_amd as tpb
    rng = np.random.default_rng(seed)
    x = synth.draw_attention_inputs(rng, dag.T, Hq, Hkv, Dh, np.zeros(dag.T, dtype=np.int64),
                                    dtype=dtype, std=0.5, with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, dtype) for k, v in x.items()}
    o, lse = tpb.attn_fwd_rope(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = tpb.attn_bwd_rope(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    ro, rl = R.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(host(o), ro, TOL[dtype], "O")
    check_close(host(lse), rl, TOL[dtype], "LSE")
    gq, gk, gv = R.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts)
    check_grad(host(dq), gq, "dQ")
    check_grad(host(dk), gk, "dK")
    check_grad(host(dv), gv, "dV")


def test_rope_fwd_bwd_tiny_fp32():
    say("case rope fwd+bwd tiny fp32")
    dag, _ = synth.build("tiny")
    _rope_case(dag, 1, 1, 64, "fp32", 1)


@pytest.mark.parametrize("name", ["episode_small", "forked", "forest_small"])
def test_rope_fwd_bwd_bf16(name):
    say(f"case rope fwd+bwd {name} bf16")
    dag, _ = synth.build(name)
    _rope_case(dag, 16, 4, 128, "bf16", 2)


@pytest.mark.parametrize("seed", range(3))
def test_rope_fwd_bwd_fuzz(seed):
    say(f"case rope fwd+bwd fuzz seed={seed}")
    dag = synth.fuzz_dag(np.random.default_rng(500 + seed), max_len=300, max_branches=7,
                         max_mounts=5)
    _rope_case(dag, 6, 2, 64, "bf16", 600 + seed)


def test_rope_decode_and_extend_queries():
    """Queries turned on the device at their tokens' positions (dag_positions); pages hold
    keys already turned at their producers' positions, so mounts copy nothing."""
    import torch
    import tree_packed_block_amd as tpb
    say("case rope decode + extend")
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=64)
    br = wl.dag.branches
    pos = tpb.dag_positions(br, wl.dag.mounts, wl.dag.T)
    x = synth.draw_decode_inputs(np.random.default_rng(12), len(wl.cursors), 16, 4, 128,
                                 wl.n_pages, 64)
    last = br[wl.cursors, 2] + br[wl.cursors, 3] - 1
    qr = tpb.rope(dev(x["q"], "bf16"), _i32(pos[last]))
    segs = tpb.decode_segments(br, wl.dag.mounts, wl.page_ptr, wl.pages, 64, wl.n_pages,
                               wl.cursors)
    od, ld = tpb.paged_mount_decode(qr, dev(x["k_pool"], "bf16"), dev(x["v_pool"], "bf16"),
                                    *[_i32(s) for s in segs], n_split=4)
    torch.cuda.synchronize()
    ro, rl = DEC.decode(R.rotate(x["q"], pos[last]), x["k_pool"], x["v_pool"], br,
                        wl.dag.mounts, wl.page_ptr, wl.pages, 64, wl.cursors)
    check_close(host(od), ro, TOL["bf16"], "decode O")
    check_close(host(ld), rl, TOL["bf16"], "decode LSE")
    # extend: the last n_c own tokens of every cursor, each at its own position
    n_new = np.minimum(br[wl.cursors, 3], 150)
    rows = np.concatenate([np.arange(int(br[b, 2] + br[b, 3] - m), int(br[b, 2] + br[b, 3]))
                           for b, m in zip(wl.cursors, n_new)])
    xe = synth.draw_extend_inputs(np.random.default_rng(13), len(rows), 16, 4, 128,
                                  wl.n_pages, 64)
    qe = tpb.rope(dev(xe["q"], "bf16"), _i32(pos[rows]))
    sp, pg, lo, hi, thr, causal, first = tpb.extend_segments(
        br, wl.dag.mounts, wl.page_ptr, wl.pages, 64, wl.n_pages, wl.cursors, n_new)
    q_ptr = np.concatenate([[0], np.cumsum(n_new)])
    oe, le = tpb.paged_mount_extend(qe, dev(xe["k_pool"], "bf16"), dev(xe["v_pool"], "bf16"),
                                    _i32(q_ptr), int(n_new.max()), _i32(first), _i32(sp),
                                    _i32(pg), _i32(lo), _i32(hi), _i32(thr), _i32(causal))
    torch.cuda.synchronize()
    reo, rel = DEC.extend(R.rotate(xe["q"], pos[rows]), xe["k_pool"], xe["v_pool"], br,
                          wl.dag.mounts, wl.page_ptr, wl.pages, 64, wl.cursors, q_ptr)
    check_close(host(oe), reo, TOL["bf16"], "extend O")
    check_close(host(le), rel, TOL["bf16"], "extend LSE")


@pytest.mark.timeout(900)
def test_rope_fwd_bwd_full_size_sampled():
    """The 131,072-token tree with unrotated Q and K (query rows and gradients turned in
    the kernels' registers, positions up to ~2*10^4): O and LSE on sampled rows, dQ on
    sampled rows, dK/dV on keys whose every reader the oracle enumerates."""
    import torch
    import tree_packed_block_amd as tpb
    from parity import sample_rows
    from test_bwd_gpu import _key_samples, _merge
    say("case rope fwd+bwd episode131k sampled")
    dag, _ = synth.build("episode131k")
    rng = np.random.default_rng(31)
    x = synth.draw_attention_inputs(rng, dag.T, 16, 4, 128, np.zeros(dag.T, dtype=np.int64),
                                    dtype="bf16", std=0.5, with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    assert int(plan.positions().max()) > 16384
    t = {k: dev(v, "bf16") for k, v in x.items()}
    o, lse = tpb.attn_fwd_rope(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = tpb.attn_bwd_rope(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = host(o), host(lse), host(dq), host(dk), host(dv)
    qrows = sample_rows(dag)
    ro, rl = R.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts, rows=qrows)
    qi = np.concatenate([np.arange(lo, hi) for lo, hi in qrows])
    check_close(o[qi], ro[qi], TOL["bf16"], "O (sampled rows)")
    check_close(lse[:, qi], rl[:, qi], TOL["bf16"], "LSE (sampled rows)")
    keys, krows = _key_samples(dag)
    rows = _merge(qrows + krows)
    gq, gk, gv = R.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts,
                            rows=rows)
    ki = np.concatenate([np.arange(lo, hi) for lo, hi in keys])
    check_grad(dq[qi], gq[qi], "dQ (sampled rows)")
    check_grad(dk[ki], gk[ki], "dK (sampled keys)")
    check_grad(dv[ki], gv[ki], "dV (sampled keys)")
