"""GPU parity of the packed-DAG attention backward against the float64 oracle,
through the C-ABI library.  Gradients: relative Frobenius error <= 5e-2 per tensor;
shared-prefix keys are owned once and mounted keys receive their readers'
gradients (both are what the packed oracle computes)."""

import numpy as np
import pytest

import synth
from oracle import attention as A
from parity import (GRAD_TOL, TOL, check_close, check_grad, dev, fuzz_workload, host,
                    sample_rows, say, workload)

pytestmark = pytest.mark.gpu


def _run(dag, x, dtype):
    import torch
    import tree_packed_block_amd as tpb
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, dtype) for k, v in x.items()}
    o, lse = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
    dq, dk, dv = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    return host(o), host(lse), host(dq), host(dk), host(dv)


def _full_case(dag, x, dtype):
    o, lse, dq, dk, dv = _run(dag, x, dtype)
    ro, _ = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(o, ro, TOL[dtype], "O")
    gq, gk, gv = A.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts)
    check_grad(dq, gq, "dQ")
    check_grad(dk, gk, "dK")
    check_grad(dv, gv, "dV")
    if dtype == "fp32":
        # float32 arithmetic end to end: far inside the gradient bound
        for got, ref, nm in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            check_close(got, ref, 1e-4, nm + " (fp32 elementwise)")


def test_bwd_tiny_fp32():
    say("case bwd tiny fp32 H=1 D=64")
    dag, x = workload("tiny", 1, 1, 64, "fp32", 1.0, with_dout=True)
    _full_case(dag, x, "fp32")


def test_bwd_episode_small_fp32_gqa():
    say("case bwd episode_small fp32 4/2 D=64")
    dag, x = workload("episode_small", 4, 2, 64, "fp32", 0.5, with_dout=True)
    _full_case(dag, x, "fp32")


@pytest.mark.parametrize("Dh", [128, 64])
def test_bwd_episode_small_bf16(Dh):
    say(f"case bwd episode_small bf16 16/4 D={Dh}")
    dag, x = workload("episode_small", 16, 4, Dh, "bf16", 0.5, with_dout=True)
    _full_case(dag, x, "bf16")


def test_bwd_episode_mid_bf16():
    say("case bwd episode_mid bf16 16/4 D=128")
    dag, x = workload("episode_mid", 16, 4, 128, "bf16", 0.5, with_dout=True)
    _full_case(dag, x, "bf16")


def test_bwd_forest_small_bf16():
    """Three trees, branch spans interleaved in the stream: one plan, one launch per
    phase."""
    say("case bwd forest_small bf16 16/4 D=128")
    dag, x = workload("forest_small", 16, 4, 128, "bf16", 0.5, with_dout=True)
    _full_case(dag, x, "bf16")


@pytest.mark.parametrize("seed", range(8))
def test_bwd_fuzz_bf16(seed):
    say(f"case bwd fuzz seed={seed}")
    dag, x = fuzz_workload(seed, 4, 2, 128, max_len=300, max_branches=7, max_mounts=5)
    _full_case(dag, x, "bf16")


# Head layouts beyond the common 16/4: an odd group (one head per wave group in dQ),
# one query head per KV head, the largest group, and head_dim 64 with an odd group.
HEAD_CASES = [(3, 1, 128), (2, 2, 128), (16, 1, 128), (6, 2, 64), (8, 8, 64)]


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("Hq,Hkv,Dh", HEAD_CASES)
def test_bwd_fuzz_heads_bf16(Hq, Hkv, Dh, seed):
    say(f"case bwd fuzz heads Hq={Hq} Hkv={Hkv} D={Dh} seed={seed}")
    dag, x = fuzz_workload(100 + seed, Hq, Hkv, Dh, max_len=300, max_branches=7,
                           max_mounts=5)
    _full_case(dag, x, "bf16")


def _key_samples(dag, width=64):
    """Keys whose every reader is cheap to enumerate: the last ``width`` keys of
    every non-root branch.  Their readers are the branch's own later rows and, for
    keys inside a mounted span, the reader branch's rows from the mount on."""
    keys, rows = [], []
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        if parent < 0:
            continue
        k0 = start + max(0, L - width)
        keys.append((k0, start + L))
        rows.append((k0, start + L))
    for (reader, rpos, producer, s, e) in dag.mounts:
        rs = int(dag.branches[reader, 2])
        rows.append((rs + int(rpos), rs + int(dag.branches[reader, 3])))
    return keys, rows


def _merge(ranges):
    out = []
    for lo, hi in sorted(ranges):
        if out and lo <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], hi))
        else:
            out.append((lo, hi))
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["episode131k", "episode262k", "forest1m"])
def test_bwd_full_size_sampled(name):
    """The full tree through the benchmark's launches.  The oracle computes dQ on
    sampled query rows, and dK/dV of sampled keys from every query that sees them
    (so mounted keys include their readers' gradients); whole-tensor identities
    check every row: sum_j dV_j = sum of dO over the group's heads, sum_j dK_j = 0.
    For the single trees, KV head 0 is also checked over every key and row (the shared
    prefix included)."""
    say(f"case bwd {name} sampled")
    dag, x = workload(name, 16, 4, 128, "bf16", 0.5, with_dout=True)
    o, lse, dq, dk, dv = _run(dag, x, "bf16")
    qrows = sample_rows(dag)
    keys, krows = _key_samples(dag)
    rows = _merge(qrows + krows)
    say(f"  oracle rows: {sum(h - l for l, h in rows)}")
    gq, gk, gv = A.attn_bwd(x["q"], x["k"], x["v"], x["do"], dag.branches, dag.mounts,
                            rows=rows)
    qi = np.concatenate([np.arange(lo, hi) for lo, hi in qrows])
    ki = np.concatenate([np.arange(lo, hi) for lo, hi in keys])
    check_grad(dq[qi], gq[qi], "dQ (sampled rows)")
    check_grad(dk[ki], gk[ki], "dK (sampled keys)")
    check_grad(dv[ki], gv[ki], "dV (sampled keys)")
    for t in (dq, dk, dv):
        assert np.all(np.isfinite(t))
    Hkv = x["k"].shape[1]
    G = x["q"].shape[1] // Hkv
    do_sum = x["do"].astype(np.float64).reshape(dag.T, Hkv, G, -1).sum(axis=(0, 2))
    dv_sum = dv.sum(axis=0)
    e = np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum)
    say(f"  sum dV vs sum dO: rel {e:.3e}")
    assert e <= GRAD_TOL
    dk_sum = np.abs(dk.sum(axis=0)).max()
    dk_mag = np.abs(dk).sum(axis=0).max()
    say(f"  |sum dK| / sum |dK| = {dk_sum / dk_mag:.3e}")
    assert dk_sum <= GRAD_TOL * dk_mag
    if name != "forest1m":
        _check_head_group0(dag, x, dq, dk, dv)


def _check_head_group0(dag, x, dq, dk, dv):
    """Whole-tensor parity for KV head 0 at full size.  Heads are independent, so the
    oracle over every query row of the first group (query heads 0..G-1, KV head 0) gives
    dK/dV of every key of KV head 0 from all its readers, and dQ of every row of those
    query heads.  The shared prefix (owned once, summing every branch's queries) and the
    mounted spans (their readers' gradients routed into the producer's tokens) are also
    reported on their own."""
    G = x["q"].shape[1] // x["k"].shape[1]
    say(f"  oracle: KV head 0 over all {dag.T} rows")
    gq, gk, gv = A.attn_bwd(x["q"][:, :G], x["k"][:, :1], x["v"][:, :1], x["do"][:, :G],
                            dag.branches, dag.mounts)
    check_grad(dq[:, :G], gq, "dQ (heads of KV head 0, all rows)")
    check_grad(dk[:, :1], gk, "dK (KV head 0, all keys)")
    check_grad(dv[:, :1], gv, "dV (KV head 0, all keys)")
    roots = [(int(s), int(s + L)) for (p, f, s, L) in dag.branches if p < 0]
    pk = np.concatenate([np.arange(lo, hi) for lo, hi in roots])
    check_grad(dk[pk, :1], gk[pk], "dK (shared prefix, KV head 0)")
    check_grad(dv[pk, :1], gv[pk], "dV (shared prefix, KV head 0)")
    spans = [(int(dag.branches[p_, 2]) + int(s_), int(dag.branches[p_, 2]) + int(e_))
             for (r_, rp_, p_, s_, e_) in dag.mounts]
    if spans:
        mk = np.concatenate([np.arange(lo, hi) for lo, hi in _merge(spans)])
        check_grad(dk[mk, :1], gk[mk], "dK (mounted spans, KV head 0)")
        check_grad(dv[mk, :1], gv[mk], "dV (mounted spans, KV head 0)")


def test_bwd_workspace_error():
    import torch
    import tree_packed_block_amd as tpb
    dag, x = workload("tiny", 1, 1, 64, "fp32", 1.0, with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "fp32") for k, v in x.items()}
    o, lse = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"], ws=small)
    assert ei.value.name == "EWORKSPACE"


def test_fwd_bwd_on_a_side_stream():
    """Work enqueued on a stream other than the current one, with outputs and workspaces
    allocated by the binding: equal to the same calls on the current stream."""
    import torch
    import tree_packed_block_amd as tpb
    say("case fwd+bwd on a side stream")
    dag, x = workload("episode_small", 16, 4, 128, "bf16", 0.5, with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "bf16") for k, v in x.items()}
    o0, l0 = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
    g0 = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o0, l0, t["do"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o1, l1 = tpb.attn_fwd(plan, t["q"], t["k"], t["v"], stream=side)
    g1 = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o1, l1, t["do"], stream=side)
    # the current stream allocates and writes while the side stream still runs
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    for a, b in zip(g1, g0):
        assert torch.equal(a, b)


def test_fwd_bwd_and_decode_are_deterministic():
    """No step sums with atomics (one writer per dK/dV row, dQ per query tile, decode
    splits merged in a fixed order), so repeated calls give the same bits."""
    import torch
    import tree_packed_block_amd as tpb
    say("case determinism: fwd, bwd and decode twice")
    dag, x = workload("episode_mid", with_dout=True)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "bf16") for k, v in x.items()}
    runs = []
    for _ in range(2):
        o, lse = tpb.attn_fwd(plan, t["q"], t["k"], t["v"])
        g = tpb.attn_bwd(plan, t["q"], t["k"], t["v"], o, lse, t["do"])
        torch.cuda.synchronize()
        runs.append((o, lse) + tuple(g))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), *runs):
        assert torch.equal(a, b), f"{name} differs between two identical calls"
    wl = synth.decode_workload(seed=7, n_cursors=9, prefix=300, own_max=700, span_max=200)
    xd = synth.draw_decode_inputs(np.random.default_rng(3), len(wl.cursors), 16, 4, 128,
                                  wl.n_pages, wl.page_size)
    segs = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages,
                               wl.page_size, wl.n_pages, wl.cursors, share=True)
    sd = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda() for a in segs]
    qkv = [dev(xd[n], "bf16") for n in ("q", "k_pool", "v_pool")]
    d1 = tpb.paged_mount_decode(*qkv, *sd, n_split=5)
    d2 = tpb.paged_mount_decode(*qkv, *sd, n_split=5)
    torch.cuda.synchronize()
    assert torch.equal(d1[0], d2[0]) and torch.equal(d1[1], d2[1]), "decode differs"
