"""GPU parity of the branch-aware gated delta-rule scan against the float64 oracle
(``oracle.recurrent``), through the C-ABI library: fuzzed DAGs (forks at 0 and at the
parent's end, nested forks, mounts that must be ignored), several trees in one plan, and
the full 262,144-token episode tree in the launch configuration the benchmark times.

Tolerance: both sides read the same bf16 inputs; the kernel keeps the state in float32
and rounds o to bf16 (relative 2^-9), so |got - ref| <= 5e-3 + 5e-3 |ref|, tighter than
the 2e-2 bound of the attention outputs (the scan's outputs are ~0.06 in magnitude)."""

import numpy as np
import pytest

import synth
from oracle import recurrent as RC
from parity import check_close, dev, host, say
from test_edge_gpu import EDGE_DAGS

pytestmark = pytest.mark.gpu

SCAN_TOL = 5e-3


def _wide_gates(x, seed):
    """Gates over their whole range instead of the recipe's: alpha exactly 1 (no decay),
    U[0.3, 1) or U[0.02, 0.3) (fast decay), beta exactly 0 (no write), exactly 1 (full
    replacement) or U[0, 1)."""
    rng = np.random.default_rng(seed)
    shape = x["alpha"].shape
    a = rng.integers(0, 3, size=shape)
    x["alpha"] = np.where(a == 0, 1.0, np.where(a == 1, rng.uniform(0.3, 1.0, shape),
                                                rng.uniform(0.02, 0.3, shape))).astype(np.float32)
    bsel = rng.integers(0, 4, size=shape)
    x["beta"] = np.where(bsel == 0, 0.0, np.where(bsel == 1, 1.0, rng.uniform(0.0, 1.0, shape))
                         ).astype(np.float32)
    return x


def _chain_dag():
    """Five levels of nested forks: a 40-token root; a child forked at 17; a grandchild
    forked at 33 of the child; a great-grandchild forked at 0 of the grandchild and another
    at its end; one-token branches forked at the root's end and at 1; a mount that the
    scan must ignore."""
    rows_b = [[-1, 0, 0, 40], [0, 17, 40, 50], [1, 33, 90, 45], [2, 0, 135, 30],
              [2, 45, 165, 31], [0, 40, 196, 1], [1, 1, 197, 1]]
    rows_m = [[3, 5, 1, 10, 20]]
    b = np.asarray(rows_b, dtype=np.int32)
    m = np.asarray(rows_m, dtype=np.int32)
    return synth.Dag("chain", b, m, 198)


def _run(dag, H, seed, wide=False):
    import torch
    import tree_packed_block_amd as tpb
    x = synth.draw_scan_inputs(np.random.default_rng(seed), dag.T, H)
    if wide:
        x = _wide_gates(x, seed + 7)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    o = tpb.gated_delta_scan(plan, dev(x["q"], "bf16"), dev(x["k"], "bf16"),
                             dev(x["v"], "bf16"), torch.from_numpy(x["alpha"]).cuda(),
                             torch.from_numpy(x["beta"]).cuda())
    torch.cuda.synchronize()
    ro, _ = RC.scan(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dag.branches, dag.mounts)
    return host(o), ro


@pytest.mark.parametrize("seed", range(4))
def test_scan_fuzz(seed):
    say(f"case scan fuzz seed={seed}")
    dag = synth.fuzz_dag(np.random.default_rng(700 + seed), max_len=300, max_branches=7,
                         max_mounts=5)
    o, ro = _run(dag, 2, 800 + seed)
    check_close(o, ro, SCAN_TOL, "o")


@pytest.mark.parametrize("name", ["episode_small", "forest_small"])
def test_scan_named(name):
    say(f"case scan {name}")
    dag, _ = synth.build(name)
    o, ro = _run(dag, 4, 11)
    check_close(o, ro, SCAN_TOL, "o")


@pytest.mark.parametrize("seed", range(3))
def test_scan_wide_gates_and_short_branches(seed):
    """Gates over their whole range on fuzzed DAGs of many short branches (one-token
    branches, forks at 0 and at the end, chunks cut at every fork)."""
    say(f"case scan wide gates seed={seed}")
    dag = synth.fuzz_dag(np.random.default_rng(1300 + seed), max_len=70, max_branches=9,
                         max_mounts=3)
    o, ro = _run(dag, 2, 1400 + seed, wide=True)
    check_close(o, ro, SCAN_TOL, "o")


def test_scan_nested_forks():
    say("case scan chain of nested forks")
    o, ro = _run(_chain_dag(), 3, 1500, wide=True)
    check_close(o, ro, SCAN_TOL, "o")


@pytest.mark.timeout(900)
def test_scan_full_episode():
    """262,144 tokens (8,192-token root, 8 workers forked at its end, continuation),
    2 heads, every output against the oracle."""
    say("case scan episode262k H=2")
    dag, _ = synth.build("episode262k")
    o, ro = _run(dag, 2, 12)
    check_close(o, ro, SCAN_TOL, "o")


# ----------------------------------------------------------------------------- backward
#
# Tolerance: dq, dk, dv are rounded to bf16 (relative 2^-9); the state, W and the gated
# score matrices enter the matrix products as bf16 high + low parts (relative 2^-16 per
# operand) and every sum is float32, so the gradients carry the bf16 rounding of the
# outputs plus float32 sums over a chunk and over the carried state gradient.  Each
# tensor is checked elementwise, |got - ref| <= SCAN_GRAD_TOL (|ref| + rms(ref)), and by
# relative Frobenius error <= SCAN_GRAD_TOL.

SCAN_GRAD_TOL = 5e-3


def _check_grad_scan(got, ref, name, tol=SCAN_GRAD_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = tol * (np.abs(ref) + rms)
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    rel = float(np.max(err / np.maximum(np.abs(ref) + rms, 1e-300))) if err.size else 0.0
    say(f"  {name}: rel_fro={fro:.3e} max_err/(|ref|+rms)={rel:.3e} (tol {tol})")
    assert fro <= tol, f"{name}: relative Frobenius error {fro:.3e}"
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} elements outside tolerance"


def _run_bwd(dag, H, seed, wide=False):
    import torch
    import tree_packed_block_amd as tpb
    x = synth.draw_scan_inputs(np.random.default_rng(seed), dag.T, H)
    if wide:
        x = _wide_gates(x, seed + 7)
    do = synth.round_bf16((0.5 * np.random.default_rng(seed + 1).standard_normal(
        x["v"].shape)).astype(np.float32))
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    got = tpb.gated_delta_scan_bwd(plan, dev(x["q"], "bf16"), dev(x["k"], "bf16"),
                                   dev(x["v"], "bf16"), torch.from_numpy(x["alpha"]).cuda(),
                                   torch.from_numpy(x["beta"]).cuda(), dev(do, "bf16"))
    torch.cuda.synchronize()
    got = [host(t) for t in got]
    ref = RC.scan_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], do, dag.branches,
                      dag.mounts)
    for name, a, b in zip(("dq", "dk", "dv", "dalpha", "dbeta"), got, ref):
        _check_grad_scan(a, b, name)


@pytest.mark.parametrize("seed", range(4))
def test_scan_bwd_fuzz(seed):
    say(f"case scan bwd fuzz seed={seed}")
    dag = synth.fuzz_dag(np.random.default_rng(900 + seed), max_len=300, max_branches=7,
                         max_mounts=5)
    _run_bwd(dag, 2, 1000 + seed)


@pytest.mark.parametrize("name", ["episode_small", "forest_small"])
def test_scan_bwd_named(name):
    say(f"case scan bwd {name}")
    dag, _ = synth.build(name)
    _run_bwd(dag, 2, 21)


@pytest.mark.timeout(900)
def test_scan_bwd_full_episode():
    """The 262,144-token episode tree, one head, every gradient against the oracle."""
    say("case scan bwd episode262k H=1")
    dag, _ = synth.build("episode262k")
    _run_bwd(dag, 1, 22)


@pytest.mark.parametrize("seed", range(3))
def test_scan_bwd_wide_gates_and_short_branches(seed):
    say(f"case scan bwd wide gates seed={seed}")
    dag = synth.fuzz_dag(np.random.default_rng(1600 + seed), max_len=70, max_branches=9,
                         max_mounts=3)
    _run_bwd(dag, 2, 1700 + seed, wide=True)


def test_scan_bwd_nested_forks():
    say("case scan bwd chain of nested forks")
    _run_bwd(_chain_dag(), 3, 1800, wide=True)


@pytest.mark.parametrize("name", sorted(EDGE_DAGS))
def test_scan_edge_dags_fwd_bwd(name):
    """The packing's degenerate cases (a single token, tile-aligned and one-past-aligned
    streams, forks at 0 and at the end, a child packed before its parent, mounted spans of
    any producer, which the scan ignores), gates over their whole range."""
    say(f"case scan edge {name}")
    rows_b, rows_m = EDGE_DAGS[name]
    b = np.asarray(rows_b, dtype=np.int32).reshape(-1, 4)
    m = np.asarray(rows_m, dtype=np.int32).reshape(-1, 5)
    dag = synth.Dag(name, b, m, int(b[:, 3].sum()))
    o, ro = _run(dag, 2, 1900, wide=True)
    check_close(o, ro, SCAN_TOL, "o")
    _run_bwd(dag, 2, 1950, wide=True)


@pytest.mark.parametrize("name", ["episode_small", "forest_small"])
def test_scan_save_then_bwd_saved(name):
    """The training pair (forward keeping its chunk states, backward without replaying the
    forward) gives bit for bit the outputs and gradients of the plain forward and backward,
    also when the backward runs a second time on the same workspace with another dO."""
    import torch
    import tree_packed_block_amd as tpb
    say(f"case scan save + bwd_saved {name}")
    dag, _ = synth.build(name)
    H = 2
    x = synth.draw_scan_inputs(np.random.default_rng(31), dag.T, H)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = [dev(x[n], "bf16") for n in ("q", "k", "v")]
    a, b = torch.from_numpy(x["alpha"]).cuda(), torch.from_numpy(x["beta"]).cuda()
    o_ref = tpb.gated_delta_scan(plan, *t, a, b)
    o, ws = tpb.gated_delta_scan_save(plan, *t, a, b)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "forward outputs differ"
    for seed in (32, 33):
        do = dev(synth.round_bf16((0.5 * np.random.default_rng(seed).standard_normal(
            x["v"].shape)).astype(np.float32)), "bf16")
        ref = tpb.gated_delta_scan_bwd(plan, *t, a, b, do)
        got = tpb.gated_delta_scan_bwd_saved(plan, *t, a, b, do, ws)
        torch.cuda.synchronize()
        for nm, g1, g2 in zip(("dq", "dk", "dv", "dalpha", "dbeta"), got, ref):
            assert torch.equal(g1, g2), f"{nm} differs from the plain backward (dO seed {seed})"
    say("  identical to the plain forward and backward")


def test_scan_on_a_side_stream():
    """The scan runs part of its work on a second stream of its own, forked from and joined
    back into the caller's stream.  On a caller's side stream, with the inputs written on that
    stream just before the call and the outputs read on it right after, forward, backward and
    the training pair give the same bits as on the current stream."""
    import torch
    import tree_packed_block_amd as tpb
    say("case scan on a side stream")
    dag, _ = synth.build("episode_small")
    H = 2
    x = synth.draw_scan_inputs(np.random.default_rng(41), dag.T, H)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = [dev(x[n], "bf16") for n in ("q", "k", "v")]
    a, b = torch.from_numpy(x["alpha"]).cuda(), torch.from_numpy(x["beta"]).cuda()
    do = dev(synth.round_bf16((0.5 * np.random.default_rng(42).standard_normal(
        x["v"].shape)).astype(np.float32)), "bf16")
    o_ref = tpb.gated_delta_scan(plan, *t, a, b)
    g_ref = tpb.gated_delta_scan_bwd(plan, *t, a, b, do)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        # inputs produced on the side stream right before the calls: the scan's own second
        # stream must start after them
        t2 = [torch.empty_like(z) for z in t]
        for dst, src in zip(t2, t):
            dst.copy_(src)
        a2, b2, do2 = a.clone(), b.clone(), do.clone()
        o = tpb.gated_delta_scan(plan, *t2, a2, b2, stream=side)
        g = tpb.gated_delta_scan_bwd(plan, *t2, a2, b2, do2, stream=side)
        o_s, ws = tpb.gated_delta_scan_save(plan, *t2, a2, b2, stream=side)
        g_s = tpb.gated_delta_scan_bwd_saved(plan, *t2, a2, b2, do2, ws, stream=side)
        # outputs consumed on the side stream right after: the joins must come first
        outs = [z.clone() for z in (o, *g, o_s, *g_s)]
    side.synchronize()
    refs = (o_ref, *g_ref, o_ref, *g_ref)
    names = ("o", "dq", "dk", "dv", "dalpha", "dbeta") * 2
    for nm, got, ref in zip(names, outs, refs):
        assert torch.equal(got, ref), f"{nm} differs on a side stream"
    say("  identical on a side stream")


def test_scan_entry_points_reject_bad_arguments():
    """Errors found on the host with an uploaded plan, before any launch: unsupported
    head sizes and dtypes, NULL tensors, a workspace that is too small."""
    import ctypes
    import torch
    import tree_packed_block_amd as tpb
    say("case scan error paths")
    dag, _ = synth.build("episode_small")
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    L = tpb.lib()
    H = 2
    buf = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    big = tpb.gdn_bwd_workspace_bytes(plan, H)

    def code(rc):
        return tpb._lib._NAMES.get(rc, rc)

    for fn, n_in in ((L.octopus_gated_delta_scan, 6), (L.octopus_gated_delta_scan_save, 6)):
        args = [p] * n_in
        assert code(fn(plan.handle, tpb.BF16, H, 64, 128, *args, p, big, None)) == "EUNSUPPORTED"
        assert code(fn(plan.handle, tpb.FP32, H, 128, 128, *args, p, big, None)) == "EUNSUPPORTED"
        assert code(fn(plan.handle, tpb.BF16, H, 128, 128, None, *args[1:], p, big,
                       None)) == "EINVAL"
        assert code(fn(plan.handle, tpb.BF16, H, 128, 128, *args, p, 16, None)) == "EWORKSPACE"
    for fn in (L.octopus_gated_delta_scan_bwd, L.octopus_gated_delta_scan_bwd_saved):
        args = [p] * 11
        assert code(fn(plan.handle, tpb.BF16, H, 128, 64, *args, p, big, None)) == "EUNSUPPORTED"
        assert code(fn(plan.handle, tpb.BF16, 0, 128, 128, *args, p, big, None)) == "EINVAL"
        assert code(fn(plan.handle, tpb.BF16, H, 128, 128, *args[:5], None, *args[6:], p, big,
                       None)) == "EINVAL"
        assert code(fn(plan.handle, tpb.BF16, H, 128, 128, *args, p, big - 1,
                       None)) == "EWORKSPACE"
