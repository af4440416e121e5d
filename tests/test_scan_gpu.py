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

pytestmark = pytest.mark.gpu

SCAN_TOL = 5e-3


def _run(dag, H, seed):
    import torch
    import tree_packed_block_amd as tpb
    x = synth.draw_scan_inputs(np.random.default_rng(seed), dag.T, H)
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


def _run_bwd(dag, H, seed):
    import torch
    import tree_packed_block_amd as tpb
    x = synth.draw_scan_inputs(np.random.default_rng(seed), dag.T, H)
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
