"""GPU parity of the packed-DAG attention forward against the float64 oracle, called
through the C-ABI library."""

import numpy as np
import pytest

from oracle import attention as A
from parity import (TOL, check_close, dev, fuzz_workload, host, sample_rows, say,
                    workload)

pytestmark = pytest.mark.gpu


def _run_fwd(dag, x, dtype):
    import torch
    import tree_packed_block_amd as tpb
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    o, lse = tpb.attn_fwd(plan, q, k, v)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _full_case(name, dtype, Hq, Hkv, Dh, std=0.5):
    say(f"case fwd {name} {dtype} Hq={Hq} Hkv={Hkv} D={Dh}")
    dag, x = workload(name, Hq, Hkv, Dh, dtype, std)
    o, lse = _run_fwd(dag, x, dtype)
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(o, ro, TOL[dtype], "O")
    check_close(lse, rl, TOL[dtype], "LSE")


def test_fwd_tiny_fp32():
    _full_case("tiny", "fp32", 1, 1, 64, std=1.0)


@pytest.mark.parametrize("Dh", [128, 64])
def test_fwd_episode_small_bf16(Dh):
    _full_case("episode_small", "bf16", 16, 4, Dh)


def test_fwd_episode_small_fp32():
    _full_case("episode_small", "fp32", 4, 2, 128)


def test_fwd_episode_mid_bf16():
    _full_case("episode_mid", "bf16", 16, 4, 128)


def test_fwd_forked_bf16():
    _full_case("forked", "bf16", 16, 4, 128)


def test_fwd_forest_small_bf16():
    """Three trees, branch spans interleaved in the stream: one plan, one launch."""
    _full_case("forest_small", "bf16", 16, 4, 128)


@pytest.mark.parametrize("seed", range(12))
def test_fwd_fuzz_bf16(seed):
    say(f"case fwd fuzz seed={seed}")
    dag, x = fuzz_workload(seed, 4, 2, 128, max_len=300, max_branches=7, max_mounts=5)
    o, lse = _run_fwd(dag, x, "bf16")
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


# Head layouts beyond the common 16/4: an odd group (one head per wave group), one
# query head per KV head, the largest group, and head_dim 64 with an odd group.
HEAD_CASES = [(3, 1, 128), (2, 2, 128), (16, 1, 128), (6, 2, 64), (8, 8, 64)]


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("Hq,Hkv,Dh", HEAD_CASES)
def test_fwd_fuzz_heads_bf16(Hq, Hkv, Dh, seed):
    say(f"case fwd fuzz heads Hq={Hq} Hkv={Hkv} D={Dh} seed={seed}")
    dag, x = fuzz_workload(100 + seed, Hq, Hkv, Dh, max_len=300, max_branches=7,
                           max_mounts=5)
    o, lse = _run_fwd(dag, x, "bf16")
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


@pytest.mark.parametrize("name", ["episode131k", "episode262k", "forest1m"])
def test_fwd_full_size_sampled_rows(name):
    """The full tree through the same launch as the benchmark; the oracle computes
    sampled row ranges (boundaries, mounts, ends) one by one."""
    say(f"case fwd {name} sampled rows")
    dag, x = workload(name, 16, 4, 128, "bf16", 0.5)
    o, lse = _run_fwd(dag, x, "bf16")
    rows = sample_rows(dag)
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts, rows=rows)
    idx = np.concatenate([np.arange(lo, hi) for lo, hi in rows])
    check_close(o[idx], ro[idx], TOL["bf16"], "O")
    check_close(lse[:, idx], rl[:, idx], TOL["bf16"], "LSE")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_fwd_error_paths():
    import torch
    import tree_packed_block_amd as tpb
    dag, x = workload("tiny", 1, 1, 64, "fp32", 1.0)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T)
    q = dev(x["q"], "fp32")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.attn_fwd(plan, q, dev(x["k"], "fp32"), dev(x["v"], "fp32"))
    assert ei.value.name == "ESTATE"
    plan.upload()
    bad = torch.zeros((dag.T, 1, 96), device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.attn_fwd(plan, bad, bad, bad)
    assert ei.value.name == "EUNSUPPORTED"


def test_fwd_workspace_error():
    import torch
    import tree_packed_block_amd as tpb
    dag, x = workload("tiny", 2, 1, 64, "bf16", 1.0)
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    t = {k: dev(v, "bf16") for k, v in x.items()}
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.attn_fwd(plan, t["q"], t["k"], t["v"], ws=small)
    assert ei.value.name == "EWORKSPACE"

