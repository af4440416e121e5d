"""GPU parity of paged mounted extend (several new tokens per cursor) against the
float64 oracle, through the C-ABI library: small batches in full, fuzzed DAGs with every
branch a cursor (mounts issued inside the new tokens, odd and large query-head groups),
one new token against decode, and the full 64-cursor batch on sampled rows."""

import numpy as np
import pytest

import synth
from oracle import decode as DEC
from parity import TOL, check_close, dev, host, say

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _q_ptr(n_new):
    return np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)


def _gpu_extend(wl, n_new, x, dtype="bf16"):
    import torch
    import tree_packed_block_amd as tpb
    segs = tpb.extend_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages,
                               wl.page_size, wl.n_pages, wl.cursors, n_new)
    sp, pg, lo, hi, thr, causal, first = segs
    q, kp, vp = dev(x["q"], dtype), dev(x["k_pool"], dtype), dev(x["v_pool"], dtype)
    o, lse = tpb.paged_mount_extend(q, kp, vp, _i32(_q_ptr(n_new)), int(max(n_new)),
                                    _i32(first), _i32(sp), _i32(pg), _i32(lo), _i32(hi),
                                    _i32(thr), _i32(causal))
    torch.cuda.synchronize()
    return host(o), host(lse)


def _oracle(wl, n_new, x, only=None):
    return DEC.extend(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                      wl.page_ptr, wl.pages, wl.page_size, wl.cursors, _q_ptr(n_new),
                      only=only)


def _inputs(wl, n_new, Hq, Hkv, seed=77, Dh=128, dtype="bf16"):
    return synth.draw_extend_inputs(np.random.default_rng(seed), int(np.sum(n_new)), Hq, Hkv,
                                    Dh, wl.n_pages, wl.page_size, dtype=dtype)


def test_extend_small():
    """Six cursors over a 256-token shared prefix with mounts; 1 to 299 new tokens each
    (one or three 128-token tiles, ragged tails)."""
    say("case extend small")
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=64)
    L = wl.dag.branches[wl.cursors, 3]
    n_new = np.minimum(L, np.random.default_rng(9).integers(1, 300, size=len(L)))
    x = _inputs(wl, n_new, 16, 4)
    o, lse = _gpu_extend(wl, n_new, x)
    ro, rl = _oracle(wl, n_new, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


@pytest.mark.parametrize("Dh,dtype", [(64, "bf16"), (64, "fp32"), (128, "fp32")])
def test_extend_small_head_dims_and_fp32(Dh, dtype):
    """head_dim 64 (bf16 MFMA kernel) and float32 pools (exact float32 kernel)."""
    say(f"case extend small D={Dh} {dtype}")
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=64)
    L = wl.dag.branches[wl.cursors, 3]
    n_new = np.minimum(L, np.random.default_rng(9).integers(1, 300, size=len(L)))
    x = _inputs(wl, n_new, 8, 2, Dh=Dh, dtype=dtype)
    o, lse = _gpu_extend(wl, n_new, x, dtype=dtype)
    ro, rl = _oracle(wl, n_new, x)
    check_close(o, ro, TOL[dtype], "O")
    check_close(lse, rl, TOL[dtype], "LSE")


@pytest.mark.parametrize("seed", range(2))
def test_extend_fuzz_head_dim_64(seed):
    say(f"case extend fuzz D=64 seed={seed}")
    rng = np.random.default_rng(400 + seed)
    dag = synth.fuzz_dag(rng, max_len=300, max_branches=7, max_mounts=6)
    n_pages, ptr, pages = synth.dags.assign_pages(dag, 64, rng)
    wl = synth.DecodeWorkload(dag, 64, n_pages, ptr, pages, np.arange(dag.nb, dtype=np.int32))
    n_new = np.array([int(rng.integers(1, L + 1)) for L in dag.branches[:, 3]])
    x = _inputs(wl, n_new, 6, 2, seed=500 + seed, Dh=64)
    o, lse = _gpu_extend(wl, n_new, x)
    ro, rl = _oracle(wl, n_new, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (3, 1), (16, 1)])
@pytest.mark.parametrize("seed", range(3))
def test_extend_fuzz(seed, Hq, Hkv):
    say(f"case extend fuzz seed={seed} Hq={Hq} Hkv={Hkv}")
    rng = np.random.default_rng(200 + seed)
    dag = synth.fuzz_dag(rng, max_len=300, max_branches=7, max_mounts=6)
    n_pages, ptr, pages = synth.dags.assign_pages(dag, 64, rng)
    wl = synth.DecodeWorkload(dag, 64, n_pages, ptr, pages, np.arange(dag.nb, dtype=np.int32))
    n_new = np.array([int(rng.integers(1, L + 1)) for L in dag.branches[:, 3]])
    x = _inputs(wl, n_new, Hq, Hkv, seed=300 + seed)
    o, lse = _gpu_extend(wl, n_new, x)
    ro, rl = _oracle(wl, n_new, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


def test_extend_one_token_matches_decode():
    import torch
    import tree_packed_block_amd as tpb
    say("case extend one token vs decode")
    wl = synth.decode_workload(seed=5, n_cursors=8, prefix=512, own_max=700, span_max=200,
                               page_size=64)
    n_new = np.ones(len(wl.cursors), dtype=np.int32)
    x = _inputs(wl, n_new, 16, 4)
    o, lse = _gpu_extend(wl, n_new, x)
    segs = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages, 64,
                               wl.n_pages, wl.cursors)
    od, ld = tpb.paged_mount_decode(dev(x["q"], "bf16"), dev(x["k_pool"], "bf16"),
                                    dev(x["v_pool"], "bf16"), *[_i32(s) for s in segs],
                                    n_split=4)
    torch.cuda.synchronize()
    check_close(o, host(od), TOL["bf16"], "extend O vs decode O")
    check_close(lse, host(ld), TOL["bf16"], "extend LSE vs decode LSE")
    ro, rl = DEC.decode(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                        wl.page_ptr, wl.pages, 64, wl.cursors)
    check_close(o, ro, TOL["bf16"], "O vs decode oracle")


@pytest.mark.timeout(900)
def test_extend_full_batch_sampled_rows():
    """64 cursors (16K shared prefix, private branches up to 32K, mounted spans up to 8K),
    each appending 256 to 2048 new tokens, through the launch the benchmark times; the
    oracle computes sampled rows: the first and last new tokens, the last rows of the
    first tile, and the rows at each mount issued inside the new tokens."""
    say("case extend 64 cursors sampled")
    wl, n_new = synth.extend_workload()
    x = _inputs(wl, n_new, 16, 4)
    o, lse = _gpu_extend(wl, n_new, x)
    q_ptr = _q_ptr(n_new)
    br = wl.dag.branches
    only = set()
    for c, b in enumerate(wl.cursors):
        m, L = int(n_new[c]), int(br[b, 3])
        js = {0, 1, m - 1, min(127, m - 1), min(128, m - 1)}
        for (reader, rpos, producer, s, e) in wl.dag.mounts:
            if reader == b and rpos >= L - m:
                js |= {rpos - (L - m), max(0, rpos - (L - m) - 1)}
        only |= {int(q_ptr[c]) + j for j in js if 0 <= j < m}
    rows = np.array(sorted(only))
    say(f"  oracle rows: {len(rows)}")
    ro, rl = _oracle(wl, n_new, x, only=only)
    check_close(o[rows], ro[rows], TOL["bf16"], "O (sampled rows)")
    check_close(lse[rows], rl[rows], TOL["bf16"], "LSE (sampled rows)")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_extend_argument_errors():
    import torch
    import tree_packed_block_amd as tpb
    z = torch.zeros(4, dtype=torch.int32, device="cuda")
    q = torch.zeros((2, 16, 96), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((4, 4, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.paged_mount_extend(q, kp, kp, z[:2], 2, z[:1], z[:2], z, z, z, z, z)
    assert ei.value.name == "EUNSUPPORTED"
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((4, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.paged_mount_extend(q, kp, kp, z[:2], 0, z[:1], z[:2], z, z, z, z, z)
    assert ei.value.name == "EINVAL"
