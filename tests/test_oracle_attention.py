"""Pins of the oracle's forward and backward: library reductions (torch on the CPU in
float64), the flattened-path formulation, closed forms, finite differences."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import synth
from oracle import dag as D
from oracle import attention as A
from conftest import read_golden


def _inputs(seed, T, Hq, Hkv, Dh):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, Dh))
    k = rng.standard_normal((T, Hkv, Dh))
    v = rng.standard_normal((T, Hkv, Dh))
    do = rng.standard_normal((T, Hq, Dh))
    return q, k, v, do


def _causal_torch(q, k, v, scale):
    """Ordinary causal attention via torch's fused routine (float64, CPU)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_single_branch_equals_causal_sdpa():
    T, H, Dh = 70, 2, 16
    q, k, v, _ = _inputs(0, T, H, H, Dh)
    br = np.array([[-1, 0, 0, T]])
    O, _ = A.attn_fwd(q, k, v, br, np.zeros((0, 5)), block=32)
    ref = _causal_torch(q, k, v, 1 / np.sqrt(Dh))
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10**9))
def test_packed_rows_equal_flattened_path_attention(seed):
    """The packed output of g(b, r) equals ordinary causal attention over branch b's
    flattened root-to-branch path (spans spliced at their offsets, repeated keys
    kept once) at the position of g(b, r)."""
    dag = synth.fuzz_dag(np.random.default_rng(seed), max_len=24)
    q, k, v, _ = _inputs(seed % 1000, dag.T, 2, 1, 8)
    O, LSE = A.attn_fwd(q, k, v, dag.branches, dag.mounts, block=16)
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        seq = np.array(D.dedup_first(D.flatten_path(dag.branches, dag.mounts, b)))
        ref = _causal_torch(q[seq], np.repeat(k[seq], 2, axis=1),
                            np.repeat(v[seq], 2, axis=1), 1 / np.sqrt(8))
        where = {int(t): n for n, t in enumerate(seq)}
        for r in range(L):
            np.testing.assert_allclose(O[start + r], ref[where[start + r]], rtol=1e-11,
                                       atol=1e-11)


def test_zero_keys_closed_form():
    """K = 0: every visible score is 0, so LSE = ln|Ctx| and O = mean of visible V."""
    dag, _ = synth.build("tiny")
    nnz, ctx448 = read_golden("tiny_nnz.txt")
    rng = np.random.default_rng(3)
    q = rng.standard_normal((dag.T, 1, 64))
    k = np.zeros((dag.T, 1, 64))
    v = rng.standard_normal((dag.T, 1, 64))
    O, LSE = A.attn_fwd(q, k, v, dag.branches, dag.mounts)
    M = D.mask(dag.branches, dag.mounts, dag.T)
    cnt = M.sum(axis=1)
    np.testing.assert_allclose(LSE[0], np.log(cnt), rtol=0, atol=1e-12)
    assert abs(LSE[0, 448] - np.log(ctx448)) < 1e-12
    mean = (M.astype(np.float64) @ v[:, 0, :]) / cnt[:, None]
    np.testing.assert_allclose(O[:, 0, :], mean, rtol=1e-12, atol=1e-12)


def test_constant_values():
    dag, _ = synth.build("episode_small")
    q, k, _, _ = _inputs(5, dag.T, 2, 2, 8)
    v = np.full((dag.T, 2, 8), 0.375)
    O, _ = A.attn_fwd(q, k, v, dag.branches, dag.mounts)
    np.testing.assert_allclose(O, 0.375, rtol=1e-13)


def test_gqa_equals_repeated_heads():
    dag = synth.fuzz_dag(np.random.default_rng(11), max_len=30)
    q, k, v, do = _inputs(1, dag.T, 4, 2, 8)
    O1, L1 = A.attn_fwd(q, k, v, dag.branches, dag.mounts)
    O2, L2 = A.attn_fwd(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1),
                        dag.branches, dag.mounts)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=1e-13, atol=1e-13)
    g1 = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts)
    g2 = A.attn_bwd(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), do,
                    dag.branches, dag.mounts)
    np.testing.assert_allclose(g1[0], g2[0], rtol=1e-12, atol=1e-12)
    # the grouped gradient sums the two repeated heads
    np.testing.assert_allclose(g1[1], g2[1][:, 0::2] + g2[1][:, 1::2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1[2], g2[2][:, 0::2] + g2[2][:, 1::2], rtol=1e-12, atol=1e-12)


def test_row_subsets_and_block_sizes_agree():
    dag, _ = synth.build("episode_small")
    q, k, v, do = _inputs(2, dag.T, 2, 1, 16)
    O, L = A.attn_fwd(q, k, v, dag.branches, dag.mounts, block=256)
    rows = [(0, 100), (1500, 1700), (2900, 3000)]
    O2, L2 = A.attn_fwd(q, k, v, dag.branches, dag.mounts, rows=rows, block=64, workers=1)
    for lo, hi in rows:
        np.testing.assert_allclose(O2[lo:hi], O[lo:hi], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(L2[:, lo:hi], L[:, lo:hi], rtol=1e-13, atol=1e-13)
    g = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts, block=100)
    g2 = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts, block=256, workers=1)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------- backward

def _loss(q, k, v, do, dag):
    O, _ = A.attn_fwd(q, k, v, dag.branches, dag.mounts, workers=1)
    return float(np.sum(O * do))


def test_backward_finite_differences():
    dag = synth.fuzz_dag(np.random.default_rng(7), max_len=12, max_branches=4)
    q, k, v, do = _inputs(4, dag.T, 2, 1, 4)
    dQ, dK, dV = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts, workers=1)
    rng = np.random.default_rng(9)
    eps = 1e-5
    for which, grad in (("q", dQ), ("k", dK), ("v", dV)):
        for _ in range(3):
            u = rng.standard_normal(grad.shape)
            args = {"q": q, "k": k, "v": v}
            plus = dict(args)
            minus = dict(args)
            plus[which] = args[which] + eps * u
            minus[which] = args[which] - eps * u
            fd = (_loss(plus["q"], plus["k"], plus["v"], do, dag)
                  - _loss(minus["q"], minus["k"], minus["v"], do, dag)) / (2 * eps)
            an = float(np.sum(grad * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_backward_matches_torch_autograd_on_dense_mask():
    dag, _ = synth.build("episode_small")
    q, k, v, do = _inputs(8, dag.T, 4, 2, 8)
    dQ, dK, dV = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts)
    M = torch.from_numpy(D.mask(dag.branches, dag.mounts, dag.T))
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kr = kt.repeat_interleave(2, dim=1)
    vr = vt.repeat_interleave(2, dim=1)
    S = torch.einsum("ihd,jhd->hij", qt, kr) / np.sqrt(8)
    S = S.masked_fill(~M[None], float("-inf"))
    O = torch.einsum("hij,jhd->ihd", torch.softmax(S, dim=-1), vr)
    (O * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dQ, qt.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dK, kt.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dV, vt.grad.numpy(), rtol=1e-10, atol=1e-10)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10**9))
def test_backward_path_scatter_add(seed):
    """Single ownership: run each branch's flattened path through causal attention
    with dO only on that branch's own rows, scatter-add the path's dK/dV into the
    packed tokens the path copied them from, sum over branches; this equals the
    packed dK/dV (and the path dQ equals the packed dQ on the branch's rows)."""
    dag = synth.fuzz_dag(np.random.default_rng(seed), max_len=16)
    q, k, v, do = _inputs(seed % 997, dag.T, 2, 1, 4)
    dQ, dK, dV = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts, workers=1)
    sK = np.zeros_like(dK)
    sV = np.zeros_like(dV)
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        seq = np.array(D.dedup_first(D.flatten_path(dag.branches, dag.mounts, b)))
        own = (seq >= start) & (seq < start + L)
        qt = torch.tensor(q[seq], requires_grad=True)
        kt = torch.tensor(k[seq], requires_grad=True)
        vt = torch.tensor(v[seq], requires_grad=True)
        n = len(seq)
        S = torch.einsum("ihd,jhd->hij", qt, kt.repeat_interleave(2, 1)) / 2.0
        causal = torch.tril(torch.ones(n, n, dtype=torch.bool))
        S = S.masked_fill(~causal[None], float("-inf"))
        O = torch.einsum("hij,jhd->ihd", torch.softmax(S, -1), vt.repeat_interleave(2, 1))
        w = torch.from_numpy(do[seq] * own[:, None, None])
        (O * w).sum().backward()
        np.add.at(sK, seq, kt.grad.numpy())
        np.add.at(sV, seq, vt.grad.numpy())
        np.testing.assert_allclose(dQ[seq[own]], qt.grad.numpy()[own], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dK, sK, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dV, sV, rtol=1e-10, atol=1e-10)


def test_backward_closed_forms():
    dag, _ = synth.build("tiny")
    rng = np.random.default_rng(12)
    T = dag.T
    q = rng.standard_normal((T, 2, 8))
    v = rng.standard_normal((T, 1, 8))
    do = rng.standard_normal((T, 2, 8))
    # all key rows equal: the softmax is uniform whatever Q is, so dQ = 0
    k = np.tile(rng.standard_normal((1, 1, 8)), (T, 1, 1))
    dQ, _, _ = A.attn_bwd(q, k, v, do, dag.branches, dag.mounts)
    assert np.abs(dQ).max() < 1e-12
    # K = 0: dV_j = sum over heads and over the queries i that see j of dO_i / |Ctx(i)|
    k0 = np.zeros((T, 1, 8))
    _, _, dV = A.attn_bwd(q, k0, v, do, dag.branches, dag.mounts)
    M = D.mask(dag.branches, dag.mounts, T).astype(np.float64)
    cnt = M.sum(axis=1)
    want = M.T @ ((do[:, 0, :] + do[:, 1, :]) / cnt[:, None])
    np.testing.assert_allclose(dV[:, 0, :], want, rtol=1e-12, atol=1e-12)
