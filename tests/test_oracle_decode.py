"""Pins of the decode and extend oracles: brute force over Python sets, consistency
with the packed forward when the pool holds the packed K/V, the K = 0 closed form, the
zero-copy property of mounts, and extend with one new token per cursor = decode."""

import math

import numpy as np

import synth
from oracle import dag as D
from oracle import attention as A
from oracle import decode as DEC


def _pool_from_packed(dag, k, v, page_size, seed):
    n_pages, ptr, pages = synth.dags.assign_pages(dag, page_size, np.random.default_rng(seed))
    Hkv, Dh = k.shape[1], k.shape[2]
    kp = np.full((n_pages, Hkv, page_size, Dh), np.nan)
    vp = np.full((n_pages, Hkv, page_size, Dh), np.nan)
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        for r in range(L):
            pg = pages[ptr[b] + r // page_size]
            kp[pg, :, r % page_size] = k[start + r]
            vp[pg, :, r % page_size] = v[start + r]
    return kp, vp, ptr, pages


def test_decode_equals_packed_forward_row():
    """Decoding the last token of every branch from pages reproduces the packed
    forward's row of that token (the rollout graph and the packed trainer agree)."""
    dag, _ = synth.build("episode_small")
    rng = np.random.default_rng(4)
    q = rng.standard_normal((dag.T, 4, 16))
    k = rng.standard_normal((dag.T, 2, 16))
    v = rng.standard_normal((dag.T, 2, 16))
    O, LSE = A.attn_fwd(q, k, v, dag.branches, dag.mounts)
    kp, vp, ptr, pages = _pool_from_packed(dag, k, v, 16, 1)
    cursors = np.arange(dag.nb)
    last = dag.branches[:, 2] + dag.branches[:, 3] - 1
    Od, Ld = DEC.decode(q[last], kp, vp, dag.branches, dag.mounts, ptr, pages, 16, cursors)
    np.testing.assert_allclose(Od, O[last], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Ld, LSE[:, last].T, rtol=1e-12, atol=1e-12)


def test_decode_brute_force_sets():
    dag = synth.fuzz_dag(np.random.default_rng(21), max_len=20)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((dag.T, 1, 4))
    v = rng.standard_normal((dag.T, 1, 4))
    kp, vp, ptr, pages = _pool_from_packed(dag, k, v, 4, 2)
    qd = rng.standard_normal((dag.nb, 2, 4))
    cursors = np.arange(dag.nb)
    Od, Ld = DEC.decode(qd, kp, vp, dag.branches, dag.mounts, ptr, pages, 4, cursors)
    for c, b in enumerate(cursors):
        start, L = int(dag.branches[b, 2]), int(dag.branches[b, 3])
        vis = sorted(D.visible(dag.branches, dag.mounts, start + L - 1))
        for h in range(2):
            s = [sum(qd[c, h, d] * k[j, 0, d] for d in range(4)) / 2.0 for j in vis]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            o = [sum(w[n] * v[j, 0, d] for n, j in enumerate(vis)) / tot for d in range(4)]
            assert abs(Ld[c, h] - (m + math.log(tot))) < 1e-12
            np.testing.assert_allclose(Od[c, h], o, rtol=1e-12, atol=1e-12)


def test_decode_zero_keys_and_zero_copy():
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300,
                               span_max=100, page_size=16)
    rng = np.random.default_rng(0)
    Hkv, Dh = 2, 8
    kp = np.zeros((wl.n_pages, Hkv, 16, Dh))
    vp = rng.standard_normal((wl.n_pages, Hkv, 16, Dh))
    q = rng.standard_normal((len(wl.cursors), 4, Dh))
    O, L = DEC.decode(q, kp, vp, wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages,
                      16, wl.cursors)
    for c, b in enumerate(wl.cursors):
        idx = DEC.cursor_tokens(wl.dag.branches, wl.dag.mounts, int(b))
        page, slot = DEC.physical_slots(wl.dag.branches, wl.page_ptr, wl.pages, 16, idx)
        # every visible token is read in place from a page its owner holds: mounts
        # add no pages beyond the page table
        owned = set(wl.pages.tolist())
        assert set(page.tolist()) <= owned
        assert len(set(zip(page.tolist(), slot.tolist()))) == len(idx)
        mean = vp[page, :, slot, :].mean(axis=0)  # [Hkv, D]
        np.testing.assert_allclose(L[c], np.log(len(idx)), atol=1e-12)
        np.testing.assert_allclose(O[c], np.repeat(mean, 2, axis=0), rtol=1e-12, atol=1e-12)


def _extend_rows(dag, m):
    """q_ptr for the last ``m[b]`` own tokens of every branch, and their packed rows."""
    q_ptr = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    rows = np.concatenate([np.arange(int(dag.branches[b, 2] + dag.branches[b, 3] - m[b]),
                                     int(dag.branches[b, 2] + dag.branches[b, 3]))
                           for b in range(dag.nb)])
    return q_ptr, rows


def test_extend_equals_packed_forward_rows():
    """The new tokens of every branch, read from pages, give the packed forward's rows
    of those tokens: causal among themselves, mounts seen from their reader offset on."""
    dag, _ = synth.build("episode_small")
    rng = np.random.default_rng(8)
    q = rng.standard_normal((dag.T, 4, 16))
    k = rng.standard_normal((dag.T, 2, 16))
    v = rng.standard_normal((dag.T, 2, 16))
    O, LSE = A.attn_fwd(q, k, v, dag.branches, dag.mounts)
    kp, vp, ptr, pages = _pool_from_packed(dag, k, v, 16, 3)
    m = np.minimum(dag.branches[:, 3], rng.integers(1, 120, size=dag.nb))
    q_ptr, rows = _extend_rows(dag, m)
    Oe, Le = DEC.extend(q[rows], kp, vp, dag.branches, dag.mounts, ptr, pages, 16,
                        np.arange(dag.nb), q_ptr)
    np.testing.assert_allclose(Oe, O[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Le, LSE[:, rows].T, rtol=1e-12, atol=1e-12)


def test_extend_one_token_is_decode():
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300,
                               span_max=100, page_size=16)
    x = synth.draw_decode_inputs(np.random.default_rng(2), len(wl.cursors), 4, 2, 8,
                                 wl.n_pages, 16, dtype="fp32")
    Od, Ld = DEC.decode(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                        wl.page_ptr, wl.pages, 16, wl.cursors)
    Oe, Le = DEC.extend(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                        wl.page_ptr, wl.pages, 16, wl.cursors,
                        np.arange(len(wl.cursors) + 1))
    np.testing.assert_allclose(Oe, Od, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Le, Ld, rtol=1e-13, atol=1e-13)


def test_extend_brute_force_sets():
    """Several new tokens per branch on a fuzzed DAG (mounts inside the new tokens
    included), against Python sets of the visibility definition."""
    dag = synth.fuzz_dag(np.random.default_rng(33), max_len=24, max_mounts=5)
    rng = np.random.default_rng(6)
    k = rng.standard_normal((dag.T, 1, 4))
    v = rng.standard_normal((dag.T, 1, 4))
    kp, vp, ptr, pages = _pool_from_packed(dag, k, v, 4, 7)
    m = np.minimum(dag.branches[:, 3], rng.integers(1, 9, size=dag.nb))
    q_ptr, rows = _extend_rows(dag, m)
    qe = rng.standard_normal((len(rows), 2, 4))
    Oe, Le = DEC.extend(qe, kp, vp, dag.branches, dag.mounts, ptr, pages, 4,
                        np.arange(dag.nb), q_ptr)
    for r, i in enumerate(rows):
        vis = sorted(D.visible(dag.branches, dag.mounts, int(i)))
        for h in range(2):
            s = [sum(qe[r, h, d] * k[j, 0, d] for d in range(4)) / 2.0 for j in vis]
            mx = max(s)
            w = [math.exp(t - mx) for t in s]
            tot = sum(w)
            o = [sum(w[n] * v[j, 0, d] for n, j in enumerate(vis)) / tot for d in range(4)]
            assert abs(Le[r, h] - (mx + math.log(tot))) < 1e-12
            np.testing.assert_allclose(Oe[r, h], o, rtol=1e-12, atol=1e-12)
