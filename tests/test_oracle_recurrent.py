"""Pins of the recurrent-scan oracle: hand-derived outputs of one and two tokens with
gates strictly between 0 and 1 (which fix where alpha and beta enter the update), every
branch equals the plain recurrence run from zero over its flattened root-to-branch token
path (an independent formulation of the fork checkpoints), the delta rule stores and
retrieves values under orthonormal keys, beta = 0 keeps the inherited state, alpha gates
it, and mounts change nothing."""

import numpy as np

import synth
from oracle import recurrent as RC


def _inputs(rng, T, H, Dk, Dv):
    q = rng.standard_normal((T, H, Dk))
    k = rng.standard_normal((T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, Dv))
    a = rng.uniform(0.8, 1.0, size=(T, H))
    b = rng.uniform(0.1, 0.9, size=(T, H))
    return q, k, v, a, b


def _plain(q, k, v, a, b):
    """The recurrence over one sequence, written out per head with plain loops."""
    T, H, Dk = q.shape
    Dv = v.shape[2]
    o = np.zeros((T, H, Dv))
    for h in range(H):
        S = np.zeros((Dv, Dk))
        for t in range(T):
            S = a[t, h] * (S - b[t, h] * np.outer(S @ k[t, h], k[t, h])) \
                + b[t, h] * np.outer(v[t, h], k[t, h])
            o[t, h] = S @ q[t, h]
    return o


def _two_tokens(k1, k2, v1, v2, q1, q2, a1, a2, b1, b2):
    T = 2
    q = np.array([q1, q2], dtype=np.float64).reshape(T, 1, -1)
    k = np.array([k1, k2], dtype=np.float64).reshape(T, 1, -1)
    v = np.array([v1, v2], dtype=np.float64).reshape(T, 1, -1)
    a = np.array([[a1], [a2]], dtype=np.float64)
    b = np.array([[b1], [b2]], dtype=np.float64)
    o, _ = RC.scan(q, k, v, a, b, np.array([[-1, 0, 0, T]]))
    return o[:, 0]


def test_gated_delta_rule_hand_derived():
    """Worked by hand from S_t = a_t (S_{t-1} - b_t (S_{t-1} k_t) k_t^T) + b_t v_t k_t^T,
    o_t = S_t q_t, from S_0 = 0, with unit keys k1 = (0.6, 0.8).

    One token: S_1 = b1 v1 k1^T whatever a1 is, so o_1 = b1 (k1.q1) v1
      = 0.5 * 2.2 * (2, -1) = (2.2, -1.1) for q1 = (1, 2).
    Second key orthogonal, k2 = (-0.8, 0.6): S_1 k2 = 0, so
      o_2 = a2 b1 (k1.q2) v1 + b2 (k2.q2) v2 = 0.5*0.5*1.4*(2, -1) + 0.25*(-0.2)*(1, 3)
          = (0.65, -0.5) for q2 = (1, 1).
      (The gate on the write term instead would give (1.375, -0.775).)
    Same key twice, k2 = k1: S_1 k1 = b1 v1, so S_2 = (a2 b1 (1 - b2) v1 + b2 v2) k1^T and
      o_2 = 1.4 * (0.1875*(2, -1) + 0.25*(1, 3)) = (0.875, 0.7875).
      (The erase term outside the gate, a2 S_1 - b2 (S_1 k2) k2^T + ..., would give
      (0.7, 0.875).)"""
    k1, k2o = (0.6, 0.8), (-0.8, 0.6)
    v1, v2 = (2.0, -1.0), (1.0, 3.0)
    o = _two_tokens(k1, k2o, v1, v2, (1.0, 2.0), (1.0, 1.0), 0.3, 0.5, 0.5, 0.25)
    np.testing.assert_allclose(o[0], [2.2, -1.1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[1], [0.65, -0.5], rtol=0, atol=1e-14)
    o = _two_tokens(k1, k1, v1, v2, (1.0, 2.0), (1.0, 1.0), 0.9, 0.5, 0.5, 0.25)
    np.testing.assert_allclose(o[0], [2.2, -1.1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[1], [0.875, 0.7875], rtol=0, atol=1e-14)


def test_branches_equal_flattened_paths():
    for seed in range(4):
        rng = np.random.default_rng(seed)
        dag = synth.fuzz_dag(rng, max_len=12, max_branches=6, max_mounts=3)
        q, k, v, a, b = _inputs(rng, dag.T, 2, 6, 5)
        o, final = RC.scan(q, k, v, a, b, dag.branches, dag.mounts)
        for br in range(dag.nb):
            idx = RC.path_tokens(dag.branches, br)
            ref = _plain(q[idx], k[idx], v[idx], a[idx], b[idx])
            start, L = int(dag.branches[br, 2]), int(dag.branches[br, 3])
            np.testing.assert_allclose(o[start:start + L], ref[len(idx) - L:], atol=1e-12)


def test_mounts_change_nothing():
    rng = np.random.default_rng(9)
    dag = synth.fuzz_dag(rng, max_len=15, max_branches=5, max_mounts=4)
    q, k, v, a, b = _inputs(rng, dag.T, 1, 4, 4)
    o1, f1 = RC.scan(q, k, v, a, b, dag.branches, dag.mounts)
    o2, f2 = RC.scan(q, k, v, a, b, dag.branches, np.zeros((0, 5), dtype=np.int32))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_delta_rule_stores_and_retrieves():
    """alpha = beta = 1 and orthonormal keys: after writing v_j under key e_j, querying
    e_j returns v_j exactly, and rewriting a key replaces its value."""
    Dk = Dv = 4
    keys = np.eye(Dk)
    vals = np.arange(Dk * Dv, dtype=np.float64).reshape(Dk, Dv)
    T = Dk + 1
    q = np.zeros((T, 1, Dk)); k = np.zeros((T, 1, Dk)); v = np.zeros((T, 1, Dv))
    for t in range(Dk):
        k[t, 0], v[t, 0] = keys[t], vals[t]
    k[Dk, 0], v[Dk, 0] = keys[1], -vals[1]     # rewrite key 1
    ones = np.ones((T, 1))
    branches = np.array([[-1, 0, 0, T]])
    _, final = RC.scan(q, k, v, ones, ones, branches)
    S = final[0, 0]
    for j in range(Dk):
        want = -vals[1] if j == 1 else vals[j]
        np.testing.assert_allclose(S @ keys[j], want, atol=1e-12)


def test_beta_zero_keeps_state_and_alpha_gates():
    rng = np.random.default_rng(4)
    branches = np.array([[-1, 0, 0, 5], [0, 5, 5, 3]])
    q, k, v, a, b = _inputs(rng, 8, 1, 3, 3)
    b[5:] = 0.0
    a[5:] = 0.5
    o, final = RC.scan(q, k, v, a, b, branches)
    np.testing.assert_allclose(final[1], 0.125 * final[0], atol=1e-12)
    np.testing.assert_allclose(o[7, 0], final[1][0] @ q[7, 0], atol=1e-12)


# ---------------------------------------------------------------------------- backward

def test_backward_one_token_hand_derived():
    """From S_0 = 0 one token gives o = b (k.q) v, so with upstream g:
    dq = b (g.v) k, dk = b (g.v) q, dv = b (k.q) g, db = (k.q)(g.v), da = 0."""
    k = np.array([[[0.6, 0.8]]]); q = np.array([[[1.0, 2.0]]]); v = np.array([[[2.0, -1.0]]])
    g = np.array([[[0.5, 3.0]]])
    a = np.array([[0.3]]); b = np.array([[0.5]])
    dq, dk, dv, da, db = RC.scan_bwd(q, k, v, a, b, g, np.array([[-1, 0, 0, 1]]))
    gv, kq = -2.0, 2.2  # g.v = 1 - 3, k.q = 0.6 + 1.6
    np.testing.assert_allclose(dq[0, 0], 0.5 * gv * np.array([0.6, 0.8]), atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], 0.5 * gv * np.array([1.0, 2.0]), atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], 0.5 * kq * np.array([0.5, 3.0]), atol=1e-14)
    np.testing.assert_allclose(db[0, 0], kq * gv, atol=1e-14)
    np.testing.assert_allclose(da[0, 0], 0.0, atol=1e-14)


def _loss(q, k, v, a, b, do, branches):
    o, _ = RC.scan(q, k, v, a, b, branches)
    return float(np.sum(o * do))


def test_backward_finite_differences():
    """Central differences of L = sum <dO, o> through forks (children forked at 0, inside
    and at the end of their parents) for every input."""
    for seed in range(3):
        rng = np.random.default_rng(40 + seed)
        dag = synth.fuzz_dag(rng, max_len=7, max_branches=5, max_mounts=2)
        q, k, v, a, b = _inputs(rng, dag.T, 2, 3, 4)
        do = rng.standard_normal(v.shape)
        grads = RC.scan_bwd(q, k, v, a, b, do, dag.branches, segment=3)
        eps = 1e-6
        for which, arr in enumerate((q, k, v, a, b)):
            for _ in range(4):
                idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
                xs = [x.copy() for x in (q, k, v, a, b)]
                xs[which][idx] += eps
                lp = _loss(*xs, do, dag.branches)
                xs[which][idx] -= 2 * eps
                lm = _loss(*xs, do, dag.branches)
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grads[which][idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx)


def test_backward_equals_autograd_over_flattened_paths():
    """An independent formulation: every branch runs the plain recurrence over its whole
    flattened root-to-branch path in torch (float64, CPU) and contributes the outputs of its
    own tokens; torch.autograd of the summed loss must equal the packed backward (shared
    prefix tokens collect the gradients of every branch that passes through them)."""
    import torch
    for seed in range(3):
        rng = np.random.default_rng(60 + seed)
        dag = synth.fuzz_dag(rng, max_len=10, max_branches=6, max_mounts=2)
        q, k, v, a, b = _inputs(rng, dag.T, 2, 4, 3)
        do = rng.standard_normal(v.shape)
        tq, tk, tv, ta, tb = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                              for x in (q, k, v, a, b))
        tdo = torch.tensor(do, dtype=torch.float64)
        loss = torch.zeros((), dtype=torch.float64)
        for br in range(dag.nb):
            idx = RC.path_tokens(dag.branches, br)
            L = int(dag.branches[br, 3])
            S = torch.zeros((2, 3, 4), dtype=torch.float64)
            for j, t in enumerate(idx):
                Sk = torch.einsum("hij,hj->hi", S, tk[t])
                S = ta[t][:, None, None] * (S - tb[t][:, None, None] * Sk[:, :, None]
                                            * tk[t][:, None, :]) \
                    + tb[t][:, None, None] * tv[t][:, :, None] * tk[t][:, None, :]
                if j >= len(idx) - L:
                    loss = loss + torch.sum(torch.einsum("hij,hj->hi", S, tq[t]) * tdo[t])
        loss.backward()
        ours = RC.scan_bwd(q, k, v, a, b, do, dag.branches, segment=4)
        for got, ref in zip(ours, (tq.grad, tk.grad, tv.grad, ta.grad, tb.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-11)


def test_backward_segment_size_does_not_matter():
    rng = np.random.default_rng(80)
    dag = synth.fuzz_dag(rng, max_len=40, max_branches=6, max_mounts=2)
    q, k, v, a, b = _inputs(rng, dag.T, 1, 4, 4)
    do = rng.standard_normal(v.shape)
    g1 = RC.scan_bwd(q, k, v, a, b, do, dag.branches, segment=1)
    g2 = RC.scan_bwd(q, k, v, a, b, do, dag.branches, segment=7)
    g3 = RC.scan_bwd(q, k, v, a, b, do, dag.branches)
    for x, y, z in zip(g1, g2, g3):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(x, z)
