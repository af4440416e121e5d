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
