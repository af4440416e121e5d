"""Pins of the RoPE oracle: hand-derived rotations of a 4-dimensional head at base 10000
(the frequency schedule and the rotate-half pairing, fixed by a golden file), agreement
with the input generator's independent rotation, orthogonality and inversion, the
relative-position property, identity at position 0, and central finite differences of
the loss through the rotation."""

import numpy as np

from conftest import read_golden

import synth
from oracle import attention as A
from oracle import dag as D
from oracle import rope as R


def test_rotate_hand_derived_golden():
    """Unit vectors of a D = 4 head at positions 1, 7 and 100: frequencies 1 and 1/100,
    pairs (x0, x2) and (x1, x3).  A wrong frequency exponent, an interleaved pairing or
    a flipped sine fails here."""
    vals = np.array(read_golden("rope_d4_base10000.txt"), dtype=np.float64).reshape(-1, 9)
    pos = vals[:, 0].astype(np.int64)
    x = vals[:, 1:5].reshape(-1, 1, 4)
    want = vals[:, 5:9].reshape(-1, 1, 4)
    np.testing.assert_allclose(R.rotate(x, pos, base=10000.0), want, rtol=0, atol=1e-15)
    back = R.rotate(want, pos, base=10000.0, inverse=True)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-15)


def test_rotate_matches_generator_rotation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 16))
    pos = rng.integers(0, 300000, size=50)
    np.testing.assert_allclose(R.rotate(x, pos), synth.rope_rotate(x, pos), rtol=0,
                               atol=2e-6)


def test_rotate_orthogonal_and_inverse():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 2, 32))
    pos = rng.integers(0, 1 << 20, size=40)
    y = R.rotate(x, pos)
    np.testing.assert_allclose(R.rotate(y, pos, inverse=True), x, atol=1e-12)
    h = 16
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, atol=1e-11)
    np.testing.assert_allclose(R.rotate(x, np.zeros(40, dtype=np.int64)), x, atol=0)


def test_scores_depend_on_position_differences_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    for p1, p2, d in ((5, 3, 1000), (70000, 12, 31), (0, 0, 262143)):
        a = np.sum(R.rotate(q, [p1]) * R.rotate(k, [p2]))
        b = np.sum(R.rotate(q, [p1 + d]) * R.rotate(k, [p2 + d]))
        assert abs(a - b) < 1e-9


def test_rope_backward_finite_differences():
    dag = synth.fuzz_dag(np.random.default_rng(7), max_len=8, max_branches=4, max_mounts=2)
    rng = np.random.default_rng(8)
    T = dag.T
    q = rng.standard_normal((T, 2, 8))
    k = rng.standard_normal((T, 1, 8))
    v = rng.standard_normal((T, 1, 8))
    do = rng.standard_normal((T, 2, 8))
    base = 100.0

    def loss(qq, kk):
        o, _ = R.attn_fwd(qq, kk, v, dag.branches, dag.mounts, base=base)
        return float(np.sum(o * do))

    dq, dk, dv = R.attn_bwd(q, k, v, do, dag.branches, dag.mounts, base=base)
    eps = 1e-6
    for idx in [(0, 0, 0), (T - 1, 1, 5), (T // 2, 0, 7)]:
        qp, qm = q.copy(), q.copy()
        qp[idx] += eps
        qm[idx] -= eps
        assert abs((loss(qp, k) - loss(qm, k)) / (2 * eps) - dq[idx]) < 1e-6
    for idx in [(0, 0, 3), (T - 1, 0, 0), (T // 2, 0, 6)]:
        kp, km = k.copy(), k.copy()
        kp[idx] += eps
        km[idx] -= eps
        assert abs((loss(q, kp) - loss(q, km)) / (2 * eps) - dk[idx]) < 1e-6
    # V is not rotated: its gradient is the plain one
    pos = D.positions(dag.branches, dag.mounts)
    _, _, dv0 = A.attn_bwd(R.rotate(q, pos, base), R.rotate(k, pos, base), v, do,
                           dag.branches, dag.mounts)
    np.testing.assert_allclose(dv, dv0, atol=0)
