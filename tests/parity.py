"""Helpers for GPU parity tests: seeded inputs (synth), oracle positions, device
copies and the tolerance checks.

Tolerances: elementwise ``|got - ref| <= atol + rtol * |ref|`` with atol = rtol =
2e-2 for bf16 and 1e-5 for fp32 forward outputs; gradients by relative Frobenius
error ``||got - ref||_F / ||ref||_F <= 5e-2`` per tensor.
"""

from __future__ import annotations

import functools
import sys

import numpy as np

import synth
from oracle import dag as D

TOL = {"bf16": 2e-2, "fp32": 1e-5}
GRAD_TOL = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def workload(name, Hq=16, Hkv=4, Dh=128, dtype="bf16", std=0.5, with_dout=False, seed=None):
    """``(dag, inputs)``: the named DAG and Q/K/V (and dO) drawn from the same
    generator, Q and K rotated at the oracle's positions."""
    dag, rng = synth.build(name, seed)
    pos = D.positions(dag.branches, dag.mounts)
    x = synth.draw_attention_inputs(rng, dag.T, Hq, Hkv, Dh, pos, dtype=dtype, std=std,
                                    with_dout=with_dout)
    return dag, x


def fuzz_workload(seed, Hq, Hkv, Dh, dtype="bf16", **kw):
    rng = np.random.default_rng(seed)
    dag = synth.fuzz_dag(rng, **kw)
    pos = D.positions(dag.branches, dag.mounts)
    x = synth.draw_attention_inputs(rng, dag.T, Hq, Hkv, Dh, pos, dtype=dtype, std=0.5,
                                    with_dout=True)
    return dag, x


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.cuda().contiguous()


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_close(got, ref, tol, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    worst = float(np.max(err - bound)) if err.size else 0.0
    mabs = float(err.max()) if err.size else 0.0
    mrel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    say(f"  {name}: max_abs={mabs:.3e} max_rel={mrel:.3e} (tol {tol})")
    assert worst <= 0.0, f"{name}: {int(np.sum(err > bound))} elements outside tolerance"


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def check_grad(got, ref, name, tol=GRAD_TOL):
    """Relative Frobenius error within ``tol``; a gradient that is exactly zero in
    the oracle (a query that sees only itself) must come out within the bf16
    elementwise bound of zero instead."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if not np.any(np.asarray(ref)):
        m = float(np.abs(np.asarray(got, dtype=np.float64)).max()) if np.size(got) else 0.0
        say(f"  {name}: oracle zero, max |got| = {m:.3e}")
        assert m <= TOL["bf16"], f"{name}: {m} away from an exact zero"
        return
    e = rel_fro(got, ref)
    say(f"  {name}: rel_fro={e:.3e} (tol {tol})")
    assert e <= tol, f"{name}: relative Frobenius error {e}"


def sample_rows(dag, width=64):
    """Row ranges covering the first and last rows, both sides of every branch
    boundary, the middle of every branch and every mount's reader offset."""
    T = dag.T
    marks = {0, max(0, T - width)}
    for (parent, fork, start, L) in dag.branches:
        marks |= {max(0, start - width // 2), start + L // 2}
    for (reader, rpos, producer, s, e) in dag.mounts:
        marks.add(max(0, int(dag.branches[reader, 2]) + int(rpos) - width // 2))
    out = []
    for m in sorted(marks):
        lo, hi = m, min(T, m + width)
        if out and lo <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], hi))
        else:
            out.append((lo, hi))
    return out


def table_workload(name, rows_b, rows_m, Hq, Hkv, Dh, dtype="bf16", seed=7):
    """A DAG given by its branch and mount rows, with seeded inputs as above."""
    b = np.asarray(rows_b, dtype=np.int32).reshape(-1, 4)
    m = np.asarray(rows_m, dtype=np.int32).reshape(-1, 5)
    T = int((b[:, 2] + b[:, 3]).max())
    dag = synth.dags.Dag(name, b, m, T)
    rng = np.random.default_rng(seed)
    pos = D.positions(dag.branches, dag.mounts)
    x = synth.draw_attention_inputs(rng, dag.T, Hq, Hkv, Dh, pos, dtype=dtype, std=0.5,
                                    with_dout=True)
    return dag, x
