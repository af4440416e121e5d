"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer, and under
ThreadSanitizer (its query tiles are planned on host threads) (CPU).

``tests/sanitize/plan_driver.cpp`` is compiled with g++ together with the planner's
source and the two sanitizers (any memory or undefined-behaviour error aborts it), then
fed valid tables (named DAGs, fuzz DAGs with forks and mounts of every kind, page
tables for the decode and extend segment builders) and invalid ones.  Valid plans must
give the oracle's nnz, both as the planner counts it and as the popcount of the mask
expanded from its tile lists; invalid tables must come back as error codes.
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import synth
from oracle import dag as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_packed_block_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build_driver(sanitize, tag):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not available")
    out = os.path.join(tempfile.mkdtemp(prefix="plan_san_"), "plan_driver_" + tag)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=" + sanitize,
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-I" + os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        if "san" in r.stdout.lower():
            pytest.skip("sanitizer runtime not available: " + r.stdout[-300:])
        raise AssertionError("driver build failed:\n" + r.stdout)
    return out


@pytest.fixture(scope="module")
def driver():
    return _build_driver("address,undefined", "asan")


@pytest.fixture(scope="module")
def tsan_driver():
    return _build_driver("thread", "tsan")


def _case_text(branches, mounts, T, page_size=16, pages=None, n_new=None):
    branches = np.asarray(branches, dtype=np.int64).reshape(-1, 4)
    mounts = np.asarray(mounts, dtype=np.int64).reshape(-1, 5)
    nb = branches.shape[0]
    if pages is None:  # no page table: the builders are not reached for invalid tables
        n_pages, ptr, pg = 0, np.zeros(nb + 1, dtype=np.int64), np.zeros(0, dtype=np.int64)
    else:
        n_pages, ptr, pg = pages
    cursors = np.arange(nb)
    if n_new is None:
        n_new = np.ones(nb, dtype=np.int64)
    lines = [f"{T} {nb} {mounts.shape[0]}"]
    lines += [" ".join(map(str, r)) for r in branches.tolist()]
    lines += [" ".join(map(str, r)) for r in mounts.tolist()]
    lines.append(f"{page_size} {n_pages}")
    lines.append(" ".join(map(str, np.asarray(ptr).tolist())))
    lines.append(" ".join(map(str, np.asarray(pg).tolist())))
    lines.append(str(nb))
    lines.append(" ".join(map(str, cursors.tolist())))
    lines.append(" ".join(map(str, np.asarray(n_new).tolist())))
    return "\n".join(lines) + "\n"


def _run(driver, text):
    r = subprocess.run([driver], input=text, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                       text=True, timeout=600)
    assert r.returncode == 0, "sanitizer report:\n" + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    out = []
    for line in r.stdout.splitlines():
        f = line.split()
        out.append({"rc": int(f[3]), "nnz": int(f[5]), "pop": int(f[7]),
                    "seg": (int(f[9]), int(f[10])), "ext": int(f[12]), "img": int(f[14])})
    return out


def _oracle_nnz(dag):
    T = dag.T
    return sum(int(D.mask_rows(dag.branches, dag.mounts, T, lo, min(T, lo + 1024)).sum())
               for lo in range(0, T, 1024))


def test_sanitized_planner_valid_tables(driver):
    rng = np.random.default_rng(11)
    dags = [synth.build("tiny")[0], synth.build("episode_small")[0]]
    for seed in range(24):
        r = np.random.default_rng(seed)
        dags.append(synth.fuzz_dag(r, max_branches=7, max_len=150, max_mounts=5))
    text = ""
    for dag in dags:
        pages = synth.dags.assign_pages(dag, 16, rng)
        n_new = np.minimum(dag.branches[:, 3], 1 + rng.integers(0, 40, dag.nb))
        text += _case_text(dag.branches, dag.mounts, dag.T, 16, pages, n_new)
    res = _run(driver, text)
    assert len(res) == len(dags)
    for dag, r in zip(dags, res):
        want = _oracle_nnz(dag)
        assert r["rc"] == 0 and r["nnz"] == want and r["pop"] == want, (r, want)
        assert r["seg"] == (0, 0) and r["ext"] == 0
        assert r["img"] == 1, r  # the device image holds the plan's own lists


def test_sanitized_planner_invalid_tables(driver):
    ok_b = [[-1, 0, 0, 4], [0, 2, 4, 3]]
    ok_m = [[1, 1, 0, 0, 2]]
    bad = [
        ([[0, 0, 0, 4], [0, 2, 4, 3]], ok_m, 7),
        ([[-1, 0, 0, 4], [1, 2, 4, 3]], ok_m, 7),
        ([[-1, 0, 0, 4], [0, 5, 4, 3]], ok_m, 7),
        ([[-1, 0, 0, 4], [0, 2, 4, 0]], ok_m, 4),
        ([[-1, 0, 0, 4], [0, 2, 5, 3]], ok_m, 8),
        ([[-1, 0, 0, 4], [0, 2, 3, 3]], ok_m, 6),
        (ok_b, [[1, 1, 1, 0, 2]], 7),
        (ok_b, [[1, 4, 0, 0, 2]], 7),
        (ok_b, [[1, 1, 0, 2, 2]], 7),
        (ok_b, [[1, 1, 0, 0, 5]], 7),
        (ok_b, [[1, 1, 2, 0, 1]], 7),
        (ok_b, [[7, 1, 0, 0, 2]], 7),
        (ok_b, [[1, 1, -3, 0, 2]], 7),
        ([[-1, 0, 0, 4], [-1, 2, 4, 3]], ok_m, 7),
        ([[-1, 0, 0, 4], [5, 0, 4, 3]], ok_m, 7),
        ([[-1, 0, 0, 4], [0, 4, 4, 6], [0, 4, 10, 6]],
         [[1, 0, 2, 0, 5], [2, 0, 1, 0, 5]], 16),  # position cycle
    ]
    # fuzz tables whose mounts may form position cycles, each rejected like the oracle
    codes = {"EINVAL": -1, "ECYCLE": -2}
    want = [-1] * (len(bad) - 1) + [-2]
    for seed in range(40):
        dag = synth.fuzz_dag(np.random.default_rng(1000 + seed), max_branches=7, max_len=60,
                             max_mounts=6, acyclic=False)
        try:
            D.positions(dag.branches, dag.mounts)
        except D.DagError as e:
            bad.append((dag.branches.tolist(), dag.mounts.tolist(), dag.T))
            want.append(codes[e.code])
    assert len(want) > 17  # some cycles among the fuzz tables
    text = "".join(_case_text(b, m, T) for b, m, T in bad)
    res = _run(driver, text)
    assert [r["rc"] for r in res] == want


def test_threaded_planner_under_thread_sanitizer(tsan_driver):
    # Trees of 16K-60K tokens: enough query tiles that the planner splits them over host
    # threads (blocks of consecutive tiles, joined in order) and transposes the masks on
    # them; ThreadSanitizer must report no race and the plans must stay exact.
    rng = np.random.default_rng(5)
    dags = [synth.build("forked")[0]]
    for seed in range(3):
        r = np.random.default_rng(70 + seed)
        dags.append(synth.fuzz_dag(r, max_branches=10, max_len=6000, max_mounts=8))
    text = ""
    for dag in dags:
        pages = synth.dags.assign_pages(dag, 16, rng)
        text += _case_text(dag.branches, dag.mounts, dag.T, 16, pages, None)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([tsan_driver], input=text, stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=900, env=env)
    assert r.returncode == 0, "thread sanitizer report:\n" + r.stderr[-4000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert len(lines) == len(dags)
    for dag, line in zip(dags, lines):
        f = line.split()
        assert int(f[3]) == 0 and int(f[7]) == int(f[5]) == _oracle_nnz(dag), (line, dag.T)
        assert int(f[14]) == 1, line
