"""CPU tests of the C-ABI library's host side: it loads and exports every declared
symbol; the planner rejects malformed tables like the oracle does; positions, the
dense mask expanded from the tile lists, nnz and the FULL/PARTIAL classification
match the oracle bit for bit; the decode segment builder covers exactly the oracle's
cursor context with the producers' own pages."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
import tree_packed_block_amd as tpb
from oracle import dag as D
from oracle import decode as DEC
from oracle.attention import useful_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "octopus_dag.h")).read()
    declared = set(re.findall(r"\b(octopus_[a-z_]+)\s*\(", header))
    assert declared == set(tpb.EXPORTS)
    L = tpb.lib()
    for name in declared:
        assert isinstance(getattr(L, name), ctypes._CFuncPtr), name
    assert b"gfx950" in L.octopus_version()


def _plan_code(br, mt, T, kv_tile=64):
    try:
        tpb.Plan(br, mt, T, kv_tile)
        return "OK"
    except tpb.OctopusError as e:
        return e.name


def test_planner_rejects_what_the_oracle_rejects():
    ok_b = np.array([[-1, 0, 0, 4], [0, 2, 4, 3]])
    ok_m = np.array([[1, 1, 0, 0, 2]])
    assert _plan_code(ok_b, ok_m, 7) == "OK"
    bad = [
        (np.array([[0, 0, 0, 4], [0, 2, 4, 3]]), ok_m, 7),
        (np.array([[-1, 0, 0, 4], [1, 2, 4, 3]]), ok_m, 7),
        (np.array([[-1, 0, 0, 4], [0, 5, 4, 3]]), ok_m, 7),
        (np.array([[-1, 0, 0, 4], [0, 2, 4, 0]]), ok_m, 4),
        (np.array([[-1, 0, 0, 4], [0, 2, 5, 3]]), ok_m, 8),
        (np.array([[-1, 0, 0, 4], [0, 2, 3, 3]]), ok_m, 6),
        (ok_b, np.array([[1, 1, 1, 0, 2]]), 7),
        (ok_b, np.array([[1, 4, 0, 0, 2]]), 7),
        (ok_b, np.array([[1, 1, 0, 2, 2]]), 7),
        (ok_b, np.array([[1, 1, 0, 0, 5]]), 7),
        (ok_b, np.array([[1, 1, 2, 0, 1]]), 7),
        (ok_b, ok_m, 0),
        (np.array([[-1, 0, 0, 4], [-1, 2, 4, 3]]), ok_m, 7),
        (np.array([[-1, 0, 0, 4], [-1, 0, 4, 3]]), ok_m, 7),
    ]
    for b, m, T in bad:
        with pytest.raises(D.DagError):
            D.validate(b, m, T)
        assert _plan_code(b, m, T) == "EINVAL", (b, m, T)
    br = np.array([[-1, 0, 0, 4], [0, 4, 4, 6], [0, 4, 10, 6]])
    assert _plan_code(br, np.array([[1, 0, 2, 0, 5], [2, 0, 1, 0, 5]]), 16) == "ECYCLE"
    assert _plan_code(ok_b, ok_m, 7, kv_tile=128) == "EUNSUPPORTED"


def _check_plan(dag, rows=None):
    p = tpb.Plan(dag.branches, dag.mounts, dag.T)
    assert np.array_equal(p.positions(), D.positions(dag.branches, dag.mounts))
    T = dag.T
    blocks = rows if rows is not None else [(lo, min(T, lo + 2048)) for lo in range(0, T, 2048)]
    nnz = 0
    for lo, hi in blocks:
        ref = D.mask_rows(dag.branches, dag.mounts, T, lo, hi)
        got = np.unpackbits(p.export_mask(lo, hi), axis=1, bitorder="little")[:, :T]
        assert np.array_equal(got.astype(bool), ref), (lo, hi)
        nnz += int(ref.sum())
    if rows is None:
        assert p.stats()["nnz"] == nnz
    _check_classification(p, dag, blocks)
    return p


def _check_classification(p, dag, blocks):
    """FULL means every valid row of the query tile sees every key of the KV tile;
    PARTIAL tiles are neither empty nor full (a ragged last KV tile is always
    PARTIAL); the lists are strictly increasing."""
    T = dag.T
    qt_ptr, kv, mk, rows = p.tiles()
    qts = sorted({lo // 128 for lo, hi in blocks} | {(hi - 1) // 128 for lo, hi in blocks})
    for qt in qts:
        r0, r1 = qt * 128, min(T, qt * 128 + 128)
        M = D.mask_rows(dag.branches, dag.mounts, T, r0, r1)
        lst = kv[qt_ptr[qt]:qt_ptr[qt + 1]]
        assert np.all(np.diff(lst) > 0)
        seen = set()
        for t, m in zip(lst, mk[qt_ptr[qt]:qt_ptr[qt + 1]]):
            k0, k1 = t * 64, min(T, t * 64 + 64)
            sub = M[:, k0:k1]
            assert sub.any()
            if m < 0:
                assert sub.all() and k1 - k0 == 64
            else:
                assert not (sub.all() and k1 - k0 == 64)
                bits = np.array([[(int(rows[m, r]) >> x) & 1 for x in range(64)]
                                 for r in range(128)], dtype=bool)
                assert np.array_equal(bits[: r1 - r0, : k1 - k0], sub)
                assert not bits[r1 - r0:].any() and not bits[:, k1 - k0:].any()
            seen.add(int(t))
        touched = {j // 64 for j in np.flatnonzero(M.any(axis=0))}
        assert touched == seen


@pytest.mark.parametrize("name", ["tiny", "episode_small", "episode_mid", "forked"])
def test_plan_bit_exact_with_oracle(name):
    dag, _ = synth.build(name)
    p = _check_plan(dag)
    if name == "forked":
        assert p.stats()["nnz"] == useful_pairs(dag.branches, dag.mounts, dag.T)


@pytest.mark.parametrize("name", ["episode131k", "episode262k"])
def test_plan_bit_exact_with_oracle_sampled_rows(name):
    """Full-size trees: positions everywhere, the mask on row blocks covering the
    start, every branch boundary, every mount's reader offset and the end."""
    dag, _ = synth.build(name)
    T = dag.T
    marks = {0, T - 130}
    for (parent, fork, start, L) in dag.branches:
        marks |= {max(0, start - 70), start + L // 2}
    for (reader, rpos, producer, s, e) in dag.mounts:
        marks.add(max(0, int(dag.branches[reader, 2]) + int(rpos) - 64))
    rows = sorted((m, min(T, m + 130)) for m in marks)
    _check_plan(dag, rows=rows)


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 10**9), st.booleans())
def test_plan_fuzz(seed, acyclic):
    dag = synth.fuzz_dag(np.random.default_rng(seed), max_len=90, max_branches=7,
                         max_mounts=5, acyclic=acyclic)
    try:
        D.positions(dag.branches, dag.mounts)
    except D.DagError as e:
        assert _plan_code(dag.branches, dag.mounts, dag.T) == e.code
        return
    _check_plan(dag)


# ----------------------------------------------------------------------------- decode

def _check_segments(wl):
    sp, pg, lo, hi = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr,
                                         wl.pages, wl.page_size, wl.n_pages, wl.cursors)
    owned = set(wl.pages.tolist())
    for c, b in enumerate(wl.cursors):
        idx = DEC.cursor_tokens(wl.dag.branches, wl.dag.mounts, int(b))
        page, slot = DEC.physical_slots(wl.dag.branches, wl.page_ptr, wl.pages,
                                        wl.page_size, idx)
        want = list(zip(page.tolist(), slot.tolist()))
        got = []
        for s in range(sp[c], sp[c + 1]):
            assert 0 <= lo[s] < hi[s] <= wl.page_size
            assert pg[s] in owned
            got.extend((int(pg[s]), x) for x in range(lo[s], hi[s]))
        assert got == want  # same keys, each once, in packed-key order
    return sp, pg, lo, hi


def test_decode_segments_match_oracle_small():
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=16)
    _check_segments(wl)


def test_decode_segments_match_oracle_full_size():
    wl = synth.decode_workload()
    sp, pg, lo, hi = _check_segments(wl)
    # mounts read the producers' pages in place: the pool holds exactly the pages
    # the branches own, and no segment names any other page
    assert wl.n_pages == int(wl.page_ptr[-1])
    assert set(pg.tolist()) <= set(wl.pages.tolist())


def _check_shared_segments(wl):
    """With sharing: groups partition the cursors, every group's cursors fork from one
    (parent, fork), and a cursor's own list plus its group's list hold exactly its
    context, each key once."""
    B = len(wl.cursors)
    sp, pg, lo, hi, gp, gc = tpb.decode_segments(wl.dag.branches, wl.dag.mounts,
                                                 wl.page_ptr, wl.pages, wl.page_size,
                                                 wl.n_pages, wl.cursors, share=True)
    n_groups = len(gp) - 1
    assert len(sp) == B + n_groups + 1 and gp[0] == 0 and gp[-1] == B
    assert sorted(gc.tolist()) == list(range(B))
    br = wl.dag.branches
    shared = 0
    for g in range(n_groups):
        members = gc[gp[g]:gp[g + 1]]
        assert len(members) >= 1
        keys = {(int(br[wl.cursors[c], 0]), int(br[wl.cursors[c], 1]) if br[wl.cursors[c], 0] >= 0 else 0)
                for c in members}
        assert len(keys) == 1
        gl = B + g
        group_keys = [(int(pg[s]), x) for s in range(sp[gl], sp[gl + 1])
                      for x in range(lo[s], hi[s])]
        shared += len(group_keys)
        for c in members:
            b = int(wl.cursors[c])
            idx = DEC.cursor_tokens(br, wl.dag.mounts, b)
            page, slot = DEC.physical_slots(br, wl.page_ptr, wl.pages, wl.page_size, idx)
            want = sorted(zip(page.tolist(), slot.tolist()))
            own = [(int(pg[s]), x) for s in range(sp[c], sp[c + 1]) for x in range(lo[s], hi[s])]
            assert sorted(own + group_keys) == want
    return n_groups, shared


def test_decode_shared_segments_full_size():
    """64 cursors forked at the end of one 16,384-token prefix: one group whose list is
    the prefix (256 pages of 64 slots), read once instead of 64 times."""
    wl = synth.decode_workload()
    n_groups, shared = _check_shared_segments(wl)
    assert n_groups == 1 and shared == 16384


@pytest.mark.parametrize("seed", range(6))
def test_decode_shared_segments_fuzz(seed):
    """Random forks (several groups, nested ones) and mounts that overlap what the
    reader inherits; every branch is a cursor."""
    rng = np.random.default_rng(seed)
    dag = synth.fuzz_dag(rng, max_len=70, max_branches=7, max_mounts=5)
    n_pages, ptr, pages = synth.dags.assign_pages(dag, 16, rng)
    wl = synth.DecodeWorkload(dag, 16, n_pages, ptr, pages,
                              np.arange(dag.nb, dtype=np.int32))
    _check_shared_segments(wl)


def _check_extend_segments(wl, n_new):
    """For every new token (own offset r) of every cursor, the slots the thresholds
    admit are exactly the oracle's context of that token, each key once; thresholds are
    sorted within a cursor; first_off is the first new token's offset."""
    sp, pg, lo, hi, thr, causal, first = tpb.extend_segments(
        wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages, wl.page_size, wl.n_pages,
        wl.cursors, n_new)
    br = wl.dag.branches
    T = int(br[:, 3].sum())
    for c, b in enumerate(wl.cursors):
        start, L = int(br[b, 2]), int(br[b, 3])
        m = int(n_new[c])
        assert first[c] == L - m
        seg = range(sp[c], sp[c + 1])
        assert all(thr[s] <= thr[s + 1] for s in list(seg)[:-1])
        keys = [(int(pg[s]), x) for s in seg for x in range(lo[s], hi[s])]
        assert len(keys) == len(set(keys))
        rows = D.mask_rows(br, wl.dag.mounts, T, start + L - m, start + L)
        for j in range(m):
            r = L - m + j
            got = sorted((int(pg[s]), x) for s in seg for x in range(lo[s], hi[s])
                         if r >= thr[s] + (x - lo[s] if causal[s] else 0))
            page, slot = DEC.physical_slots(br, wl.page_ptr, wl.pages, wl.page_size,
                                            np.flatnonzero(rows[j]))
            assert got == sorted(zip(page.tolist(), slot.tolist())), (c, j)


def test_extend_segments_match_oracle_small():
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=16)
    rng = np.random.default_rng(3)
    L = wl.dag.branches[wl.cursors, 3]
    _check_extend_segments(wl, np.minimum(L, rng.integers(1, 90, size=len(L))))


@pytest.mark.parametrize("seed", range(6))
def test_extend_segments_fuzz(seed):
    """Every branch a cursor, mounts issued inside the new tokens, spans that overlap
    what the reader inherits."""
    rng = np.random.default_rng(40 + seed)
    dag = synth.fuzz_dag(rng, max_len=70, max_branches=7, max_mounts=6)
    n_pages, ptr, pages = synth.dags.assign_pages(dag, 16, rng)
    wl = synth.DecodeWorkload(dag, 16, n_pages, ptr, pages, np.arange(dag.nb, dtype=np.int32))
    n_new = np.array([int(rng.integers(1, L + 1)) for L in dag.branches[:, 3]])
    _check_extend_segments(wl, n_new)


def test_extend_segments_errors():
    wl = synth.decode_workload(seed=5, n_cursors=4, prefix=64, own_max=100, page_size=16)
    L = wl.dag.branches[wl.cursors, 3]
    for bad in (np.zeros_like(L), L + 1):
        with pytest.raises(tpb.OctopusError) as ei:
            tpb.extend_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages, 16,
                                wl.n_pages, wl.cursors, bad)
        assert ei.value.name == "EINVAL"


def test_decode_segments_errors():
    wl = synth.decode_workload(seed=5, n_cursors=4, prefix=64, own_max=100, page_size=16)
    bad_pages = wl.pages.copy()
    bad_pages[0] = wl.n_pages
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, bad_pages, 16,
                            wl.n_pages, wl.cursors)
    assert ei.value.name == "EINVAL"
    short = wl.page_ptr.copy()
    short[1:] -= 1
    with pytest.raises(tpb.OctopusError):
        tpb.decode_segments(wl.dag.branches, wl.dag.mounts, short, wl.pages, 16, wl.n_pages,
                            wl.cursors)


def test_workspace_sizes():
    """Forward: bf16 V re-laid per 64-key tile; backward: LSE2/Delta float32 rows padded
    to 128."""
    import tree_packed_block_amd as tpb
    dag = synth.build("forked")[0]
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T)
    n_kt = -(-dag.T // 64)
    tp = -(-dag.T // 128) * 128
    for hq, hkv, d in ((4, 2, 64), (16, 4, 128)):
        tiles = hkv * n_kt * 64 * d * 2
        assert tpb.fwd_workspace_bytes(plan, tpb.BF16, hq, hkv, d) == tiles
        assert tpb.fwd_workspace_bytes(plan, tpb.FP32, hq, hkv, d) == 0
        floats = 2 * hq * tp * 4
        assert tpb.bwd_workspace_bytes(plan, tpb.FP32, hq, hkv, d) == floats
        assert tpb.bwd_workspace_bytes(plan, tpb.BF16, hq, hkv, d) == floats



def test_extend_pair_count_matches_oracle():
    """The benchmark's count of visible (new token, key) pairs equals the oracle's mask
    row sums."""
    import bench
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=16)
    L = wl.dag.branches[wl.cursors, 3]
    n_new = np.minimum(L, np.random.default_rng(4).integers(1, 200, size=len(L)))
    segs = tpb.extend_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages, 16,
                               wl.n_pages, wl.cursors, n_new)
    br = wl.dag.branches
    T = int(br[:, 3].sum())
    want = 0
    for c, b in enumerate(wl.cursors):
        end = int(br[b, 2] + br[b, 3])
        want += int(D.mask_rows(br, wl.dag.mounts, T, end - int(n_new[c]), end).sum())
    assert bench.extend_pairs(segs, n_new, br, wl.cursors) == want


def _code(rc):
    names = {0: "OK", -1: "EINVAL", -2: "ECYCLE", -3: "EUNSUPPORTED", -4: "ENOMEM",
             -5: "EWORKSPACE", -6: "EHIP", -7: "ESTATE"}
    return names[rc]


def test_new_entry_points_reject_bad_arguments_before_any_launch():
    """Errors the RoPE, extend and scan entry points detect on the host (no device
    memory is touched): unsupported head sizes and dtypes, bad counts, NULL pointers, a
    plan that was never uploaded."""
    L = tpb.lib()
    dag, _ = synth.build("tiny")
    p = tpb.Plan(dag.branches, dag.mounts, dag.T)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call fails first
    # RoPE pass
    assert _code(L.octopus_rope(tpb.BF16, 4, 2, 96, 10000.0, 0, fake, fake, fake, None)) == "EUNSUPPORTED"
    assert _code(L.octopus_rope(tpb.BF16, 4, 2, 128, 1.0, 0, fake, fake, fake, None)) == "EINVAL"
    assert _code(L.octopus_rope(tpb.BF16, 4, 2, 128, 10000.0, 0, None, fake, fake, None)) == "EINVAL"
    assert _code(L.octopus_rope(7, 4, 2, 128, 10000.0, 0, fake, fake, fake, None)) == "EUNSUPPORTED"
    # RoPE attention entry points on a plan that was never uploaded
    assert _code(L.octopus_dag_attn_fwd_rope(p.handle, tpb.BF16, 4, 2, 128, 0.0, 10000.0, fake,
                                             fake, fake, fake, fake, fake, 1 << 30, None)) == "ESTATE"
    assert _code(L.octopus_dag_attn_bwd_rope(p.handle, tpb.BF16, 4, 2, 128, 0.0, 10000.0, fake,
                                             fake, fake, fake, fake, fake, fake, fake, fake,
                                             fake, 1 << 30, None)) == "ESTATE"
    # recurrent scan
    assert _code(L.octopus_gated_delta_scan(p.handle, tpb.BF16, 2, 128, 128, fake, fake, fake,
                                            fake, fake, fake, fake, 1 << 30, None)) == "ESTATE"
    assert _code(L.octopus_gated_delta_scan_save(p.handle, tpb.BF16, 2, 128, 128, fake, fake,
                                                 fake, fake, fake, fake, fake, 1 << 30,
                                                 None)) == "ESTATE"
    assert _code(L.octopus_gated_delta_scan_bwd(p.handle, tpb.BF16, 2, 128, 128, *[fake] * 11,
                                                fake, 1 << 30, None)) == "ESTATE"
    assert _code(L.octopus_gated_delta_scan_bwd_saved(p.handle, tpb.BF16, 2, 128, 128,
                                                      *[fake] * 11, fake, 1 << 30,
                                                      None)) == "ESTATE"
    assert tpb.lib().octopus_gdn_workspace_bytes(p.handle, 2, 64, 128) == 0
    assert tpb.lib().octopus_gdn_bwd_workspace_bytes(p.handle, 0, 128, 128) == 0
    # both children fork from the root at offset 256: one checkpoint slot; chunks end every
    # 32 own tokens and at every fork offset; one 5,376-float record per (chunk, head)
    br = np.asarray(dag.branches).reshape(-1, 4)
    n_chunks = 0
    for b, (_, _, _, ln) in enumerate(br):
        cuts = set(range(32, int(ln), 32)) | {int(f) for par, f, _, _ in br
                                              if par == b and 0 < f < ln}
        n_chunks += len(cuts) + 1 if ln > 0 else 0
    state = 2 * 128 * 128 * 4
    assert tpb.gdn_workspace_bytes(p, 2) == 1 * state + n_chunks * 2 * 5376 * 4
    # backward: checkpoint slots, one initial-state gradient per branch, two state sets
    # per chunk, the records
    assert tpb.gdn_bwd_workspace_bytes(p, 2) == (1 + len(br) + 2 * n_chunks) * state + \
        n_chunks * 2 * 5376 * 4
    # extend
    assert _code(L.octopus_paged_mount_extend(tpb.BF16, 1, 16, 4, 96, 64, 0.0, fake, fake, fake,
                                              4, fake, 1, fake, fake, fake, fake, fake, fake,
                                              fake, fake, fake, None)) == "EUNSUPPORTED"
    assert _code(L.octopus_paged_mount_extend(5, 1, 16, 4, 64, 64, 0.0, fake, fake, fake,
                                              4, fake, 1, fake, fake, fake, fake, fake, fake,
                                              fake, fake, fake, None)) == "EUNSUPPORTED"
    assert _code(L.octopus_paged_mount_extend(tpb.BF16, 1, 16, 4, 128, 64, 0.0, fake, fake, fake,
                                              4, fake, 0, fake, fake, fake, fake, fake, fake,
                                              fake, fake, fake, None)) == "EINVAL"
    assert _code(L.octopus_paged_mount_extend(tpb.BF16, 1, 16, 4, 128, 32, 0.0, fake, fake, fake,
                                              4, fake, 1, fake, fake, fake, fake, fake, fake,
                                              fake, fake, fake, None)) == "EUNSUPPORTED"


def test_positions_without_a_plan_match_the_oracle():
    for name in ("tiny", "episode_mid", "forest_small"):
        dag, _ = synth.build(name)
        assert np.array_equal(tpb.dag_positions(dag.branches, dag.mounts, dag.T),
                              D.positions(dag.branches, dag.mounts))
    br = np.array([[-1, 0, 0, 4], [0, 4, 4, 6], [0, 4, 10, 6]])
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.dag_positions(br, np.array([[1, 0, 2, 0, 5], [2, 0, 1, 0, 5]]), 16)
    assert ei.value.name == "ECYCLE"


def test_plan_upload_rejects_a_host_or_mistyped_buffer():
    """The plan image goes to a caller-owned device buffer; a host tensor or one of
    another element type is refused before any copy is issued."""
    import torch
    dag = synth.build("tiny")[0]
    p = tpb.Plan(dag.branches, dag.mounts, dag.T)
    n = p.device_bytes()
    for buf in (torch.empty(n, dtype=torch.uint8), torch.empty(n, dtype=torch.float32)):
        with pytest.raises(tpb.OctopusError):
            p.upload(buffer=buf)
    assert p.dev is None


def test_plan_at_the_token_limit():
    """2^24 tokens (the planner's limit) as a forest of 4,096 causal trees of 4,096 tokens:
    the plan is built in seconds (its cost follows the listed pairs, not query tiles x KV
    tiles), with the closed-form counts: nnz = n L (L + 1) / 2, 2j + 2 KV tiles for query
    tile j of a tree, two of them PARTIAL (the diagonal); one token more is refused."""
    import time
    n, L = 4096, 4096
    br = np.array([[-1, 0, i * L, L] for i in range(n)], dtype=np.int32)
    t0 = time.time()
    p = tpb.Plan(br, np.zeros((0, 5), np.int32), n * L)
    took = time.time() - t0
    st = p.stats()
    assert st["nnz"] == n * L * (L + 1) // 2
    assert st["n_pairs"] == n * sum(2 * j + 2 for j in range(L // 128))
    assert st["n_partial"] == n * 2 * (L // 128)
    pos = p.positions()
    assert np.array_equal(pos[:L], np.arange(L)) and np.array_equal(pos[-L:], np.arange(L))
    assert took < 120, took
    del p
    with pytest.raises(tpb.OctopusError):
        tpb.Plan(np.array([[-1, 0, 0, n * L + 1]], np.int32), np.zeros((0, 5), np.int32),
                 n * L + 1)


def _nnz_closed_form(br, mt):
    """Visible pairs of an episode-shaped tree (or a forest of them) where no mounted key
    is otherwise visible to its reader: every branch's rows see their inherited context
    (the parent's first `fork` tokens, the parent's own context there, and mounts the
    parent had read by then), their own tokens causally, and every span mounted at or
    before their offset.  Every non-root branch of these trees forks from its tree's root,
    which has no mounts, so the inherited context is `fork` keys."""
    total = 0
    for b, (parent, fork, start, L) in enumerate(br):
        L = int(L)
        inherited = 0 if parent < 0 else int(fork)
        total += L * inherited + L * (L + 1) // 2
        for (reader, rpos, producer, s, e) in mt:
            if int(reader) == b:
                total += (L - int(rpos)) * (int(e) - int(s))
    return total


@pytest.mark.parametrize("name,want", [("episode131k", 1_514_769_199),
                                       ("episode262k", 6_058_939_877),
                                       ("forest1m", 24_310_578_842)])
def test_plan_nnz_full_size_closed_form(name, want):
    """The numerator of the headline FLOP count: the planner's visible-pair count at
    full size equals the closed form over the tables, and the stated figure."""
    dag, _ = synth.build(name)
    br, mt = dag.branches, dag.mounts
    for (parent, fork, start, L) in br:  # the closed form's premise
        assert parent < 0 or br[parent][0] < 0
    for (reader, rpos, producer, s, e) in mt:
        assert br[reader][0] >= 0 and br[producer][0] >= 0 and reader != producer
    assert _nnz_closed_form(br, mt) == want
    p = tpb.Plan(br, mt, dag.T)
    assert p.stats()["nnz"] == want


def test_gpu_fuzz_any_producer_draws_descendants():
    """The any-producer GPU fuzz cases (tests/test_edge_gpu.py) do mount spans of the
    reader's own descendants, so the kernels are known to consume that layout."""
    import test_edge_gpu as E
    n = 0
    for seed in range(8):
        dag, _ = E._any_producer_dag(1000 + seed)
        n += sum(E._descends(dag.branches, int(p), int(r)) for (r, rp, p, s, e) in dag.mounts)
    assert n >= 3
