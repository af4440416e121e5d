"""GPU parity of paged mounted decode against the float64 oracle (and against the
packed forward), through the C-ABI library."""

import numpy as np
import pytest

import synth
from oracle import attention as A
from oracle import dag as D
from oracle import decode as DEC
from parity import TOL, check_close, dev, host, say

pytestmark = pytest.mark.gpu


def _decode_inputs(wl, Hq=16, Hkv=4, Dh=128, seed=55, dtype="bf16"):
    rng = np.random.default_rng(seed)
    return synth.draw_decode_inputs(rng, len(wl.cursors), Hq, Hkv, Dh, wl.n_pages,
                                    wl.page_size, dtype=dtype)


def _gpu_decode(wl, x, n_split, segs=None, share=False, dtype="bf16"):
    """Through the C ABI; with ``share``, the inherited context of every group of cursors
    is a list of its own, read once per block of cursors."""
    import torch
    import tree_packed_block_amd as tpb
    if segs is None:
        segs = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages,
                                   wl.page_size, wl.n_pages, wl.cursors, share=share)
    sd = [torch.from_numpy(np.ascontiguousarray(s, dtype=np.int32)).cuda() for s in segs]
    q, kp, vp = dev(x["q"], dtype), dev(x["k_pool"], dtype), dev(x["v_pool"], dtype)
    o, lse = tpb.paged_mount_decode(q, kp, vp, *sd, n_split=n_split)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _oracle(wl, x):
    return DEC.decode(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                      wl.page_ptr, wl.pages, wl.page_size, wl.cursors)


@pytest.mark.parametrize("share", [False, True])
@pytest.mark.parametrize("n_split", [1, 3, 16])
def test_decode_small(n_split, share):
    say(f"case decode small n_split={n_split} share={share}")
    wl = synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                               page_size=64)
    x = _decode_inputs(wl)
    o, lse = _gpu_decode(wl, x, n_split, share=share)
    ro, rl = _oracle(wl, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


@pytest.mark.parametrize("share", [False, True])
@pytest.mark.parametrize("n_split", [1, 3])
@pytest.mark.parametrize("Dh,dtype", [(64, "bf16"), (64, "fp32"), (128, "fp32")])
def test_decode_small_head_dims_and_fp32(Dh, dtype, n_split, share):
    """head_dim 64 (bf16 MFMA kernel) and float32 pools (exact float32 kernel) with the
    same segment lists, shared or not."""
    say(f"case decode small D={Dh} {dtype} n_split={n_split} share={share}")
    wl = synth.decode_workload(seed=6, n_cursors=7, prefix=200, own_max=260, span_max=90,
                               page_size=64)
    x = _decode_inputs(wl, Hq=8, Hkv=2, Dh=Dh, dtype=dtype)
    o, lse = _gpu_decode(wl, x, n_split, share=share, dtype=dtype)
    ro, rl = _oracle(wl, x)
    check_close(o, ro, TOL[dtype], "O")
    check_close(lse, rl, TOL[dtype], "LSE")


def test_decode_full_batch_head_dim_64():
    """The 64-cursor batch at head_dim 64: every cursor against the oracle."""
    say("case decode 64 cursors D=64")
    wl = synth.decode_workload()
    x = _decode_inputs(wl, Dh=64)
    o, lse = _gpu_decode(wl, x, 32, share=True)
    ro, rl = _oracle(wl, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")


def test_decode_full_batch():
    """64 cursors, 16K shared radix prefix, private branches up to 32K, up to three
    mounted spans of up to 8K: every cursor against the oracle; the result does not
    depend on the split count."""
    say("case decode 64 cursors")
    wl = synth.decode_workload()
    x = _decode_inputs(wl)
    o, lse = _gpu_decode(wl, x, 32)
    ro, rl = _oracle(wl, x)
    check_close(o, ro, TOL["bf16"], "O")
    check_close(lse, rl, TOL["bf16"], "LSE")
    o2, lse2 = _gpu_decode(wl, x, 128)
    check_close(o2, ro, TOL["bf16"], "O (128 splits)")
    check_close(lse2, rl, TOL["bf16"], "LSE (128 splits)")
    o3, lse3 = _gpu_decode(wl, x, 32, share=True)
    check_close(o3, ro, TOL["bf16"], "O (shared prefix list)")
    check_close(lse3, rl, TOL["bf16"], "LSE (shared prefix list)")


def test_decode_matches_packed_forward():
    """K/V of a packed tree written into pool pages: decoding the last token of every
    branch gives the packed forward's row of that token (rollout and packed trainer
    read the same graph)."""
    import torch
    import tree_packed_block_amd as tpb
    say("case decode vs packed forward")
    dag, rng = synth.build("episode_small")
    pos = D.positions(dag.branches, dag.mounts)
    x = synth.draw_attention_inputs(rng, dag.T, 16, 4, 128, pos, dtype="bf16")
    n_pages, ptr, pages = synth.dags.assign_pages(dag, 64, np.random.default_rng(9))
    kp = np.zeros((n_pages, 4, 64, 128), dtype=np.float32)
    vp = np.zeros_like(kp)
    for b, (parent, fork, start, L) in enumerate(dag.branches):
        r = np.arange(L)
        kp[pages[ptr[b] + r // 64], :, r % 64] = x["k"][start + r]
        vp[pages[ptr[b] + r // 64], :, r % 64] = x["v"][start + r]
    last = dag.branches[:, 2] + dag.branches[:, 3] - 1
    wl = synth.DecodeWorkload(dag, 64, n_pages, ptr, pages,
                              np.arange(dag.nb, dtype=np.int32))
    xd = {"q": x["q"][last], "k_pool": kp, "v_pool": vp}
    od, ld = _gpu_decode(wl, xd, 4)
    os_, ls_ = _gpu_decode(wl, xd, 4, share=True)
    check_close(os_, od, TOL["bf16"], "decode O, shared lists vs whole lists")
    check_close(ls_, ld, TOL["bf16"], "decode LSE, shared lists vs whole lists")
    plan = tpb.Plan(dag.branches, dag.mounts, dag.T).upload()
    of, lf = tpb.attn_fwd(plan, dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"))
    torch.cuda.synchronize()
    of, lf = host(of)[last], host(lf)[:, last].T
    ro, rl = A.attn_fwd(x["q"], x["k"], x["v"], dag.branches, dag.mounts)
    check_close(od, ro[last], TOL["bf16"], "decode O vs oracle")
    check_close(od, of, TOL["bf16"], "decode O vs packed forward")
    check_close(ld, lf, TOL["bf16"], "decode LSE vs packed forward")


def test_decode_skips_out_of_range_pages():
    """A segment naming a page outside the pool is skipped (no read).  One split, so the
    extra segment does not move any split boundary and the results must be identical."""
    say("case decode bad page")
    import tree_packed_block_amd as tpb
    wl = synth.decode_workload(seed=5, n_cursors=4, prefix=128, own_max=200, span_max=50,
                               page_size=64)
    x = _decode_inputs(wl)
    sp, pg, lo, hi = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr,
                                         wl.pages, 64, wl.n_pages, wl.cursors)
    # insert a bogus segment at the front of cursor 0
    sp2 = sp.copy()
    sp2[1:] += 1
    pg2 = np.concatenate([[wl.n_pages + 1000], pg]).astype(np.int32)
    lo2 = np.concatenate([[0], lo]).astype(np.int32)
    hi2 = np.concatenate([[64], hi]).astype(np.int32)
    o1, l1 = _gpu_decode(wl, x, 1, (sp, pg, lo, hi))
    o2, l2 = _gpu_decode(wl, x, 1, (sp2, pg2, lo2, hi2))
    check_close(o2, o1, 1e-6, "O with a skipped segment")
    check_close(l2, l1, 1e-6, "LSE with a skipped segment")


def test_decode_argument_errors():
    import torch
    import tree_packed_block_amd as tpb
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((4, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    seg = torch.zeros(3, dtype=torch.int32, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.paged_mount_decode(q, kp, kp, seg, seg, seg, seg, n_split=0)
    assert ei.value.name == "EINVAL"
    q96 = torch.zeros((2, 16, 96), dtype=torch.bfloat16, device="cuda")
    kp96 = torch.zeros((4, 4, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.paged_mount_decode(q96, kp96, kp96, seg, seg, seg, seg, n_split=2)
    assert ei.value.name == "EUNSUPPORTED"
