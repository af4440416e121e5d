"""GPU test of the decode entry point that allocates nothing: through the C ABI, equal to
the allocating entry point (same kernels, so bit for bit) and within the bf16 tolerance
of the float64 oracle, on two calls in a row, the second with a smaller batch; a batch
whose partial states exceed the scratch array is refused before any launch."""

import numpy as np
import pytest

import synth
from oracle import decode as DEC
from parity import TOL, check_close, dev, host, say

pytestmark = pytest.mark.gpu


def _case(wl, n_split, Hq=16, Hkv=4, Dh=128, seed=55):
    import torch
    import tree_packed_block_amd as tpb
    x = synth.draw_decode_inputs(np.random.default_rng(seed), len(wl.cursors), Hq, Hkv, Dh,
                                 wl.n_pages, wl.page_size)
    segs = tpb.decode_segments(wl.dag.branches, wl.dag.mounts, wl.page_ptr, wl.pages,
                               wl.page_size, wl.n_pages, wl.cursors, share=True)
    sd = [torch.from_numpy(np.ascontiguousarray(s, dtype=np.int32)).cuda() for s in segs]
    q, kp, vp = dev(x["q"], "bf16"), dev(x["k_pool"], "bf16"), dev(x["v_pool"], "bf16")
    need = tpb.decode_workspace_bytes(len(wl.cursors), Hq, Dh, n_split)
    assert need <= tpb.DECODE_SCRATCH_BYTES
    o1, l1 = tpb.paged_mount_decode(q, kp, vp, *sd, n_split=n_split)
    o2, l2 = tpb.paged_mount_decode_noalloc(q, kp, vp, *sd, n_split=n_split)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(l2, l1)
    ro, rl = DEC.decode(x["q"], x["k_pool"], x["v_pool"], wl.dag.branches, wl.dag.mounts,
                        wl.page_ptr, wl.pages, wl.page_size, wl.cursors)
    check_close(host(o2), ro, TOL["bf16"], "O (no allocation)")
    check_close(host(l2), rl, TOL["bf16"], "LSE (no allocation)")
    return sd, q, kp, vp


def test_decode_noalloc_two_calls_then_smaller():
    import torch
    import tree_packed_block_amd as tpb
    say("case decode without allocation: 64 cursors, then 6")
    sd, q, kp, vp = _case(synth.decode_workload(), 32)
    _case(synth.decode_workload(seed=5, n_cursors=6, prefix=256, own_max=300, span_max=100,
                                page_size=64), 3)
    # 64 cursors in 256 splits need more partial states than the scratch array holds: the
    # call is refused before any launch and the outputs stay as they were
    B, Hq, Dh = q.shape
    assert tpb.decode_workspace_bytes(B, Hq, Dh, 256) > tpb.DECODE_SCRATCH_BYTES
    o = torch.full_like(q, 3.0)
    lse = torch.full((B, Hq), 3.0, dtype=torch.float32, device=q.device)
    with pytest.raises(tpb.OctopusError) as ei:
        tpb.paged_mount_decode_noalloc(q, kp, vp, *sd, n_split=256, o=o, lse=lse)
    assert ei.value.name == "EWORKSPACE"
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 3.0).all())
