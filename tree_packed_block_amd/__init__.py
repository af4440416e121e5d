"""Packed-DAG attention for AMD Instinct MI355X (gfx950).

Block-sparse attention over one episode DAG of branches packed into a single
unpadded token stream (forward and backward), and paged decode of cursors over
ancestor, own and mounted pages, as described on the Octopus project page (sections
"Architecture & Co-Design": primitives table, cards "02 · Memory" and
"03 · Training").  The compute lives in ``liboctopus_dag.so`` (C ABI declared in
``include/octopus_dag.h``); this package only binds it.
"""

from ._lib import (  # noqa: F401
    BF16,
    DECODE_SCRATCH_BYTES,
    FP32,
    EXPORTS,
    LIB_PATH,
    OctopusError,
    Plan,
    attn_bwd,
    attn_bwd_phase,
    attn_fwd,
    attn_fwd_rope,
    attn_bwd_rope,
    dag_positions,
    rope,
    rope_workspace_bytes,
    bwd_workspace_bytes,
    decode_segments,
    decode_workspace_bytes,
    extend_segments,
    gated_delta_scan,
    gated_delta_scan_bwd,
    gated_delta_scan_bwd_saved,
    gated_delta_scan_save,
    gdn_bwd_workspace_bytes,
    gdn_workspace_bytes,
    default_scale,
    fwd_workspace_bytes,
    lib,
    paged_mount_decode,
    paged_mount_decode_noalloc,
    paged_mount_extend,
)
