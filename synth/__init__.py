"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This package only draws structure (branch and mount tables, page tables, cursor
lists) and tensor values from a seeded ``numpy.random.Generator``.  It holds none of
the attention method's arithmetic: it computes no positions, no visibility and no
attention.  Where a draw needs token positions (the RoPE pre-rotation of Q and K),
the caller passes the positions in.

Workload shapes follow the episode statistics of the Octopus project page
("Octopus: One Brain, Many Branches ...", section "Architecture & Co-Design",
primitives table): isolated branches of at most 32K own tokens, up to 262K packed
tokens per tree, a handful of lateral read_thread mounts per episode.
"""

from .dags import Dag, DecodeWorkload, build, fuzz_dag, decode_workload, extend_workload  # noqa: F401
from .tensors import (  # noqa: F401
    round_bf16,
    bf16_bits,
    rope_rotate,
    draw_attention_inputs,
    draw_decode_inputs,
    draw_extend_inputs,
    draw_scan_inputs,
)
