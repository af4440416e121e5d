"""CPU oracle for packed-DAG attention and paged mounted decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library under
``tree_packed_block_amd/`` never imports it, and nothing here imports that library:
the two share no code.  The only module both sides use is ``synth`` (seeded input
draws, no method arithmetic).

Everything here is a plain, slow transcription of the definitions on the Octopus
pages, in float64:

* ``dag``       -- table validation, token positions under the rotation-free monotonic
                   jump, the visibility of every packed token (fork shares the parent
                   prefix, read_thread adds a sibling span), and a second, sequential
                   formulation of the same visibility (flattened root-to-branch paths).
* ``attention`` -- dense masked softmax attention forward and backward over the
                   explicit visibility mask, with grouped KV heads.
* ``decode``    -- one-query attention of each decode cursor over the physical
                   (page, slot) pairs its context maps to through the page table.

Every public function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, library reductions, brute force and invariants; the one reading the
pages leave unpinned (the literal ``+1`` gap of the position jump) is named in
``dag.positions``.
"""
