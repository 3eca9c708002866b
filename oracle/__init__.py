"""CPU oracle for the ChunkAttention decode step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The library under
``decode_attention_prefix_tree_amd/`` never routes through it, and it shares no
code, header, table or helper with that library; both sides only consume the
seeded arrays from ``workloads``.

* ``oracle.attention`` -- fp64 softmax(q K^T / sqrt(d)) V over each sequence's
  fully materialised keys/values, plus the partial-result form (o, m, s) and
  the log-sum-exp merge that the two-phase partition relies on.
* ``oracle.tree_model`` -- a plain-Python prefix tree of fixed-size chunks and
  its DFS-ordered chunk table, written from the prefix-aware KV cache
  description; used to check the library's table bit for bit.
"""
