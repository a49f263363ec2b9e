"""fp64 CPU oracle for the tiled online-softmax attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP library or its
Python binding.  It shares no code with the HIP path.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    block_average_attention,
    direct_attention,
    direct_attention_rows,
    last_visible_key,
    max_abs_diff,
    online_tiled_attention,
)
