"""Oracle for the fused attention forward: test infrastructure, not product code.

Plain fp64 CPU NumPy.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
It shares no code with the HIP path and imports nothing from it.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_chain,
    attention_chain_backward,
    attention_chain_head_rows,
    attention_forward,
    attention_head_rows,
    attention_partial,
    merge_partials,
    merge_states,
    online_attention_forward,
    softmax_two_pass,
)
