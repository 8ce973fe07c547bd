"""CPU oracle for the MoBA causal block-sparse attention forward and its gradients.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code, header, table or helper with it.

Everything here is plain NumPy in float64, written from the method as the MoBA
pages describe it; see ``moba_oracle`` for the passage each function follows.
"""

from .moba_oracle import (  # noqa: F401
    block_mean,
    gate_scores,
    select_blocks,
    select_all,
    attend,
    moba_reference,
    full_reference,
    naive_mask_reference,
    brute_force_select,
    routing_table,
    moba_decode_reference,
    attend_lse,
    moba_lse_reference,
    moba_backward_reference,
)
