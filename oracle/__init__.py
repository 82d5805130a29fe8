"""CPU fp64 oracle for the fused exact-attention forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (``exact_attention_18_amd``) and imports nothing from it; the two
meet only at the seeded input tensors.

Every function is pinned by ``tests/test_oracle.py`` (forward) and
``tests/test_oracle_backward.py`` (backward) to facts the pages and the
mathematics fix (worked example, closed forms, invariants, a library routine of
the same definition, brute force).  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_head,
    attention_probs,
    attention_forward,
    attention_forward_varlen,
    attention_rows,
    attention_forward_blocksparse,
    block_mask_to_elements,
    online_softmax_head,
)
from .backward import (  # noqa: F401,E402
    attention_backward,
    attention_backward_head,
    attention_backward_varlen,
    blockwise_backward_head,
    softmax_backward_delta,
)
