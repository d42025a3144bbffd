"""fp64 CPU oracle for fused attention — test infrastructure, never the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import anything under ``oracle/``.  The HIP library and its Python
binding do not import it, and it does not import them.

``oracle.attention``   the plain definition (S, P materialised), forward + backward
``oracle.online_walk`` the online softmax as a fold of key-block summaries, used to pin the above
                       against the printed worked example
``oracle.brute``       pure-Python loops for tiny shapes (an independent pin)

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, invariants, finite differences and brute force.
"""

from . import attention, brute, online_walk  # noqa: F401
from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_forward_rows,
    kv_head_of,
    softmax_backward_rows,
    softmax_rows,
)
