"""CPU float64 oracle for attention forward/backward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    head_backward,
    head_forward,
    head_rows,
    head_tail_keys,
    rowsum_o_do,
    rowsum_p_dp,
    valid_mask,
)
