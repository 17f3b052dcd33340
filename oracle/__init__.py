"""fp64 CPU oracle (test infrastructure only; see ``oracle/attention.py`` for the import rule)."""
from . import attention, brute  # noqa: F401
from .attention import (  # noqa: F401
    allowed,
    backward,
    decode,
    forward,
    head_backward,
    head_forward,
    kv_append,
    prefill,
    rows_forward,
)
