"""CPU oracle for exact attention: TEST INFRASTRUCTURE ONLY.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path. See ``oracle/attention.py`` for the definitions
and the pages they follow.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_forward_blockwise,
    attention_probabilities,
    merge_partials,
)
from .e4m3 import attention_forward_e4m3, e4m3_decode  # noqa: F401
