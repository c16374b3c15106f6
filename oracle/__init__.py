"""CPU oracle for the LLM.int8() linear layer and the 4-bit weight path (test
infrastructure only).

Imported by the test-suite, the smoke check and the benchmark's CPU-baseline
leg; never by the product path.
"""
from .llmint8_oracle import *  # noqa: F401,F403
from .llmint8_oracle import __all__ as _int8_all
from .fourbit_oracle import *  # noqa: F401,F403
from .fourbit_oracle import __all__ as _fourbit_all

__all__ = list(_int8_all) + list(_fourbit_all)
