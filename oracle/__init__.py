"""CPU oracle for the LLM.int8() linear layer (test infrastructure only).

Imported by the test-suite, the smoke check and the benchmark's CPU-baseline
leg; never by the product path.
"""
from .llmint8_oracle import *  # noqa: F401,F403
from .llmint8_oracle import __all__  # noqa: F401
