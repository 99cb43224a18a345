"""CPU oracle for fused attention — test infrastructure only.

Imported only by the test suite, the smoke check and the benchmark's
CPU-baseline leg. It shares no code with the HIP library.
"""
from . import oracle, brute  # noqa: F401
