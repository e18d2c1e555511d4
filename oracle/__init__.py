"""CPU oracle for the SERQ quantized linear layer -- test infrastructure only.

Imported by tests/, by the smoke check and by the benchmark's CPU-baseline
leg, never by the library. See serq_oracle.py for the sources it follows.
"""
from . import serq_oracle  # noqa: F401
