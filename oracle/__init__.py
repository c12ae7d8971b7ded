"""CPU oracle for the KV-correction path (test infrastructure only).

Imported only by tests/, by the package smoke check and by the benchmark's
CPU-baseline leg; the product path never touches it.
"""
from . import kvref  # noqa: F401
