"""CPU oracle for the quantized KV cache (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. It shares no code with the HIP library or its Python binding, and
imports neither of them.
"""
from . import brute, kitty, kivi, skvq  # noqa: F401
