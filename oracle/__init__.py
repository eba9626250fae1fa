"""CPU oracle of the HQQ solver (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package. The GPU library never loads it and shares no code with it.

The arithmetic lives in ``hqq_oracle.c`` (plain C, binary32, sequential sums); this module
only builds it with gcc and marshals numpy arrays through ctypes.
"""
from .hqq_oracle import Oracle, build, lib_path  # noqa: F401
