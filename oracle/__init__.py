"""CPU oracle for the byte-level BPE encode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
shares no code with the GPU library.
"""
from .oracle import Oracle, build, LIB_PATH, utf8_complete_len  # noqa: F401
