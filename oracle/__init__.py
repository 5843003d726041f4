"""fp64 CPU oracle for the GMA forward mixer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here.
"""
from .oracle import (  # noqa: F401
    build,
    library_path,
    log_joint,
    responsibilities,
    forward,
    forward_cross,
    memory,
    decode_step,
    resp_stats,
    backward,
    num_threads,
)
