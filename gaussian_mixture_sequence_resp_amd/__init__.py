"""Gaussian Mixture Attention (GMA) forward mixer for MI355X (gfx950).

The compute runs in ``libgma.so`` (hand-written HIP kernels behind the C ABI of
``include/gma.h``); this package only binds it (``binding``), builds it
(``build``) and draws seeded synthetic inputs (``inputs``).
"""
from .binding import (  # noqa: F401
    GMAError,
    backward,
    DecodeParams,
    decode_prepare,
    decode_step,
    decode_step_prepared,
    forward,
    forward_cross,
    forward_noalloc,
    load_library,
    make_desc,
    memory,
    resp_stats,
    strerror,
    version,
    workspace_size,
    workspace_size_cross,
)
