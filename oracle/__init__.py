"""fp64 CPU oracle for sink-anchored rolling-cache chunk attention with 3D RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, tables or helpers) and imports nothing from
``streaming_causal_video_amd``.
"""

from .scv_oracle import *  # noqa: F401,F403
from .scv_oracle import __all__  # noqa: F401
