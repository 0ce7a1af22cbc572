"""libhga: the gfx950 (MI355X) hot path of Hierarchical Global Attention.

The C ABI (include/hga.h) lives in ``libhga.so``; ``hga`` is its thin Python
binding and ``inputs`` the seeded synthetic workloads.
"""
from . import inputs  # noqa: F401
