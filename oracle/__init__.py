"""Oracle for the MLA library: explicit Multi-head Latent Attention in float64.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP path, and the library never imports it.
"""
from . import mla_oracle  # noqa: F401
