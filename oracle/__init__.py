"""Float64 CPU oracle for the KDA layer — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never imports, links or calls anything here,
and nothing here imports the library.
"""
from .kda_oracle import *  # noqa: F401,F403
