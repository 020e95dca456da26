"""fp64 CPU oracle for weight-absorbed MLA decode and chunked prefill.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .mla_oracle import *  # noqa: F401,F403
from . import mla_oracle  # noqa: F401
