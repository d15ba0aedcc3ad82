"""fp64 CPU oracle for MLA decode.  Test infrastructure only: imported by the
tests, the smoke check and the CPU-baseline leg of the benchmark, never by the
HIP library or its binding."""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import scale_for  # noqa: F401
