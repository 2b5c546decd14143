"""CPU oracle for the KDA layer core -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does.
"""
from .kda_oracle import kda_decode_step, kda_recurrent, gate_rmsnorm, kda_chunked  # noqa: F401
