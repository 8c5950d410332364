"""CPU oracle (test infrastructure only: tests, the smoke check and the benchmark's
CPU-baseline leg use it; the library never does)."""
from .svg_oracle import *  # noqa: F401,F403
from .svg_oracle import SPATIAL, TEMPORAL, DENSE  # noqa: F401
