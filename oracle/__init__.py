"""CPU oracle of the indexer hot path.  Test infrastructure only: imported by tests/,
the smoke check and the benchmark's CPU-baseline leg, never by the product library."""
from .oracle import *  # noqa: F401,F403
