"""Seeded synthetic inputs (symbols, indexes and CDF tables) shared by the oracle tests,
the GPU parity tests and the benchmark.  No coder arithmetic lives here."""
from .configs import MAKERS, EDGE_RAWS, Workload, load, raw_to_value, y_tables  # noqa: F401
from .tables import (  # noqa: F401
    TOTAL,
    gaussian_table_set,
    logistic_table_set,
    quantise_pmf,
    freqs_to_cdf,
)
