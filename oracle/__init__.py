"""Reference oracle for the QSA c4 hot path: test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library.
"""
from . import qsa_oracle  # noqa: F401
