"""fp64 CPU oracle of the SageSLA attention forward (test infrastructure; see sagesla.py's header)."""
from . import sagesla  # noqa: F401
