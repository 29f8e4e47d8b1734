"""fp64 CPU oracles (test infrastructure only): the SageSLA attention forward (sagesla.py) and the W8A8
block-quantized linear layer (w8a8.py); see each module's header."""
from . import sagesla  # noqa: F401
from . import w8a8  # noqa: F401
