"""float64 CPU oracle of the trellis-quantized routed MoE layer (test infrastructure).

Only tests/, the smoke check and the benchmark's CPU-baseline leg load this package. The
HIP library never imports, links or calls it, and the two share no code.
"""
from .loader import build, load  # noqa: F401
