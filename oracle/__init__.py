"""fp64 CPU oracle of the tensor-parallel GPT layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""

from . import tp_layer_oracle  # noqa: F401
