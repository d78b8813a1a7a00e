"""MI355X-native MoE expert-parallel dispatch/combine data path.

The hot path lives in the HIP library ``libmoe_route.so`` (gfx950) behind a
C ABI (``include/moe_route.h``).  ``binding`` marshals torch tensors into that
ABI, ``driver`` sequences the per-chunk calls on HIP streams, ``inputs`` draws
the seeded synthetic workloads.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""

__all__ = ["binding", "driver", "inputs"]
