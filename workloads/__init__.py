"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package only *generates inputs*: sparse surface-voxel token sets (integer
coordinates plus ``cu_seqlens``) and the random per-token tensors (Q, K, V,
gates).  It holds none of the attention method's arithmetic: no block keys, no
sorting, no pooling, no softmax.  Both the CPU oracle and the GPU path read what
it produces; neither imports the other.

The token sets stand in for the latent sparse-voxel tokens of Direct3D-S2
(hyper.ai summary of arXiv 2505.17412, "Method": at 1024^3 the latent holds
more than 100k tokens; "Experiments": 128k tokens for the speed comparison).
"""

from .geometry import (  # noqa: F401
    ellipsoid_band,
    primitive_union_band,
    make_primitives,
)
from .configs import CONFIGS, Workload, make_workload, make_custom  # noqa: F401
from .tensors import bf16_bits_from_f32, bf16_bits_to_f32  # noqa: F401
