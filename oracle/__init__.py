"""fp64 CPU oracle (test infrastructure only; see :mod:`oracle.nystrom`)."""
from . import backward, block, nystrom, solvers  # noqa: F401
from .nystrom import (  # noqa: F401
    GAUSSIAN, LAPLACIAN, distance_matrix, forward, forward_workload,
    full_kernel_attention, kernel_map, landmark_matrix, landmarks_avg_pool,
    newton_schulz, ns_alpha, nystrom_head, widen)
