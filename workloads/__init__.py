"""Seeded synthetic workloads (shapes and input generators) for the block-sparse
3D-video attention path.  Holds no arithmetic of the method itself."""
from .configs import CONFIGS, n_tokens, q_grid, q_frame_offset  # noqa: F401
