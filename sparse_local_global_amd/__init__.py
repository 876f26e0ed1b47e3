"""PACK3D local-global attention for MI355X (gfx950): HIP kernels behind a C ABI.

The library is ``libpack3d.so`` (built in-tree by ``sparse_local_global_amd.build``);
``sparse_local_global_amd.pack3d`` is its thin Python binding.
"""
from .pack3d import (  # noqa: F401
    Index,
    Pack3DError,
    attention,
    backward,
    build_index,
    forward,
    load_library,
    workspace_bytes,
    workspace_views,
)
