"""fp64 CPU oracle of the PACK3D local-global attention operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package.
The HIP library never calls it, and it shares no code, table or constant with
the HIP path.

Source: "Geometry Matters in Packed 3D Attention" (arXiv:2610.38694), abstract:
exact local neighbourhood attention, distant context compressed into
contiguous 3D block summaries, axial RoPE on true token-grid coordinates for
every query-key and query-summary logit, rotation applied before a block is
summarized, one softmax over local keys and summaries.  The RoPE convention
(frequency set, half-split pairs) follows the "SpatioTemporal RoPE" section of
the HorizonStream blog post, with three axes (z, y, x) in place of four.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants and brute force; see the module docstrings for the readings of the
pages each function takes.
"""
from .pack3d import (  # noqa: F401
    CoordsError,
    build_index,
    rope,
    rope_1d,
    rotate,
    POSITION_MODES,
    rope_tables,
    pool_blocks,
    forward,
    forward_naive,
    backward,
    dense_attention,
)
