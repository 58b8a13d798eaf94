"""CPU fp64 oracle for variable-length block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.
"""
from .ref import (  # noqa: F401
    scale_of,
    lengths,
    selected_blocks,
    visited_blocks,
    index_products,
    tile_index_products,
    forward,
    backward,
)
