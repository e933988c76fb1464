"""NOSA decode-step hot path on MI355X: binding of the libnosa C ABI.

``NosaLayer`` holds one layer's decode state and exposes the four calls of a
decode step (compress_append, select, fetch_delta, sparse_decode). All of the
method's computation runs in the HIP kernels of libnosa.so; importing this
package does not load the library, the first call does (and raises if it was
not built).
"""

from ._lib import (  # noqa: F401
    KIND_AGNOSTIC, KIND_NONE, KIND_QUERY, KIND_SINK, KIND_WINDOW,
    NosaConfig, NosaError, NosaState, header_functions, lib,
)
from .layer import (  # noqa: F401
    LayerAheadStack, LayerShape, NosaLayer, to_block_layout, v_from_tiles, v_to_tiles,
)
