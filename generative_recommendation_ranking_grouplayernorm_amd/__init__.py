"""MTGR HSTU layer on AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libmtgr.so`` (C ABI: include/mtgr.h);
``binding`` exposes the same entry points to Python with torch tensors as
device buffers.
"""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MtgrError,
    load_library,
    mtgr_group_layernorm,
    mtgr_group_layernorm_bwd,
    mtgr_hstu_attn_bwd,
    mtgr_hstu_attn_fwd,
    mtgr_hstu_layer_bwd,
    mtgr_hstu_layer_fwd,
    mtgr_jagged_prep,
    mtgr_status_string,
    mtgr_version,
    mtgr_workspace_size,
)
