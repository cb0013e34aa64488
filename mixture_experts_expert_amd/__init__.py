"""MI355X-native capacity-padded, permute-free MoE FFN forward and backward.

The compute lives in libmoe_native.so (hand-written HIP for gfx950, C ABI in
include/moe_native.h); this package is its thin ctypes binding plus a
static-buffer forward helper.  Importing it fails loudly if the library is
not built: there is no CPU or PyTorch fallback.
"""

from ._native import (  # noqa: F401
    LIB_PATH,
    MoEError,
    header_functions,
    lib,
    moe_align,
    moe_dispatch_rows,
    moe_dropless_bound,
    moe_gather_combine,
    moe_grouped_fc1_dgrad,
    moe_grouped_fc1_swiglu,
    moe_grouped_fc1_swiglu_dropless,
    moe_grouped_fc1_swiglu_save,
    moe_grouped_fc1_wgrad,
    moe_grouped_fc1_wgrad_accum,
    moe_grouped_fc2,
    moe_grouped_fc2_rows,
    moe_grouped_fc2_dgrad,
    moe_grouped_fc2_dropless,
    moe_grouped_fc2_wgrad,
    moe_grouped_fc2_wgrad_accum,
    moe_grouped_ffn_fwd,
    moe_grouped_ffn_fwd_dropless,
    moe_layout_block_m,
    moe_padded_capacity,
    moe_probe_copy,
    moe_probe_gemm_loop,
    moe_probe_lds_read,
    moe_probe_lds_ring,
    moe_probe_mfma_rate,
    moe_probe_read,
    moe_probe_read_pieces,
    moe_probe_write,
    moe_probe_write_pieces,
    moe_probe_write_tiles,
    PROBE_HEADER_PATH,
    moe_route_bwd,
    moe_route_capacity,
    moe_route_capacity_align,
    moe_route_capacity_align_noalloc,
    moe_route_capacity_workspace_bytes,
    moe_route_dropless,
    moe_route_dropless_live,
    moe_source_capacity,
    moe_status_string,
    moe_swiglu_bwd,
    route_workspace,
)
from .serving import BucketLadder, ServingLadder  # noqa: F401
from .forward import (  # noqa: F401
    DroplessBuffers,
    MoEBackwardBuffers,
    MoEBuffers,
    forward,
    forward_dropless,
)
