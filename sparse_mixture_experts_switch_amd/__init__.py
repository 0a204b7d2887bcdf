"""Switch FFN layer forward for one AMD MI355X (gfx950), hand-written HIP.

The layer runs in libswitchmoe.so (C ABI in include/switch_moe.h); this
package holds its ctypes binding (`binding`), the build script (`build`) and
the seeded synthetic input generator (`inputs`).  Importing the package does
not load the library; the first binding call does, and fails loudly if the
library has not been built.
"""

from .binding import (  # noqa: F401
    BACKWARD_KERNELS,
    SWITCH_BF16,
    SWITCH_F32,
    SwitchError,
    add_norm,
    backward_workspace_bytes,
    capacity,
    combine,
    combine_add_norm,
    dispatch,
    expert_ffn,
    layer_backward,
    layer_backward_profiled,
    layer_forward,
    layer_forward_noalloc,
    layer_forward_profiled,
    layer_forward_train,
    layer_forward_add_norm,
    launch_names,
    load_library,
    noalloc_scratch_bytes,
    route,
    route_dispatch,
    tile_router,
    tile_weights,
    tiled_router_bytes,
    tiled_router_shape,
    topk_layer_forward,
    topk_workspace_bytes,
    untile_weights,
    workspace_bytes,
)
