"""MI355X (gfx950) implementation of the Single-Pass mHC residual step.

The step runs in hand-written HIP kernels behind the C ABI of
``include/mhc.h`` (``libmhc.so``, built in-tree by
``stream_hyper_connections_amd.build``); ``binding`` is a thin ctypes layer
for torch tensors, and ``workloads`` holds the seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    MhcError,
    abi_version,
    clear_split_status,
    d_granule,
    PATHS,
    PATHS_N,
    COOPERATIVE,
    fused_step,
    fused_step_backward_n,
    fused_step_backward_workspace_bytes_n,
    fused_step_n,
    fused_step_noalloc,
    fused_step_n_workspace_bytes,
    fused_step_route,
    fused_step_route_n,
    fused_step_workspace_bytes,
    hc_post,
    hc_pre,
    last_error,
    load,
    mixes,
    mixes_n,
    new_workspace,
    n_mix,
    pack_wmix,
    pack_wmix_n,
    rmsnorm,
    sinkhorn4,
    sinkhorn_n,
    split_status,
    status_string,
    three_kernel_step,
    wmix_packed_bytes,
    wmix_packed_bytes_n,
    workspace_for,
)
