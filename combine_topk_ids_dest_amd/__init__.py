"""MI355X-native MoE expert-parallel dispatch/combine layout transform.

The path runs in the HIP kernels of libmoe_ep.so (built for gfx950 by
`python -m combine_topk_ids_dest_amd.build`) behind the C ABI of
include/moe_ep.h. `binding` is the thin ctypes layer with the C names;
`emulate` runs W logical expert-parallel ranks on one GPU, where the
exchange between ranks is a rank-stride view of the send buffers.
"""
from .binding import (  # noqa: F401
    MoeEpError,
    load,
    moe_ep_capacities,
    moe_ep_combine_reduce,
    moe_ep_combine_reduce_peers,
    moe_ep_combine_unpack,
    moe_ep_combine_unpack_fused,
    moe_ep_dispatch_pack,
    moe_ep_dispatch_pack_fp4,
    moe_ep_dispatch_pack_fp8,
    moe_ep_expert_batch,
    moe_ep_expert_batch_copy,
    moe_ep_expert_batch_plan,
    moe_ep_sanitize_expert_ids,
    moe_ep_workspace_bytes,
    status_string,
)
