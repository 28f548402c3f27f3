"""libpagedattn: paged decode attention for AMD MI355X (gfx950).

The compute path is the C-ABI shared library ``libpagedattn.so`` (hand-written
HIP kernels, declared in ``include/pagedattn.h``); ``binding`` wraps it for
torch tensors.  ``block_manager`` holds the host-side allocator (free list,
block tables, reference counts, copy-on-write plans) and ``workloads`` the
seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    PagedAttnError,
    load_library,
    new_workspace,
    pa_copy_blocks,
    pa_copy_blocks_fp8,
    pa_decode,
    pa_decode_fp8,
    pa_decode_gqa,
    pa_decode_gqa_workspace_size,
    pa_decode_mla,
    pa_decode_mla_workspace_size,
    pa_decode_noalloc,
    pa_decode_workspace_size,
    pa_prefill,
    pa_prefill_workspace_size,
    pa_reshape_and_cache,
    pa_reshape_and_cache_fp8,
    pa_swap_blocks,
    status_string,
)
from .block_manager import BlockManager  # noqa: F401
