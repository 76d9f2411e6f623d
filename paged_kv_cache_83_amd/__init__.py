"""paged_kv_cache_83_amd: paged-KV attention decode for AMD MI355X (gfx950).

The computation lives in libpa.so (HIP kernels for gfx950 plus a host block
manager, C interface in include/pa.h). This package is its Python binding.
Importing it loads the library and fails if it has not been built: there is no
fallback implementation.
"""

from ._lib import (DoubleFreeError, OutOfBlocksError, OutOfFramesError, PagedKVError,  # noqa: F401
                   LIB_PATH, PA_TIER_HBM, PA_TIER_HOST, PA_TIER_PENDING_IN, PA_TIER_PENDING_OUT,
                   load as _load)
from .api import (BlockManager, Geometry, Profiler, RadixCache, Swapper, alloc_pools, append_kv,  # noqa: F401
                  blocks_for_tokens, bytes_per_block, bytes_per_token, copy_blocks,
                  copy_to_device, copy_to_host, decode, decode_append, decode_append_noalloc,
                  DecodeAppendCall,
                  decode_workspace_bytes, NOALLOC_SCRATCH_BYTES,
                  gather_blocks, pool_bytes, prefill, prefill_workspace_bytes, scatter_blocks)

_load()
