"""Layerwise weight offload for a DiT block stack on one MI355X (gfx950).

Thin Python binding over the C ABI in ``include/lwo.h`` (``liblwo.so``,
built in-tree by ``layerwise_weight_offload_amd.build``).  Every function
here only marshals arguments; all work runs in the library's C++ host code
and HIP kernels.  Device buffers and streams are passed as raw integers
(``tensor.data_ptr()``, ``stream.cuda_stream``), so the binding uses nothing
from PyTorch; when PyTorch is installed it is imported before the library is
loaded, so that both bind to one HIP runtime in the process.

Importing fails loudly if the library has not been built: there is no
fallback implementation.
"""
from ._binding import (  # noqa: F401
    BF16, F32, FP8_E4M3, KTILED, ROWS, HOST_PIN_COPY, HOST_REGISTER, HOST_SHARD, HOST_STAGED, KIND_DIT, KIND_VIDEO, LIB_PATH,
    LwoError, ModelDesc, Stats, Store, block_layout, build_block_store, extent_checksum, last_error,
    pack_block, register_ranges, exported_symbols, op_attention, op_layernorm, op_linear, op_quantize_rows,
    op_rmsnorm_qk, probe_mfma, sha256, cache_publish, cache_open, CacheEntry, CacheExtents, build_mixed_store,
    build_shard_store, tile_weight, run_blocks_noalloc, NOALLOC_SCRATCH_BYTES,
)
