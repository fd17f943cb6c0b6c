"""MI355X (gfx950) implementation of the VideoMLA latent-KV chunk step.

The work happens in libmla.so (C ABI in include/mla.h, HIP kernels in csrc/);
this package only marshals arguments to it (see _lib) and offers a small
device-memory holder for one layer (see layer).
"""
from ._lib import (  # noqa: F401
    MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_ALIGNMENT, MLA_ERR_WORKSPACE,
    MLA_ERR_HIP, MLA_BF16, MLA_F32, MLA_ROPE_AT_WRITE, MLA_ROPE_AT_READ, Config, Weights, Chunk,
    Cache, interleaved_cache, split_cache,
    MLAError, load, make_config, make_chunk, make_weights, validate, workspace_bytes, cache_bytes, cache_write,
    chunk_attention, step, step_static, MLA_STATIC_SCRATCH_BYTES, value_absorbed_weights, query_absorbed_weights, latent_attention,
    set_timing_events, attention_grid, overflow_flags, status_string,
    last_error, SIGNATURES, LIB_PATH,
)
