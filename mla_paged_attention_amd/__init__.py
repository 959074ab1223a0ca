"""Absorbed Multi-head Latent Attention decode over a paged latent KV cache,
native to AMD Instinct MI355X (gfx950).

The computation lives in ``libmla_mi355x.so`` (hand-written HIP kernels behind
the C ABI declared in ``include/mla.h``); this package is its ctypes binding.
Build the library with ``python -m mla_paged_attention_amd.build``.
"""
from ._binding import (  # noqa: F401
    BLOCK_SIZES,
    EXPORTED_SYMBOLS,
    HEAD_DIM_K,
    HEAD_DIM_V,
    LIBRARY_PATH,
    MAX_FORCED_SPLITS,
    MAX_HEADS,
    MAX_QUERY_LEN,
    MAX_TOPK,
    FP8_GROUP,
    MLA_ERR_HIP,
    MLA_ERR_INVALID_ARG,
    MLA_ERR_NO_DEVICE,
    MLA_ERR_UNSUPPORTED,
    MLA_ERR_WORKSPACE_TOO_SMALL,
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3,
    MLA_OK,
    NOALLOC_SCRATCH_BYTES,
    MLAError,
    abi_version,
    absorb_out,
    absorb_q,
    combine,
    decode,
    decode_noalloc,
    decode_sparse,
    gemm_fp8_blockscale,
    get_workspace_size,
    get_workspace_size_sparse,
    library,
    quant_fp8_groups,
    status_string,
    release_workspaces,
    workspace_for,
)
