"""MI355X-native Video Sparse Attention (VSA): the forward pass and its backward.

The compute lives in libvsa.so (hand-written HIP kernels for gfx950, C ABI in
include/vsa.h); this package is its Python binding plus the seeded synthetic
workloads.  Importing the package does not load the library: the first call
of a binding function does, and raises if the library is missing.
"""
from ._lib import (  # noqa: F401
    Problem, VsaError, VSA_BF16, VSA_F32, load,
    vsa_permute, vsa_unpermute, vsa_pool, vsa_coarse_topk, vsa_sparse_attn_fwd,
    vsa_check_lut, vsa_perm_index, vsa_status_str, vsa_abi_version,
    vsa_sparse_attn_bwd, vsa_sparse_attn_bwd_workspace_size, vsa_sparse_attn_bwd_noalloc,
    vsa_permute_pool, vsa_sparse_attn_fwd_raster, vsa_sparse_attn_fwd_gather, vsa_mask_to_lut,
    vsa_combine, vsa_combine_bwd, vsa_coarse_bwd, vsa_coarse_bwd_workspace_size, vsa_pool_unpermute_bwd,
    vsa_permute_bnhd, vsa_permute_pool_bnhd, vsa_sparse_attn_fwd_bnhd, vsa_pool_unpermute_bwd_bnhd,
    vsa_cube_table, VSA_CUBES_RASTER, VSA_CUBES_HILBERT, clear_cube_tables, vsa_device_peak,
)
from .pipeline import (VsaAttentionFunction, VsaBackward, VsaForward, clear_forward_cache,  # noqa: F401
                       vsa_attention, vsa_forward)

__all__ = [
    "Problem", "VsaError", "VSA_BF16", "VSA_F32", "load", "VsaForward", "vsa_forward",
    "vsa_permute", "vsa_unpermute", "vsa_pool", "vsa_coarse_topk", "vsa_sparse_attn_fwd",
    "vsa_check_lut", "vsa_perm_index", "vsa_status_str", "vsa_abi_version",
    "vsa_sparse_attn_bwd", "vsa_sparse_attn_bwd_workspace_size", "vsa_sparse_attn_bwd_noalloc",
    "vsa_permute_pool", "vsa_sparse_attn_fwd_raster", "vsa_sparse_attn_fwd_gather", "vsa_mask_to_lut",
    "vsa_combine", "vsa_combine_bwd", "vsa_coarse_bwd", "vsa_coarse_bwd_workspace_size", "vsa_pool_unpermute_bwd",
    "VsaBackward",
    "vsa_permute_bnhd", "vsa_permute_pool_bnhd", "vsa_sparse_attn_fwd_bnhd", "vsa_pool_unpermute_bwd_bnhd",
    "vsa_cube_table", "VSA_CUBES_RASTER", "VSA_CUBES_HILBERT", "clear_cube_tables", "clear_forward_cache",
    "vsa_device_peak", "vsa_attention", "VsaAttentionFunction",
]
