"""fp64 CPU oracle of the VSA forward pass and its backward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package; the product path never does.
"""
from .vsa_oracle import (  # noqa: F401
    check_grid, perm_index, permute, unpermute, pool, coarse_scores,
    softmax_rows, coarse_attention, topk_lut, fine_attention,
    fine_attention_masked, fine_attention_bwd, combine, vsa_forward, mask_to_lut,
    combine_bwd, coarse_attention_bwd, pool_bwd, vsa_backward,
    kv_group, expand_kv_heads, reduce_kv_heads,
    token_layout, hilbert_index, cube_sequence, gather_padded, scatter_padded, pool_real, pool_real_bwd,
)
