"""ST-DiT attention block on AMD MI355X (gfx950): Python binding of libst.so.

The compute path is the HIP library; this package only marshals arguments
(torch tensors provide device memory and streams).  See include/st.h for the
meaning, layout and error behaviour of every entry point.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, ST_BF16, ST_EALIGN, ST_EINVAL, ST_ELAUNCH, ST_EUNSUPPORTED, ST_EWORKSPACE, ST_F32, ST_OK,
    ST_A2A_S2T, ST_A2A_T2S, ST_ROPE_1D, ST_ROPE_2D, ST_ROPE_NONE, STError, layer_weights, lib, st_a2a_pack,
    st_a2a_unpack, st_attn_chunk, st_attn_chunk_acc, st_attn_merge,
    st_attn_spatial, st_attn_temporal, st_attn_workspace,
    st_block_sliced, st_block_sliced_2s, st_block_sliced_workspace, st_block_sliced_2s_workspace, st_block_sliced_noalloc,
    st_block_sliced_noalloc_max, st_v_change, st_layer_weights, st_out_proj,
    st_out_proj_relayout, st_qkv_norm_rope, st_layer_scales, st_relayout,
    st_rope_table, st_rope_table_floats, st_status_str,
)
