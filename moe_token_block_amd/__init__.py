"""moe_token_block_amd -- block-scaled NVFP4 / MXFP8 quantization of MoE token rows on MI355X (gfx950).

The compute path is the HIP library ``libmoe_token_block.so`` behind the C ABI
declared in ``include/moe_token_block.h``; ``binding`` is its thin Python
binding (PyTorch supplies device memory and streams).
"""

from .binding import (  # noqa: F401
    EP_ROUND_NEAREST, EP_ROUND_SR_ELEMENT, EP_ROUND_SR_STREAM, EP_ROUND_SR_ELEMENT_CARRY, EP_ROUND_SR_STREAM_CARRY,
    EP_DEVERR_EXPERT_ID, EpError,
    ep_abi_version, ep_status_string, ep_nvfp4_packed_row_bytes, ep_route_capacity, ep_rht_sign_mask,
    ep_nvfp4_pack, ep_nvfp4_unpack, ep_mxfp8_pack, ep_route_plan, ep_nvfp4_direct_receive,
    ep_mxfp8_direct_receive, ep_nvfp4_expert_scale, ep_nvfp4_direct_receive_scaled, dswiglu_nvfp4_quant,
    ep_nvfp4_pack_scatter, ep_nvfp4_columnwise_grouped, ep_nvfp4_direct_receive_kblock, ep_mxfp4_direct_receive, ep_mxfp4_kblock_tile,
    ep_nvfp4_direct_receive_sr, ep_receive_workspace_bytes, ep_nvfp4_direct_receive_topk,
    dswiglu_nvfp4_quant_noalloc, EP_NOALLOC_SCRATCH_BYTES, EP_ERR_SCRATCH,
    lib, LIB_PATH, EXPORTS,
)
