"""MI355X-native compressed-sparse-attention (CSA) decode path.

The compute lives in ``libcsa.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/csa.h``); this package is its thin Python
binding.  Build the library with ``compressed_sparse_attention_reduce_amd.build.build()``.
"""

from .binding import (  # noqa: F401
    CSA_BF16,
    CSA_F32,
    CSA_FP8_E4M3,
    CsaError,
    LayerDesc,
    StepIO,
    csa_compress,
    csa_decode_step,
    csa_decode_step_workspace_size,
    csa_decode_step_noalloc,
    csa_decode_step_scan,
    csa_decode_step_attend,
    csa_decode_step_noalloc_max_bytes,
    csa_gather,
    csa_hca_decode_step,
    csa_hca_decode_step_workspace_size,
    csa_index_score,
    csa_index_score_fp8,
    csa_index_topk,
    csa_index_topk_fp8,
    csa_pack_kv_mixed,
    csa_read_probe,
    csa_decode_step_dev,
    csa_decode_step_dev_ring_size,
    MIX_REC_BYTES,
    csa_index_topk_workspace_size,
    csa_last_error,
    csa_layer_advance,
    csa_prefill_attn,
    csa_prefill_attn_mixed,
    csa_quantize_fp8,
    csa_quantize_query_fp8,
    csa_sparse_attn,
    csa_sparse_attn_workspace_size,
    csa_topk,
    csa_topk_workspace_size,
    lib,
    make_layer_desc,
    make_step_io,
)
