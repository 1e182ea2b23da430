"""MI355X (gfx950) implementation of the DeepSeek-V4 CSA / HCA attention forward.

The computation lives in hand-written HIP kernels behind the C ABI of
``libcsa.so`` (``include/csa.h``); this package is the thin Python binding over it
(torch tensors supply device memory and streams).  Build the library with
``python -m compressed_sparse_attention_07_amd.build``.
"""

from ._lib import (  # noqa: F401
    CSA_BF16, CSA_F32, CSA_FLAG_BF16_SCORES, CSA_FLAG_QKV_NORM, CSA_FP8MIX, CSA_MODE_CSA, CSA_MODE_HCA, CSA_MXFP4, Buf, CSAError, EXPORTS, LIB_PATH,
    DecodePool, ForwardCall, PreparedCall, csa_decode_step, csa_decode_step_workspace_size, decode_desc,
    csa_compress, csa_compress_norm, csa_forward, csa_grouped_out_proj, csa_grouped_out_proj_workspace_size,
    csa_rmsnorm, csa_forward_workspace_size, csa_index_scores, csa_index_topk, csa_quantize, csa_sparse_mqa, csa_sparse_mqa_noalloc, csa_topk,
    hca_dense_attn, layer_desc, lib,
)
