"""MI355X (gfx950) DeepSeek Sparse Attention layer step.

The computation lives in ``libdsa_amd.so`` (HIP kernels behind the C ABI of
``include/dsa.h``); this package is its Python binding:

    indexer_prep(q, k, rope_cos, rope_sin, start, rope_dim, k_cache, k_scale)
                                                                         -> (q_fp8, q_scale)
    index_scores(q_fp8, q_scale, w, k_fp8, k_scale, lens, sm_scale_i)  -> scores
    topk(scores, lens, k)                                                -> idx
    sparse_mla_decode(q, latent, idx, lens, Dv, sm_scale)                -> (out, lse)
        (latent: q's dtype, or uint8 [B,Lmax,656] rows in the FP8 storage form with
         bf16 q: 512 e4m3fn codes, four fp32 block scales, 64 bf16 rope values)
    sparse_mla_prefill(q, k, v, idx, sm_scale)                           -> (out, lse)
    LayerStep(...)()                                                     -> (out, lse)
    LayerStep(..., workspace=False).call_noalloc()                       -> (out, lse)
        (the library's fixed per-device scratch instead of a workspace; at most
         NOALLOC_SCRATCH_BYTES of it)

    diag_fp8_mfma_dots(a, b)                                             -> (fp8, bf16)
        (diagnostic: 128-code FP8 dot products on both matrix-core forms)

Build the library with ``python -m deepseek_dsa_indexer_amd.build``.
"""
from ._native import (NOALLOC_SCRATCH_BYTES, DSAError, LayerStep, diag_fp8_mfma_dots, index_scores,
                      indexer_prep, library_path, load, profile_begin, profile_end,
                      sparse_mla_decode, sparse_mla_prefill, topk)

__all__ = ["NOALLOC_SCRATCH_BYTES", "DSAError", "LayerStep", "diag_fp8_mfma_dots", "index_scores",
           "indexer_prep", "library_path", "load", "profile_begin", "profile_end",
           "sparse_mla_decode", "sparse_mla_prefill", "topk"]
