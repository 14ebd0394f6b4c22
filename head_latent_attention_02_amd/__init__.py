"""MI355X (gfx950) single-step MLA / GQLA decode attention.

The compute lives in ``libmla.so`` (hand-written HIP kernels behind the C ABI of
``include/mla.h``); this package is its thin ctypes binding.  Importing it does not load
the library; the first call does, and raises if the library has not been built.
"""
from ._lib import (  # noqa: F401
    CHECKED_LIB_PATH, EXPORTS, LIB_PATH, MLA_BF16, MLA_ERR_HIP, MLA_ERR_NULL, MLA_ERR_SHAPE,
    MLA_ERR_TOO_LARGE, MLA_ERR_UNSUPPORTED, MLA_F32, MLA_NOALLOC_SCRATCH_BYTES, MLA_OK,
    MlaError, MlaShape, gqla_cache_scalars_per_token,
    gqla_decode_gqa, gqla_decode_kernel_kind, gqla_decode_step, gqla_expand_cache, load,
    make_shape, mla_absorb_q, mla_cache_append, mla_cache_scalars_per_token,
    mla_decode_absorbed, mla_decode_kernel_kind, mla_decode_step, mla_decode_step_noalloc,
    mla_out_uv,
    mla_checked_bad_pages, mla_splitkv_combine, mla_status_str, mla_project_q,
    mla_fold_q_weights, mla_project_q_folded, mla_out_project, mla_fold_o_weights,
    mla_out_project_folded)
