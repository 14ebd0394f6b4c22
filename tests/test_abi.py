"""The C ABI loads, exports every declared symbol, and validates on the host (CPU only).

Every call here fails validation before any HIP call, so no device is needed.
"""
import ctypes
import os
import re
import subprocess

import pytest

import head_latent_attention_02_amd as mla
from oracle import mla as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH),
                                reason="libmla.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", text, flags=re.M)))


def good_shape(**kw):
    base = dict(batch=2, s_q=1, n_heads=8, n_wheads=8, d_c=64, d_rope=16, d_nope=32, d_v=32,
                max_pages=4, num_pages=8, n_splits=4, softmax_scale=0.1, dtype="f32")
    base.update(kw)
    return mla.make_shape(**base)


def test_header_and_binding_agree():
    assert declared_functions() == sorted(mla.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = mla.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported


def test_checked_library_exports_every_declared_symbol():
    """libmla_checked.so is the same library with device-side page-table checks."""
    assert os.path.exists(mla.CHECKED_LIB_PATH)
    lib = mla.load(checked=True)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_unchecked_library_reports_no_checks():
    # returns before any HIP call in libmla.so
    assert mla.mla_checked_bad_pages(checked=False) == -1


def test_shape_struct_layout():
    assert ctypes.sizeof(mla.MlaShape) == 15 * 4


def test_status_strings():
    for st in range(5):
        assert isinstance(mla.mla_status_str(st), str) and mla.mla_status_str(st)
    assert mla.mla_status_str(99) == "unknown status"


def test_cache_sizes_match_oracle_and_pages():
    s = good_shape(d_c=512, d_rope=64, d_nope=128, d_v=128, n_heads=32, n_wheads=8,
                   dtype="bf16")
    assert mla.mla_cache_scalars_per_token(s) == ref.mla_cache_scalars_per_token(512, 64) == 576
    assert mla.gqla_cache_scalars_per_token(s) == \
        ref.gqla_expanded_cache_scalars_per_token(8, 128, 128, 64) == 2112
    assert mla.mla_cache_scalars_per_token(s) / ref.gqa_cache_scalars_per_token(8, 128) \
        == 0.28125


@pytest.mark.parametrize("bad,status", [
    (dict(batch=0), mla.MLA_ERR_SHAPE),
    (dict(s_q=-1), mla.MLA_ERR_SHAPE),
    (dict(n_heads=8, n_wheads=3), mla.MLA_ERR_SHAPE),
    (dict(n_splits=0), mla.MLA_ERR_SHAPE),
    (dict(softmax_scale=0.0), mla.MLA_ERR_SHAPE),
    (dict(softmax_scale=float("nan")), mla.MLA_ERR_SHAPE),
    (dict(page_size=32), mla.MLA_ERR_UNSUPPORTED),
    (dict(d_c=60), mla.MLA_ERR_UNSUPPORTED),
    (dict(d_c=1024, d_rope=64), mla.MLA_ERR_UNSUPPORTED),
    (dict(dtype=7), mla.MLA_ERR_UNSUPPORTED),
    (dict(split_tokens=100), mla.MLA_ERR_SHAPE),
    (dict(split_tokens=64, n_splits=3), mla.MLA_ERR_SHAPE),
    (dict(max_pages=0), mla.MLA_ERR_SHAPE),
    # products of individually valid sizes that would overflow a launch grid
    (dict(batch=65535, n_splits=65535), mla.MLA_ERR_UNSUPPORTED),
    (dict(batch=40000, s_q=8, n_heads=128, n_wheads=128), mla.MLA_ERR_UNSUPPORTED),
    (dict(batch=4096, s_q=1, n_heads=8192, n_wheads=8192, n_splits=1),
     mla.MLA_ERR_UNSUPPORTED),
    (dict(batch=65535, s_q=5), mla.MLA_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected_before_any_hip_call(bad, status):
    s = good_shape(**bad)
    fake = 0x1000   # never dereferenced: validation fails first
    assert mla.mla_absorb_q(s, fake, fake, fake, stream=0, check=False) == status
    assert mla.mla_decode_absorbed(s, fake, fake, fake, fake, fake, fake, stream=0,
                                   check=False) == status
    assert mla.gqla_decode_gqa(s, fake, fake, fake, fake, fake, fake, fake, fake, stream=0,
                               check=False) == status
    assert mla.mla_decode_kernel_kind(s) == -1
    assert mla.mla_cache_scalars_per_token(s) == -1


def test_null_pointers_rejected():
    s = good_shape()
    f = 0x1000
    assert mla.mla_absorb_q(s, None, f, f, stream=0, check=False) == mla.MLA_ERR_NULL
    assert mla.mla_decode_absorbed(s, f, f, None, f, f, f, stream=0,
                                   check=False) == mla.MLA_ERR_NULL
    assert mla.mla_splitkv_combine(s, 64, f, None, f, stream=0,
                                   check=False) == mla.MLA_ERR_NULL
    assert mla.mla_out_uv(s, f, f, None, stream=0, check=False) == mla.MLA_ERR_NULL
    assert mla.gqla_expand_cache(s, f, f, f, f, f, None, stream=0,
                                 check=False) == mla.MLA_ERR_NULL
    assert mla.mla_decode_step(s, f, f, f, f, f, f, f, f, f, f, None, stream=0,
                               check=False) == mla.MLA_ERR_NULL
    assert mla.gqla_decode_step(s, f, f, f, f, f, f, f, f, None, stream=0,
                                check=False) == mla.MLA_ERR_NULL
    assert mla.mla_cache_append(s, 5120, 1e4, f, f, f, f, f, None, stream=0,
                                check=False) == mla.MLA_ERR_NULL
    # a NULL shape pointer
    lib = mla.load()
    assert lib.mla_absorb_q(None, f, f, f, None) == mla.MLA_ERR_NULL


def test_combine_width_checked():
    s = good_shape()
    f = 0x1000
    assert mla.mla_splitkv_combine(s, 0, f, f, f, stream=0, check=False) == mla.MLA_ERR_SHAPE
    assert mla.mla_splitkv_combine(s, 2048, f, f, f, stream=0,
                                   check=False) == mla.MLA_ERR_UNSUPPORTED


def test_cache_append_arguments_checked():
    s = good_shape()
    f = 0x1000
    for d_model, base, status in ((0, 1e4, mla.MLA_ERR_SHAPE), (-8, 1e4, mla.MLA_ERR_SHAPE),
                                  (5120, 0.0, mla.MLA_ERR_SHAPE),
                                  (5120, float("nan"), mla.MLA_ERR_SHAPE),
                                  (5124, 1e4, mla.MLA_ERR_UNSUPPORTED)):
        assert mla.mla_cache_append(s, d_model, base, f, f, f, f, f, f, stream=0,
                                    check=False) == status
    assert mla.mla_cache_append(good_shape(batch=0), 5120, 1e4, f, f, f, f, f, f, stream=0,
                                check=False) == mla.MLA_ERR_SHAPE


def test_error_raises_with_check():
    with pytest.raises(mla.MlaError):
        mla.mla_absorb_q(good_shape(batch=0), 1, 1, 1, stream=0)


def test_projection_arguments_checked():
    s = good_shape(d_c=512, d_rope=64, d_nope=128, d_v=128, n_heads=128, n_wheads=128,
                   dtype="bf16")
    fake = 0x1000
    assert mla.mla_project_q(s, 5120, 1e4, fake, fake, fake, None, stream=0,
                             check=False) == mla.MLA_ERR_NULL
    assert mla.mla_project_q(s, 5000, 1e4, fake, fake, fake, fake, stream=0,
                             check=False) == mla.MLA_ERR_UNSUPPORTED   # d_model % 256
    assert mla.mla_project_q(s, 0, 1e4, fake, fake, fake, fake, stream=0,
                             check=False) == mla.MLA_ERR_SHAPE
    assert mla.mla_project_q(s, 5120, -1.0, fake, fake, fake, fake, stream=0,
                             check=False) == mla.MLA_ERR_SHAPE
    f32 = good_shape(d_c=512, d_rope=64, d_nope=128, d_v=128, n_heads=128, n_wheads=128)
    for fn, args in ((mla.mla_fold_q_weights, (fake, fake, fake)),
                     (mla.mla_out_project, (fake, fake, fake)),
                     (mla.mla_fold_o_weights, (fake, fake, fake)),
                     (mla.mla_out_project_folded, (fake, fake, fake))):
        assert fn(f32, 5120, *args, stream=0, check=False) == mla.MLA_ERR_UNSUPPORTED
        assert fn(s, 5120, fake, fake, None, stream=0, check=False) == mla.MLA_ERR_NULL


def test_kernel_kind_is_host_only():
    assert mla.mla_decode_kernel_kind(good_shape()) in (0, 1)
    assert mla.gqla_decode_kernel_kind(good_shape(n_wheads=2)) in (0, 1)


def test_noalloc_step_rejects_workspaces_beyond_its_scratch():
    """mla_decode_step_noalloc checks that q_abs, o_part, lse_part and o_lat (each rounded up
    to 256 bytes) fit its fixed scratch before it looks the scratch up or launches."""
    fake = 0x1000

    def need(B, s_q, H, S, d_c=512, d_rope=64, es=2):
        up = lambda x: -(-x // 256) * 256   # noqa: E731
        rows = B * s_q * H
        return (up(rows * (d_c + d_rope) * es) + up(rows * S * d_c * 4) + up(rows * S * 4)
                + up(rows * d_c * 4))

    dims = dict(d_c=512, d_rope=64, d_nope=128, d_v=128, n_heads=128, n_wheads=128,
                dtype="bf16", max_pages=2048, num_pages=8192)
    args = (fake,) * 7
    for B, s_q, S in ((8, 1, 32), (64, 2, 6)):   # 8 x 128 heads x 32 splits; ragged MTP
        assert need(B, s_q, 128, S) > mla.MLA_NOALLOC_SCRATCH_BYTES
        s = good_shape(batch=B, s_q=s_q, n_splits=S, **dims)
        assert mla.mla_decode_step_noalloc(s, *args, fake, stream=0,
                                           check=False) == mla.MLA_ERR_TOO_LARGE
    assert need(7, 1, 128, 32) <= mla.MLA_NOALLOC_SCRATCH_BYTES   # the largest B that fits
    s = good_shape(batch=4, n_splits=32, **dims)
    assert mla.mla_decode_step_noalloc(s, *args[:6], None, fake, stream=0,   # out NULL
                                       check=False) == mla.MLA_ERR_NULL
    assert mla.mla_decode_step_noalloc(good_shape(batch=0), *args, fake, stream=0,
                                       check=False) == mla.MLA_ERR_SHAPE
    assert "scratch" in mla.mla_status_str(mla.MLA_ERR_TOO_LARGE)
