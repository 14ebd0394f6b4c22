"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Each function has the C entry point's name and argument order.  Tensor arguments may be
torch tensors (their device pointer is passed), integers (raw device addresses) or None
(NULL).  ``stream`` defaults to torch's current HIP stream.  A non-OK status raises
``MlaError`` unless ``check=False``, in which case the status code is returned.  Nothing
here computes: every step runs in the HIP kernels of libmla.so, and a missing library is
an error, never a fallback.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
# the same library built with MLA_CHECKED: page-table entries bounds-checked on the device
CHECKED_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_checked.so")

MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP, MLA_ERR_TOO_LARGE = range(6)
# size of the per-device scratch array of mla_decode_step_noalloc
MLA_NOALLOC_SCRATCH_BYTES = 64 << 20
MLA_F32, MLA_BF16 = 0, 1

# every symbol include/mla.h declares
EXPORTS = ("mla_absorb_q", "mla_decode_absorbed", "mla_splitkv_combine", "mla_out_uv",
           "gqla_decode_gqa", "gqla_expand_cache", "mla_cache_append", "mla_decode_step",
           "mla_decode_step_noalloc", "gqla_decode_step", "mla_project_q", "mla_fold_q_weights", "mla_project_q_folded",
           "mla_out_project", "mla_fold_o_weights", "mla_out_project_folded",
           "mla_cache_scalars_per_token", "gqla_cache_scalars_per_token",
           "mla_decode_kernel_kind", "gqla_decode_kernel_kind", "mla_checked_bad_pages",
           "mla_status_str")


class MlaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("s_q", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_wheads", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("n_splits", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return "MlaShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class MlaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")


_libs = {}


def load(checked=False):
    """Load libmla.so, or libmla_checked.so with checked=True (once each).  Raises if it has
    not been built."""
    path = CHECKED_LIB_PATH if checked else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        S = ctypes.POINTER(MlaShape)
        sig = {
            "mla_absorb_q": [S, P, P, P, P],
            "mla_decode_absorbed": [S, P, P, P, P, P, P, P],
            "mla_splitkv_combine": [S, ctypes.c_int32, P, P, P, P, P],
            "mla_out_uv": [S, P, P, P, P],
            "gqla_decode_gqa": [S, P, P, P, P, P, P, P, P, P],
            "gqla_expand_cache": [S, P, P, P, P, P, P, P],
            "mla_cache_append": [S, ctypes.c_int32, ctypes.c_float, P, P, P, P, P, P, P],
            "mla_decode_step": [S, P, P, P, P, P, P, P, P, P, P, P, P, P],
            "mla_decode_step_noalloc": [S, P, P, P, P, P, P, P, P, P],
            "gqla_decode_step": [S, P, P, P, P, P, P, P, P, P, P, P],
            "mla_project_q": [S, ctypes.c_int32, ctypes.c_float, P, P, P, P, P],
            "mla_fold_q_weights": [S, ctypes.c_int32, P, P, P, P],
            "mla_project_q_folded": [S, ctypes.c_int32, ctypes.c_float, P, P, P, P, P],
            "mla_out_project": [S, ctypes.c_int32, P, P, P, P],
            "mla_fold_o_weights": [S, ctypes.c_int32, P, P, P, P],
            "mla_out_project_folded": [S, ctypes.c_int32, P, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, ctypes.c_int
        for name in ("mla_cache_scalars_per_token", "gqla_cache_scalars_per_token"):
            f = getattr(lib, name)
            f.argtypes, f.restype = [S], ctypes.c_int64
        for name in ("mla_decode_kernel_kind", "gqla_decode_kernel_kind"):
            f = getattr(lib, name)
            f.argtypes, f.restype = [S], ctypes.c_int32
        lib.mla_checked_bad_pages.argtypes, lib.mla_checked_bad_pages.restype = [], ctypes.c_int32
        lib.mla_status_str.argtypes, lib.mla_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        _libs[path] = lib
    return _libs[path]


def mla_checked_bad_pages(checked=True):
    """1 if a checked call met an out-of-range page-table entry since the last query (then
    cleared), 0 if not; -1 from libmla.so, which has no checks; -2 on a HIP error."""
    return int(load(checked).mla_checked_bad_pages())


def make_shape(batch, s_q, n_heads, n_wheads, d_c, d_rope, d_nope, d_v, max_pages,
               num_pages, n_splits, softmax_scale, dtype, page_size=64, split_tokens=0):
    if isinstance(dtype, str):
        dtype = {"f32": MLA_F32, "bf16": MLA_BF16}[dtype]
    return MlaShape(batch, s_q, n_heads, n_wheads, d_c, d_rope, d_nope, d_v, page_size,
                    max_pages, num_pages, n_splits, split_tokens, softmax_scale, dtype)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _call(name, shape, ptrs, stream, check, mid=()):
    st = getattr(load(), name)(ctypes.byref(shape), *mid, *[_ptr(p) for p in ptrs],
                               _stream(stream))
    if check and st != MLA_OK:
        raise MlaError(name, st)
    return st


def status_str(status):
    return load().mla_status_str(status).decode()


def mla_absorb_q(shape, q, w_uk, q_abs, stream=None, check=True):
    return _call("mla_absorb_q", shape, (q, w_uk, q_abs), stream, check)


def mla_decode_absorbed(shape, q_abs, kv_pool, page_table, ctx_lens, o_part, lse_part,
                        stream=None, check=True):
    return _call("mla_decode_absorbed", shape,
                 (q_abs, kv_pool, page_table, ctx_lens, o_part, lse_part), stream, check)


def mla_splitkv_combine(shape, width, o_part, lse_part, o, lse=None, stream=None, check=True):
    st = load().mla_splitkv_combine(ctypes.byref(shape), int(width), _ptr(o_part),
                                    _ptr(lse_part), _ptr(o), _ptr(lse), _stream(stream))
    if check and st != MLA_OK:
        raise MlaError("mla_splitkv_combine", st)
    return st


def mla_out_uv(shape, o_lat, w_uv, out, stream=None, check=True):
    return _call("mla_out_uv", shape, (o_lat, w_uv, out), stream, check)


def gqla_decode_gqa(shape, q, k_pool, v_pool, kr_pool, page_table, ctx_lens, o_part,
                    lse_part, stream=None, check=True):
    return _call("gqla_decode_gqa", shape,
                 (q, k_pool, v_pool, kr_pool, page_table, ctx_lens, o_part, lse_part),
                 stream, check)


def gqla_expand_cache(shape, kv_pool, w_uk, w_uv, k_pool, v_pool, kr_pool, stream=None,
                      check=True):
    return _call("gqla_expand_cache", shape, (kv_pool, w_uk, w_uv, k_pool, v_pool, kr_pool),
                 stream, check)


def mla_cache_append(shape, d_model, rope_base, h, w_dkv, w_kr, page_table, ctx_lens,
                     kv_pool, stream=None, check=True):
    return _call("mla_cache_append", shape, (h, w_dkv, w_kr, page_table, ctx_lens, kv_pool),
                 stream, check, mid=(int(d_model), float(rope_base)))


def mla_decode_step(shape, q, w_uk, w_uv, kv_pool, page_table, ctx_lens, q_abs, o_part,
                    lse_part, o_lat, out, lse=None, stream=None, check=True):
    return _call("mla_decode_step", shape,
                 (q, w_uk, w_uv, kv_pool, page_table, ctx_lens, q_abs, o_part, lse_part,
                  o_lat, out, lse), stream, check)


def mla_decode_step_noalloc(shape, q, w_uk, w_uv, kv_pool, page_table, ctx_lens, out,
                            lse=None, stream=None, check=True):
    return _call("mla_decode_step_noalloc", shape,
                 (q, w_uk, w_uv, kv_pool, page_table, ctx_lens, out, lse), stream, check)


def gqla_decode_step(shape, q, k_pool, v_pool, kr_pool, page_table, ctx_lens, o_part,
                     lse_part, out, lse=None, stream=None, check=True):
    return _call("gqla_decode_step", shape,
                 (q, k_pool, v_pool, kr_pool, page_table, ctx_lens, o_part, lse_part, out,
                  lse), stream, check)


def mla_cache_scalars_per_token(shape):
    return load().mla_cache_scalars_per_token(ctypes.byref(shape))


def gqla_cache_scalars_per_token(shape):
    return load().gqla_cache_scalars_per_token(ctypes.byref(shape))


def mla_decode_kernel_kind(shape):
    return load().mla_decode_kernel_kind(ctypes.byref(shape))


def gqla_decode_kernel_kind(shape):
    return load().gqla_decode_kernel_kind(ctypes.byref(shape))


def mla_status_str(status):
    return status_str(status)


def mla_project_q(shape, d_model, rope_base, x, w_q, ctx_lens, q, stream=None, check=True):
    return _call("mla_project_q", shape, (x, w_q, ctx_lens, q), stream, check,
                 mid=(int(d_model), float(rope_base)))


def mla_fold_q_weights(shape, d_model, w_q, w_uk, w_q_folded, stream=None, check=True):
    return _call("mla_fold_q_weights", shape, (w_q, w_uk, w_q_folded), stream, check,
                 mid=(int(d_model),))


def mla_project_q_folded(shape, d_model, rope_base, x, w_q_folded, ctx_lens, q_abs,
                         stream=None, check=True):
    return _call("mla_project_q_folded", shape, (x, w_q_folded, ctx_lens, q_abs), stream,
                 check, mid=(int(d_model), float(rope_base)))


def mla_out_project(shape, d_model, out, w_o, y, stream=None, check=True):
    return _call("mla_out_project", shape, (out, w_o, y), stream, check, mid=(int(d_model),))


def mla_fold_o_weights(shape, d_model, w_o, w_uv, w_o_folded, stream=None, check=True):
    return _call("mla_fold_o_weights", shape, (w_o, w_uv, w_o_folded), stream, check,
                 mid=(int(d_model),))


def mla_out_project_folded(shape, d_model, o_lat, w_o_folded, y, stream=None, check=True):
    return _call("mla_out_project_folded", shape, (o_lat, w_o_folded, y), stream, check,
                 mid=(int(d_model),))
