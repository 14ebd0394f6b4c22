"""GPU parity of the cache-append step (``mla_cache_append``) against the float64 oracle.

Written rows: rel_err = max |gpu - oracle| / max |oracle| over the written rows, bars 1e-4
(fp32) and 2e-2 (bf16; the row is rounded to bf16 once).  Every other pool row must keep
its bits (NaN padding included).  The last test decodes over the appended cache.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_02_amd as mla
from oracle import append as ref_append
from oracle import mla as ref
from workloads import get_config, make_append_inputs, make_inputs
from workloads.device import DeviceInputs, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
BASE = ref_append.ROPE_BASE


def announce(msg):
    print(msg, flush=True)


def pool_bits(d, inp):
    """Device pool -> numpy bit patterns (uint16 for bf16, uint32 for fp32)."""
    if inp.is_bf16:
        return d.pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return d.pool.cpu().numpy().view(np.uint32)


def bits_to_f32(bits):
    if bits.dtype == np.uint16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits.view(np.float32)


def run_append(inp, ap, d=None):
    c = inp.cfg
    d = d or DeviceInputs(inp)
    h, w_dkv, w_kr = (to_dev(x, c.dtype) for x in (ap.h, ap.w_dkv, ap.w_kr))
    mla.mla_cache_append(d.shape, ap.d_model, BASE, h, w_dkv, w_kr, d.page_table,
                         d.ctx_lens, d.pool)
    torch.cuda.synchronize()
    return d


def check_append(inp, ap, d=None):
    c = inp.cfg
    announce(f"case append {c.name} B={c.batch} s_q={c.s_q} d_model={ap.d_model} "
             f"ctx={list(inp.ctx_lens)[:6]}")
    before = inp.pool.view(np.uint16 if inp.is_bf16 else np.uint32).copy()
    d = run_append(inp, ap, d)
    got = pool_bits(d, inp)
    pos = ref_append.new_token_positions(inp.ctx_lens, c.s_q)
    rows = ref_append.append_rows(ap.h, ap.w_dkv, ap.w_kr, np.maximum(pos, 0), BASE)
    written = np.zeros(before.shape[:2], bool)
    want, have = [], []
    for b in range(c.batch):
        for s in range(c.s_q):
            t = int(pos[b, s])
            if t < 0:
                continue
            page = int(inp.page_table[b, t // c.page_size])
            if page < 0:
                continue
            written[page, t % c.page_size] = True
            want.append(rows[b, s])
            have.append(bits_to_f32(got[page, t % c.page_size]))
    assert np.array_equal(got[~written], before[~written]), "rows outside the new tokens changed"
    if want:
        e = float(np.max(np.abs(np.array(have) - np.array(want))) / np.max(np.abs(want)))
        announce(f"  {len(want)} rows written, rel_err {e:.3e}")
        assert e <= TOL[c.dtype]
    return d, int(written.sum())


def test_tiny_f32_append():
    cfg = get_config("tiny-f32", batch=4, s_q=2, ctx=("list", [1, 64, 65, 200]))
    inp = make_inputs(cfg, seed=31)
    _, n = check_append(inp, make_append_inputs(cfg, d_model=64, seed=31))
    assert n == 7                       # the first sequence holds one token: one row


@pytest.mark.parametrize("s_q,ctx", [(1, [1, 63, 64, 65, 131072]), (2, [1, 2, 130, 4097])])
def test_bf16_append_dsv2_shapes(s_q, ctx):
    """Page boundaries (slots 63 and 0), a position near 2^17 (large rotation angles), and
    at s_q = 2 a sequence with fewer tokens than new queries."""
    cfg = get_config("dsv2-b16-t4096", batch=len(ctx), s_q=s_q, ctx=("list", ctx))
    inp = make_inputs(cfg, seed=32)
    check_append(inp, make_append_inputs(cfg, seed=32))


def test_bf16_append_vector_path():
    """A hidden width that is a multiple of 8 but not of 32 takes the vector-unit kernel
    (the matrix-core one needs whole 32-wide K-steps)."""
    cfg = get_config("dsv2-b16-t4096", batch=3, s_q=2, ctx=("list", [1, 64, 3000]))
    inp = make_inputs(cfg, seed=36)
    check_append(inp, make_append_inputs(cfg, d_model=200, seed=36))


def test_bf16_append_gqla_shape():
    cfg = get_config("gqla-b32-t8192", batch=3, ctx=("list", [5, 700, 65536]))
    inp = make_inputs(cfg, seed=33)
    check_append(inp, make_append_inputs(cfg, d_model=4096, seed=33))


def test_unmapped_pages_are_left_alone():
    cfg = get_config("dsv2-b16-t4096", batch=3, ctx=("list", [100, 200, 300]))
    inp = make_inputs(cfg, seed=34)
    inp.page_table[1, :] = -1           # sequence 1 has no pages mapped: nothing written
    _, n = check_append(inp, make_append_inputs(cfg, seed=34))
    assert n == 2


def test_full_long_b4_t131072_append():
    """The long-context workload's four new tokens, in the configuration the benchmark
    times (positions 131071, hidden 5120)."""
    cfg = get_config("long-b4-t131072")
    inp = make_inputs(cfg)
    _, n = check_append(inp, make_append_inputs(cfg))
    assert n == 4


def test_decode_over_the_appended_cache():
    """Append, then run the absorbed step: the output matches the oracle's decode over the
    oracle's appended cache (the new rows are the last tokens each query row sees)."""
    cfg = get_config("dsv2-b16-t4096", batch=3, s_q=2, ctx=("list", [2, 129, 1000]))
    inp = make_inputs(cfg, seed=35)
    ap = make_append_inputs(cfg, seed=35)
    d, _ = check_append(inp, ap)
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    pool = ref_append.cache_append(inp.pool_f32(), inp.page_table, inp.ctx_lens, ap.h,
                                   ap.w_dkv, ap.w_kr, cfg.s_q, cfg.page_size, BASE)
    # the decode reads the bf16 rows the GPU wrote; the oracle's rows are rounded the same
    # way so both sides attend over the same cache
    from workloads.gen import bf16_round
    pool = bf16_round(pool.astype(np.float32))
    out, lse = ref.mla_decode_naive(inp.q, pool, inp.page_table, inp.ctx_lens, inp.w_uk,
                                    inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
    fin = np.isfinite(out)
    e = float(np.max(np.abs(d.out.cpu().numpy()[fin] - out[fin])) / np.max(np.abs(out[fin])))
    announce(f"  decode after append rel_err {e:.3e}")
    assert e <= TOL["bf16"]
    assert np.array_equal(np.isneginf(d.lse.cpu().numpy()), np.isneginf(lse))


def test_decode_loop_across_page_boundaries():
    """Four decode steps in a row, each appending one new token per sequence and then
    decoding over the grown cache, with new tokens that cross page boundaries (positions
    63 -> 66 and 127 -> 130) and one long sequence; every step against the oracle's decode over the
    oracle's cache after the same appends (rows rounded to bf16 as the GPU stores them)."""
    from workloads.gen import bf16_round
    final = [67, 131, 504]
    cfg = get_config("dsv2-b16-t4096", batch=3, s_q=1, ctx=("list", final), n_splits=3)
    inp = make_inputs(cfg, seed=37)
    ap = make_append_inputs(cfg, seed=37)
    d = DeviceInputs(inp)
    w_dkv, w_kr = to_dev(ap.w_dkv, cfg.dtype), to_dev(ap.w_kr, cfg.dtype)
    pool_ref = inp.pool_f32().astype(np.float64)
    rng = np.random.default_rng(np.random.SeedSequence([37, 9]))
    for k in range(4):
        T = np.array([f - 3 + k for f in final], dtype=np.int32)
        announce(f"case decode loop step {k}: ctx={list(T)}")
        d.ctx_lens.copy_(torch.from_numpy(T))
        h = bf16_round(rng.standard_normal((cfg.batch, cfg.s_q, ap.d_model)).astype(np.float32))
        mla.mla_cache_append(d.shape, ap.d_model, BASE, to_dev(h, cfg.dtype), w_dkv, w_kr,
                             d.page_table, d.ctx_lens, d.pool)
        mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                            d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
        torch.cuda.synchronize()
        pool_ref = ref_append.cache_append(pool_ref, inp.page_table, T, h, ap.w_dkv, ap.w_kr,
                                           cfg.s_q, cfg.page_size, BASE)
        pool_ref = bf16_round(pool_ref.astype(np.float32)).astype(np.float64)
        out, lse = ref.mla_decode_naive(inp.q, pool_ref, inp.page_table, T, inp.w_uk,
                                        inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
        e = float(np.max(np.abs(d.out.cpu().numpy() - out)) / np.max(np.abs(out)))
        le = float(np.max(np.abs(d.lse.cpu().numpy() - lse)))
        announce(f"  step {k}: out rel_err {e:.3e}, lse max abs {le:.3e}")
        assert e <= TOL["bf16"] and le <= 1e-2
