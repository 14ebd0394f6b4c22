"""GPU parity: every C-ABI entry point against the float64 CPU oracle (needs gfx950).

Error measure (as the tolerances are stated): rel_err = max |gpu - oracle| / max |oracle|
over the compared tensor.  Bars: 1e-4 for fp32 workloads, 2e-2 for bf16 cache / fp32
accumulate workloads; log-sum-exps also meet an absolute bound (LSE_ABS), and the worst
per-row relative error is logged beside every comparison as a diagnostic.  Small cases compare every output; full-size workloads compare
sampled (sequence, head) rows that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_02_amd as mla
from oracle import mla as ref
from workloads import Config, get_config, make_inputs
from workloads.device import DeviceInputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
# Absolute bound on every log-sum-exp (natural-log units), beside the relative bar: lse is
# about 5-12 here, so the relative bar alone would admit errors of a tenth of a nat and
# more.  1e-2 nats is a 1 % error in a softmax normaliser and about 4x the largest bf16
# error measured on these cases (2.7e-3, a partial over a few tokens; q_abs and P are
# rounded to bf16 for the matrix cores); fp32 measured 1.6e-6 and does no such rounding.
LSE_ABS = {"f32": 1e-5, "bf16": 1e-2}


def rel_err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), "-inf pattern differs"
    assert np.all(np.isfinite(got[fin])), "non-finite values where the oracle is finite"
    return float(np.max(np.abs(got[fin] - want[fin])) / np.max(np.abs(want[fin])))


def row_err(got, want):
    """Diagnostic: the worst per-row relative error, a row being one (sequence, query row,
    head) output vector: max over rows of max |gpu - oracle| / max |oracle| within the row.
    Returns (error, row index in the flattened leading dimensions)."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
    want = np.asarray(want, np.float64).reshape(-1, np.shape(want)[-1])
    rows = np.all(np.isfinite(want), axis=1)
    scale = np.max(np.abs(want[rows]), axis=1)
    err = np.max(np.abs(got[rows] - want[rows]), axis=1) / np.where(scale > 0, scale, 1.0)
    i = int(np.argmax(err))
    return float(err[i]), int(np.flatnonzero(rows)[i])


def lse_abs_err(got, want):
    """max |gpu - oracle| over the finite log-sum-exps (the -inf pattern must agree)."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), "-inf pattern differs"
    return float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0


def announce(msg):
    print(msg, flush=True)


def absorbed_step(d, sync=True):
    c = d.inp.cfg
    op = d.o_part_view(c.d_c)
    mla.mla_absorb_q(d.shape, d.q, d.w_uk, d.q_abs)
    mla.mla_decode_absorbed(d.shape, d.q_abs, d.pool, d.page_table, d.ctx_lens, op,
                            d.lse_part)
    mla.mla_splitkv_combine(d.shape, c.d_c, op, d.lse_part, d.o_lat, d.lse)
    mla.mla_out_uv(d.shape, d.o_lat, d.w_uv, d.out)
    if sync:
        torch.cuda.synchronize()
    return op


def small(name="dsv2-b16-t4096", **kw):
    return get_config(name, **kw)


def check_absorbed_all_steps(inp, S=None, split_tokens=None):
    """Compare a1..a4 one by one against the oracle's plain steps; returns the errors."""
    c = inp.cfg
    announce(f"case {c.name} B={c.batch} s_q={c.s_q} H={c.n_heads}/{c.n_wheads} "
             f"ctx={list(inp.ctx_lens)[:6]} S={S or c.n_splits} L={split_tokens}")
    d = DeviceInputs(inp, n_splits=S, split_tokens=split_tokens)
    op = absorbed_step(d)
    tol = TOL[c.dtype]
    sh = d.shape
    pool = inp.pool_view()
    q_abs = ref.absorb_query(inp.q, inp.w_uk, c.d_nope)
    e1 = rel_err(d.q_abs.float().cpu().numpy(), q_abs)
    o_p, l_p = ref.absorbed_split_partials(q_abs, pool, inp.page_table, inp.ctx_lens,
                                           sh.n_splits, c.scale, c.page_size, c.d_c,
                                           sh.split_tokens)
    e2 = rel_err(op.cpu().numpy(), o_p)
    e2l = rel_err(d.lse_part.cpu().numpy(), l_p)
    o_l, lse = ref.combine_splits(o_p, l_p)
    e3 = rel_err(d.o_lat.cpu().numpy(), o_l)
    out, lse_n = ref.mla_decode_naive(inp.q, pool, inp.page_table, inp.ctx_lens, inp.w_uk,
                                      inp.w_uv, c.scale, c.page_size, c.d_c)
    e4 = rel_err(d.out.cpu().numpy(), out)
    e4l = rel_err(d.lse.cpu().numpy(), lse_n)
    errs = dict(absorb=e1, partial_o=e2, partial_lse=e2l, combine=e3, out=e4, lse=e4l)
    worst_row, at = row_err(d.out.cpu().numpy(), out)
    lse_abs = max(lse_abs_err(d.lse_part.cpu().numpy(), l_p),
                  lse_abs_err(d.lse.cpu().numpy(), lse_n))
    announce(f"  errors {errs} kind={mla.mla_decode_kernel_kind(sh)}; worst row "
             f"{worst_row:.3e} (row {at}), lse max abs {lse_abs:.3e}")
    for k, v in errs.items():
        assert v <= tol, f"{k}: {v} > {tol}"
    assert lse_abs <= LSE_ABS[c.dtype], f"lse abs {lse_abs} > {LSE_ABS[c.dtype]}"
    return errs


# ------------------------------------------------------------------ tiny fp32

@pytest.mark.parametrize("S,L", [(1, 0), (4, 0), (2, 128), (7, 0)])
def test_tiny_f32_all_steps(S, L):
    inp = make_inputs(get_config("tiny-f32"))
    check_absorbed_all_steps(inp, S=S, split_tokens=L)


def test_tiny_f32_ragged_mtp_and_empty_rows():
    cfg = get_config("tiny-f32", batch=4, s_q=2, ctx=("list", [1, 2, 65, 255]))
    check_absorbed_all_steps(make_inputs(cfg, seed=1), S=5)


def test_tiny_f32_zero_length_sequences():
    """Sequences with no cached token at all (every chunk empty): out = 0, lse = -inf."""
    cfg = get_config("tiny-f32", batch=4, s_q=2, ctx=("list", [0, 65, 0, 30]))
    check_absorbed_all_steps(make_inputs(cfg, seed=5), S=3)


def test_tiny_f32_step_entry_point_matches_steps():
    inp = make_inputs(get_config("tiny-f32"))
    d = DeviceInputs(inp)
    absorbed_step(d)
    out1, lse1 = d.out.clone(), d.lse.clone()
    d.out.fill_(7.0)
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    assert torch.equal(out1, d.out) and torch.equal(lse1, d.lse)


# ------------------------------------------------------------- bf16, small sizes

@pytest.mark.parametrize("name,s_q,ctx,S", [
    ("dsv2-b16-t4096", 1, [4096, 577, 64, 33], 32),
    ("dsv2-b16-t4096", 2, [1 + (97 * i) % 300 for i in range(20)], 3),
    ("dsv2-b16-t4096", 2, [2 + (53 * i) % 400 for i in range(33)], 4),
    ("dsv2-b16-t4096", 2, [1280 + 37 * i for i in range(33)], 20),
    ("dsv2-b16-t4096", 2, [0 if i % 5 == 0 else 1 + (71 * i) % 500 for i in range(33)], 6),
    ("dsv2-b16-t4096", 1, [4096 - 61 * i for i in range(16)], 8),
    ("dsv2-b16-t4096", 1, [300 + 29 * i for i in range(32)], 6),
    ("dsv2-b16-t4096", 1, [5000, 64], 64),
    ("dsv2-b16-t4096", 2, [1, 2, 130], 1),
    ("dsv2-b16-t4096", 1, [0, 577, 0, 64], 4),
    ("gqla-b32-t8192", 2, [700, 64, 1999], 5),
    ("gqla-b32-t8192", 1, [0, 700, 0], 3),
    ("gqla-shard-b32-t65536", 1, [700, 64, 1999], 3),
])
def test_bf16_step_entry_point_matches_steps(name, s_q, ctx, S):
    """At bf16 with d_c 512 and d_v 128 the step entry point merges the splits and
    up-projects in one kernel; its outputs must equal those of the separate entry points
    bit for bit (20 and 33 sequences at s_q = 2 give two and three query blocks of 32, the
    last ragged, on the fused kernel with whole heads per workgroup, which loads the
    partials 8 splits at a time, so 20 splits take three batches, and empty sequences
    among them give rows whose chunks are all empty; 4, 16 and 32 queries on the
    one with half heads, which merges four queries a pass);
    s_q = 2 over one token gives rows with no visible token, and sequences of length 0 give
    whole sequences of empty chunks; the 32- and 4-head shapes have too few workgroups for
    the fused kernel and take the separate kernels inside the step), and match the oracle."""
    cfg = get_config(name, batch=len(ctx), s_q=s_q, ctx=("list", ctx))
    inp = make_inputs(cfg, seed=21)
    announce(f"case {name} s_q={s_q} ctx={ctx[:6]} S={S}")
    d = DeviceInputs(inp, n_splits=S)
    absorbed_step(d)
    want = [t.clone() for t in (d.out, d.lse, d.o_lat)]
    for t in (d.out, d.lse, d.o_lat):
        t.fill_(7.0)
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    for got, exp, what in zip((d.out, d.lse, d.o_lat), want, ("out", "lse", "o_lat")):
        assert torch.equal(got, exp), f"{what} differs from the separate entry points"
    c = inp.cfg
    out, lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                    inp.w_uk, inp.w_uv, c.scale, c.page_size, c.d_c)
    assert rel_err(d.out.cpu().numpy(), out) <= TOL["bf16"]
    assert rel_err(d.lse.cpu().numpy(), lse) <= TOL["bf16"]



@pytest.mark.parametrize("H,Hw,s_q", [(96, 96, 1), (160, 160, 1), (64, 64, 3), (32, 8, 3)])
def test_odd_row_block_counts(H, Hw, s_q):
    """Query rows per sequence (s_q x H) that give the matrix-core kernels an odd number of
    row blocks, so the workgroup-to-(chunk, row block) mapping and the output row offsets
    are exercised beyond the two blocks of the 128-head shapes: 96 and 160 rows (32-row
    blocks, 3 and 5), 192 rows (64-row blocks, 3) and GQLA-style grouped heads at s_q = 3
    (96 rows, 4 query heads per weight head).  Every step against the oracle, then the step
    entry point against the separate entry points bit for bit."""
    cfg = small(n_heads=H, n_wheads=Hw, s_q=s_q, batch=3, ctx=("list", [700, 130, 197]))
    inp = make_inputs(cfg, seed=31)
    check_absorbed_all_steps(inp, S=4)
    d = DeviceInputs(inp, n_splits=4)
    absorbed_step(d)
    want = [t.clone() for t in (d.out, d.lse, d.o_lat)]
    for t in (d.out, d.lse, d.o_lat):
        t.fill_(7.0)
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    for got, exp, what in zip((d.out, d.lse, d.o_lat), want, ("out", "lse", "o_lat")):
        assert torch.equal(got, exp), f"{what} differs from the separate entry points"


@pytest.mark.parametrize("name,batch,s_q", [
    ("dsv2-b16-t4096", 3, 1), ("dsv2-b16-t4096", 12, 1), ("dsv2-b16-t4096", 17, 1),
    ("dsv2-b16-t4096", 33, 1), ("dsv2-b16-t4096", 50, 2), ("dsv2-b16-t4096", 65, 2),
    ("gqla-b32-t8192", 20, 1), ("dsv2-b16-t4096", 1, 1), ("dsv2-b16-t4096", 8, 1),
    ("gqla-b32-t8192", 5, 1)])
def test_absorb_query_counts(name, batch, s_q):
    """a1 alone at query counts that exercise both kernels: the streaming kernel's 4- and
    8-query blocks (1, 3, 5, 8, 12: one block partly filled or full, or a full one and a
    partial one), and matrix-core workgroups of 1, 2 or 4 blocks of 32 queries, partly
    filled (17, 33, 100) or more than one along the queries (130), at 128 heads and at
    GQLA's grouped heads (32 heads over 8 weight heads)."""
    cfg = small(name, batch=batch, s_q=s_q, ctx=("list", [64 + 7 * b for b in range(batch)]))
    inp = make_inputs(cfg, seed=21)
    announce(f"case absorb {cfg.name} NQ={batch * s_q} H={cfg.n_heads}/{cfg.n_wheads}")
    d = DeviceInputs(inp)
    d.q_abs.fill_(float("nan"))
    mla.mla_absorb_q(d.shape, d.q, d.w_uk, d.q_abs)
    torch.cuda.synchronize()
    want = ref.absorb_query(inp.q, inp.w_uk, cfg.d_nope)
    assert rel_err(d.q_abs.float().cpu().numpy(), want) <= TOL["bf16"]


@pytest.mark.parametrize("S,L,ctx", [
    (1, 0, [1000, 64]), (4, 0, [4096, 577]), (3, 128, [300, 129]), (8, 0, [33, 1])])
def test_bf16_mla_small_all_steps(S, L, ctx):
    cfg = small(batch=len(ctx), ctx=("list", ctx))
    check_absorbed_all_steps(make_inputs(cfg, seed=2), S=S, split_tokens=L)


@pytest.mark.parametrize("ctx", [[2, 3, 130, 1025], [64, 65, 127, 2000]])
def test_bf16_mtp_small_all_steps(ctx):
    cfg = small(batch=len(ctx), s_q=2, ctx=("list", ctx))
    check_absorbed_all_steps(make_inputs(cfg, seed=3), S=3)


@pytest.mark.parametrize("S,ctx", [(9, [4096, 4096]), (3, [4096, 1, 64])])
def test_chunks_past_the_last_page(S, ctx):
    """Page tables exactly as long as the longest sequence, with trailing empty chunks
    (their first token index points one page past the table row)."""
    cfg = small(batch=len(ctx), ctx=("list", ctx))
    check_absorbed_all_steps(make_inputs(cfg, seed=13, max_pages=max(ctx) // 64), S=S)


@pytest.mark.parametrize("s_q,S,L", [(1, 5, 0), (2, 3, 0), (1, 11, 192)])
def test_bf16_gqla_absorbed_shapes(s_q, S, L):
    """32 query heads in 8 groups: 32-row workgroups at s_q = 1, 64-row ones at s_q = 2."""
    cfg = get_config("gqla-b32-t8192", batch=3, s_q=s_q, ctx=("list", [700, 64, 1999]))
    check_absorbed_all_steps(make_inputs(cfg, seed=14), S=S, split_tokens=L)


def test_bf16_gqla_absorbed_small():
    cfg = get_config("gqla-b32-t8192", batch=3, ctx=("list", [500, 64, 1999]))
    check_absorbed_all_steps(make_inputs(cfg, seed=4), S=2)


def test_identity_vs_permuted_page_table_bitwise():
    cfg = small(batch=3, ctx=("list", [700, 300, 1100]))
    a = make_inputs(cfg, seed=5)
    d = DeviceInputs(a)
    absorbed_step(d)
    out_perm = d.out.clone()
    # the same logical content laid out in order
    order = [int(p) for b in range(cfg.batch) for p in a.page_table[b] if p >= 0]
    b_in = make_inputs(cfg, seed=5)
    b_in.pool = a.pool[order]
    tbl = np.full_like(a.page_table, -1)
    off = 0
    for b in range(cfg.batch):
        n = int(np.sum(a.page_table[b] >= 0))
        tbl[b, :n] = np.arange(off, off + n)
        off += n
    b_in.page_table = tbl
    d2 = DeviceInputs(b_in)
    absorbed_step(d2)
    assert torch.equal(out_perm, d2.out)


def test_pages_above_4gib_bitwise():
    """The same sequences with their pages moved past byte 4 GiB of a ~5.9 GB pool (page
    ids from 80000, 73,728 bytes each) give bitwise the same step outputs: page and row
    offsets are formed in 64 bits.  Every page below the moved ones is NaN."""
    from workloads.device import shape_of
    cfg = small(batch=2, ctx=("list", [700, 1100]))
    a = make_inputs(cfg, seed=6)
    d = DeviceInputs(a)
    absorbed_step(d)
    want, want_lse = d.out.clone(), d.lse.clone()
    shift = 80000
    big = torch.full((shift + a.num_pages, cfg.page_size, cfg.D), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    big[shift:] = d.pool
    sh = shape_of(a)
    sh.num_pages = shift + a.num_pages
    table = torch.where(d.page_table >= 0, d.page_table + shift, d.page_table)
    announce(f"case pages above 4 GiB: pool {big.numel() * 2 / 2**30:.2f} GiB")
    op = d.o_part_view(cfg.d_c)
    mla.mla_absorb_q(sh, d.q, d.w_uk, d.q_abs)
    mla.mla_decode_absorbed(sh, d.q_abs, big, table, d.ctx_lens, op, d.lse_part)
    mla.mla_splitkv_combine(sh, cfg.d_c, op, d.lse_part, d.o_lat, d.lse)
    mla.mla_out_uv(sh, d.o_lat, d.w_uv, d.out)
    torch.cuda.synchronize()
    assert torch.equal(want, d.out) and torch.equal(want_lse, d.lse)
    del big
    torch.cuda.empty_cache()


def test_deterministic_over_repeats():
    cfg = small(batch=2, ctx=("list", [1500, 900]))
    d = DeviceInputs(make_inputs(cfg, seed=6))
    absorbed_step(d)
    first = d.out.clone()
    for _ in range(5):
        absorbed_step(d)
        assert torch.equal(first, d.out)


def test_negative_control_uniform_attention_fails():
    """Uniform attention (q = 0) is far from the real output: the bar has teeth."""
    cfg = small(batch=2, ctx=("list", [1024, 512]))
    inp = make_inputs(cfg, seed=7)
    out, _ = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                  inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c,
                                  heads=[0, 5, 64])
    inp.q = np.zeros_like(inp.q)
    d = DeviceInputs(inp)
    absorbed_step(d)
    err = rel_err(d.out.cpu().numpy()[:, :, [0, 5, 64]], out[:, :, [0, 5, 64]])
    announce(f"  negative control rel err {err:.3f}")
    assert err > 10 * TOL["bf16"]


def test_nan_poisoned_pages_never_read():
    cfg = small(batch=2, ctx=("list", [100, 65]))
    inp = make_inputs(cfg, seed=8, extra_pages=3, max_pages=6)
    d = DeviceInputs(inp)
    absorbed_step(d)
    assert torch.isfinite(d.out).all() and torch.isfinite(d.o_lat).all()


# ----------------------------------------------------------------- GQA path

def gqa_step(d, k, v, kr, sync=True):
    c = d.inp.cfg
    op = d.o_part_view(c.d_v)
    mla.gqla_decode_gqa(d.shape, d.q, k, v, kr, d.page_table, d.ctx_lens, op, d.lse_part)
    mla.mla_splitkv_combine(d.shape, c.d_v, op, d.lse_part, d.out, d.lse)
    if sync:
        torch.cuda.synchronize()
    return op


def expanded_pools(d):
    c = d.inp.cfg
    wdt = torch.bfloat16 if d.inp.is_bf16 else torch.float32
    n = d.inp.num_pages
    k = torch.empty(n, c.page_size, c.n_wheads, c.d_nope, dtype=wdt, device="cuda")
    v = torch.empty(n, c.page_size, c.n_wheads, c.d_v, dtype=wdt, device="cuda")
    kr = torch.empty(n, c.page_size, c.d_rope, dtype=wdt, device="cuda")
    return k, v, kr


@pytest.mark.parametrize("dtype,ctx,S", [("f32", [300, 64, 1], 3), ("bf16", [1000, 129], 2),
                                         ("bf16", [4096, 2000], 4),
                                         ("bf16", [1, 33, 64, 65, 95], 8),
                                         ("bf16", [0, 700, 0, 65], 3),
                                         ("shard", [1, 700, 2049], 5),
                                         ("mtp", [1, 2, 130, 1999], 3)])
def test_gqla_expand_and_gqa_path(dtype, ctx, S):
    if dtype == "f32":
        cfg = Config("gqla-tiny-f32", "f32", len(ctx), 1, 8, 2, 64, 16, 32, 32,
                     ("list", ctx), S)
    elif dtype == "shard":   # one group and its 4 heads
        cfg = get_config("gqla-shard-b32-t65536", batch=len(ctx), ctx=("list", ctx),
                         n_splits=S)
    elif dtype == "mtp":     # s_q = 2
        cfg = get_config("gqla-mtp-b32-t65536", batch=len(ctx), ctx=("list", ctx),
                         n_splits=S)
    else:
        cfg = get_config("gqla-b32-t8192", batch=len(ctx), ctx=("list", ctx), n_splits=S)
    inp = make_inputs(cfg, seed=9)
    announce(f"case gqa {dtype} ctx={ctx} S={S}")
    d = DeviceInputs(inp)
    k, v, kr = expanded_pools(d)
    mla.gqla_expand_cache(d.shape, d.pool, d.w_uk, d.w_uv, k, v, kr)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    # a6 against the oracle's expansion (rows past the context are NaN on both sides)
    ek, ev, ekr = ref.expand_cache(inp.pool_f32(), inp.w_uk, inp.w_uv, cfg.d_c)
    fin = np.isfinite(ek)
    gk = k.float().cpu().numpy()
    assert np.array_equal(np.isfinite(gk), fin)
    assert rel_err(gk[fin], ek[fin]) <= tol
    gv = v.float().cpu().numpy()
    assert rel_err(gv[np.isfinite(ev)], ev[np.isfinite(ev)]) <= tol
    assert np.array_equal(kr.float().cpu().numpy(), ekr.astype(np.float32), equal_nan=True)
    # a5 + a3 against the plain definition (naive over the latent cache)
    gqa_step(d, k, v, kr)
    out, lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                    inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
    e_out = rel_err(d.out.cpu().numpy(), out)
    e_lse = rel_err(d.lse.cpu().numpy(), lse)
    worst_row, at = row_err(d.out.cpu().numpy(), out)
    lse_abs = lse_abs_err(d.lse.cpu().numpy(), lse)
    announce(f"  gqa errors out={e_out:.3e} lse={e_lse:.3e} "
             f"kind={mla.gqla_decode_kernel_kind(d.shape)}; worst row {worst_row:.3e} "
             f"(row {at}), lse max abs {lse_abs:.3e}")
    assert e_out <= tol and e_lse <= tol
    assert lse_abs <= LSE_ABS[cfg.dtype]


@pytest.mark.parametrize("H,G,s_q,kind", [(16, 16, 1, 1), (32, 16, 1, 1), (64, 4, 1, 1),
                                           (24, 3, 2, 1), (40, 5, 1, 1), (64, 2, 1, 0)])
def test_gqa_path_group_counts(H, G, s_q, kind):
    """The GQA path (a6 then a5 + a3) at other group shapes: one, two and sixteen query
    rows per group (16 is the matrix-core kernel's limit), odd group counts (3 and 5, which
    also give the expansion kernel page ranges that are not a power of two), and 32 rows per
    group, which takes the generic kernel; against the oracle's expansion and the plain
    definition."""
    cfg = get_config("gqla-b32-t8192", n_heads=H, n_wheads=G, s_q=s_q, batch=3,
                     ctx=("list", [700, 130, 65]), n_splits=3)
    inp = make_inputs(cfg, seed=41)
    announce(f"case gqa groups H={H} G={G} s_q={s_q}")
    d = DeviceInputs(inp)
    assert mla.gqla_decode_kernel_kind(d.shape) == kind
    k, v, kr = expanded_pools(d)
    mla.gqla_expand_cache(d.shape, d.pool, d.w_uk, d.w_uv, k, v, kr)
    torch.cuda.synchronize()
    ek, ev, ekr = ref.expand_cache(inp.pool_f32(), inp.w_uk, inp.w_uv, cfg.d_c)
    fin = np.isfinite(ek)
    gk = k.float().cpu().numpy()
    assert np.array_equal(np.isfinite(gk), fin)
    assert rel_err(gk[fin], ek[fin]) <= TOL["bf16"]
    gv = v.float().cpu().numpy()
    assert rel_err(gv[np.isfinite(ev)], ev[np.isfinite(ev)]) <= TOL["bf16"]
    gqa_step(d, k, v, kr)
    out, lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                    inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
    e_out, e_lse = rel_err(d.out.cpu().numpy(), out), rel_err(d.lse.cpu().numpy(), lse)
    announce(f"  gqa errors out={e_out:.3e} lse={e_lse:.3e}")
    assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]
    assert lse_abs_err(d.lse.cpu().numpy(), lse) <= LSE_ABS["bf16"]


@pytest.mark.parametrize("d_rope", [0, 32, 64])
def test_gqla_expand_rope_widths(d_rope):
    """The matrix-core expansion with a RoPE key narrower than 64 (its lanes past the key's
    width re-read the last chunk and store nothing) and with none at all; 67 pages, so page
    ranges of three pages (six half pages: the three-slot ring wraps), a shorter last range
    and empty ranges past the end.  K and V against the oracle's expansion, the keys copied
    exactly."""
    cfg = get_config("gqla-b32-t8192", d_rope=d_rope, batch=3,
                     ctx=("list", [3000, 1100, 65]), n_splits=3)
    inp = make_inputs(cfg, seed=43)
    announce(f"case expand d_rope={d_rope} pages={inp.num_pages}")
    d = DeviceInputs(inp)
    k, v, kr = expanded_pools(d)
    mla.gqla_expand_cache(d.shape, d.pool, d.w_uk, d.w_uv, k, v, kr)
    torch.cuda.synchronize()
    ek, ev, ekr = ref.expand_cache(inp.pool_f32(), inp.w_uk, inp.w_uv, cfg.d_c)
    fin = np.isfinite(ek)
    gk = k.float().cpu().numpy()
    assert np.array_equal(np.isfinite(gk), fin)
    assert rel_err(gk[fin], ek[fin]) <= TOL["bf16"]
    gv = v.float().cpu().numpy()
    assert np.array_equal(np.isfinite(gv), np.isfinite(ev))
    assert rel_err(gv[np.isfinite(ev)], ev[np.isfinite(ev)]) <= TOL["bf16"]
    assert np.array_equal(kr.float().cpu().numpy(), ekr.astype(np.float32), equal_nan=True)


def test_gqa_path_uses_matrix_cores_at_gqla_shapes():
    for sq in (1, 2):
        cfg = get_config("gqla-b32-t8192", s_q=sq)
        d = DeviceInputs(make_inputs(cfg.with_(batch=1, ctx=("list", [64]))))
        assert mla.gqla_decode_kernel_kind(d.shape) == 1


def test_gqa_decode_on_oracle_expanded_cache():
    """a5 alone: fed the oracle's expansion rounded to bf16, compared with the oracle's
    GQA-path partials over that same cache."""
    from workloads.gen import bf16_round
    cfg = get_config("gqla-b32-t8192", batch=2, s_q=2, ctx=("list", [777, 130]), n_splits=3)
    inp = make_inputs(cfg, seed=10)
    ek, ev, ekr = ref.expand_cache(inp.pool_f32(), inp.w_uk, inp.w_uv, cfg.d_c)
    k_np, v_np, kr_np = (bf16_round(x.astype(np.float32)) for x in (ek, ev, ekr))
    d = DeviceInputs(inp)
    k = torch.from_numpy(k_np).cuda().to(torch.bfloat16)
    v = torch.from_numpy(v_np).cuda().to(torch.bfloat16)
    kr = torch.from_numpy(kr_np).cuda().to(torch.bfloat16)
    op = gqa_step(d, k, v, kr)
    o_p, l_p = ref.gqa_split_partials(inp.q, k_np, v_np, kr_np, inp.page_table, inp.ctx_lens,
                                      3, cfg.scale, cfg.page_size)
    assert rel_err(op.cpu().numpy(), o_p) <= TOL["bf16"]
    assert rel_err(d.lse_part.cpu().numpy(), l_p) <= TOL["bf16"]


# -------------------------------------------------- full-size workloads (sampled)

def sampled_full_check(cfg, batches, heads, S=None, split_tokens=None):
    inp = make_inputs(cfg)
    announce(f"case full {cfg.name} tokens={inp.total_tokens} S={S or cfg.n_splits}")
    d = DeviceInputs(inp, n_splits=S, split_tokens=split_tokens)
    # the step entry point, as the benchmark times it
    mla.mla_decode_step(d.shape, d.q, d.w_uk, d.w_uv, d.pool, d.page_table, d.ctx_lens,
                        d.q_abs, d.o_part, d.lse_part, d.o_lat, d.out, d.lse)
    torch.cuda.synchronize()
    got = d.out.cpu().numpy()
    got_lse = d.lse.cpu().numpy()
    del d
    torch.cuda.empty_cache()
    want, lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                     inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c,
                                     batches=batches, heads=heads)
    sel = np.ix_(batches, range(cfg.s_q), heads)
    e = rel_err(got[sel], want[sel])
    el = rel_err(got_lse[sel], lse[sel])
    worst_row, at = row_err(got[sel], want[sel])
    lse_abs = lse_abs_err(got_lse[sel], lse[sel])
    announce(f"  sampled errors out={e:.3e} lse={el:.3e} "
             f"(rows {len(batches)}x{cfg.s_q}x{len(heads)}); worst row {worst_row:.3e} "
             f"(row {at}), lse max abs {lse_abs:.3e}")
    assert e <= TOL[cfg.dtype] and el <= TOL[cfg.dtype]
    assert lse_abs <= LSE_ABS[cfg.dtype]


def test_full_dsv2_b16_t4096():
    sampled_full_check(get_config("dsv2-b16-t4096"), list(range(16)), [0, 31, 64, 127])


def test_full_long_b4_t131072():
    # ten heads per sequence: rows of both score waves of both 64-row blocks, each block's
    # first and last row
    sampled_full_check(get_config("long-b4-t131072"), [0, 1, 2, 3],
                       [0, 13, 31, 45, 63, 64, 77, 90, 101, 127])


def test_full_gqla_b32_t65536_absorbed():
    sampled_full_check(get_config("gqla-b32-t65536"), [0, 17, 31], list(range(32)))


@pytest.mark.parametrize("name", ["gqla-b32-t8192", "gqla-b32-t16384", "gqla-b32-t32768"])
def test_full_gqla_context_sweep_absorbed(name):
    """The other points of the GQLA context sweep, at full size (32 sequences)."""
    sampled_full_check(get_config(name), [0, 31], [0, 5, 13, 31])


def test_full_mtp_b64_ragged():
    sampled_full_check(get_config("mtp-b64-ragged"), [0, 17, 40, 63], [0, 127, 77])


@pytest.mark.parametrize("name", ["gqla-b32-t65536", "gqla-mtp-b32-t65536",
                                  "gqla-shard-b32-t65536", "gqla-b32-t8192"])
def test_full_gqla_b32_t65536_gqa_path(name):
    """GQA path at its largest size: 32 sequences of 65536 tokens, expanded on the GPU; the
    same at s_q = 2 (two query rows per head, causal), and one rank's share under 8-way
    tensor parallelism over the groups (one group, 4 heads)."""
    cfg = get_config(name)
    inp = make_inputs(cfg)
    announce(f"case full gqa {cfg.name} tokens={inp.total_tokens} S={cfg.n_splits}")
    d = DeviceInputs(inp)
    assert mla.gqla_decode_kernel_kind(d.shape) == 1
    k, v, kr = expanded_pools(d)
    mla.gqla_expand_cache(d.shape, d.pool, d.w_uk, d.w_uv, k, v, kr)
    gqa_step(d, k, v, kr)
    got, got_lse = d.out.cpu().numpy(), d.lse.cpu().numpy()
    del d, k, v, kr
    torch.cuda.empty_cache()
    batches, heads = [0, 13, 31], list(range(cfg.n_heads))
    want, lse = ref.mla_decode_naive(inp.q, inp.pool_view(), inp.page_table, inp.ctx_lens,
                                     inp.w_uk, inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c,
                                     batches=batches, heads=heads)
    sel = np.ix_(batches, range(cfg.s_q), heads)
    e, el = rel_err(got[sel], want[sel]), rel_err(got_lse[sel], lse[sel])
    worst_row, at = row_err(got[sel], want[sel])
    lse_abs = lse_abs_err(got_lse[sel], lse[sel])
    announce(f"  sampled errors out={e:.3e} lse={el:.3e}; worst row {worst_row:.3e} "
             f"(row {at}), lse max abs {lse_abs:.3e}")
    assert e <= TOL["bf16"] and el <= TOL["bf16"]
    assert lse_abs <= LSE_ABS["bf16"]


# ------------------------------------ reference moves (online-softmax rescale path)

@pytest.mark.parametrize("slack", ["0", "0.25"])
def test_reference_moves_rescale_path(slack, monkeypatch):
    """With no slack the per-row reference moves whenever a tile raises the maximum, so
    the matrix-core kernel rescales running sums and accumulators many times; the result
    must not change."""
    monkeypatch.setenv("MLA_DECODE_REF_SLACK", slack)
    cfg = small(batch=3, s_q=2, ctx=("list", [1500, 700, 65]))
    errs = check_absorbed_all_steps(make_inputs(cfg, seed=12), S=3)
    assert errs["out"] <= TOL["bf16"]


@pytest.mark.parametrize("slack", ["0", "0.25"])
def test_reference_moves_rescale_path_32_row_blocks(slack, monkeypatch):
    """The rescale path of the 32-row-block kernel (GQLA's absorbed shape, 32 heads): with no
    slack every raised maximum rescales; the result must not change."""
    monkeypatch.setenv("MLA_DECODE_REF_SLACK", slack)
    cfg = small("gqla-b32-t8192", batch=3, s_q=1, ctx=("list", [1500, 700, 65]))
    assert cfg.s_q * cfg.n_heads == 32          # one block of 32 query rows per sequence
    errs = check_absorbed_all_steps(make_inputs(cfg, seed=14), S=3)
    assert errs["out"] <= TOL["bf16"]


def test_growing_scores_move_the_reference_by_large_steps():
    """Scores that climb by ~38 log2 units per tile move the reference at the default
    slack on every tile; the result must still match the oracle."""
    from workloads.gen import growing_score_inputs
    cfg = small(batch=2, ctx=("list", [2000, 900]), n_splits=3)
    check_absorbed_all_steps(growing_score_inputs(cfg, period_tokens=1 << 20, seed=13))


@pytest.mark.parametrize("name", ["long-b4-t131072", "gqla-b32-t8192"])
def test_growing_scores_full_chunks(name):
    """A reference move on every tile of every chunk (scores restart their climb at each
    chunk start), for both ring kernels, on shortened contexts; against the oracle."""
    from workloads.gen import growing_score_inputs
    kw = dict(batch=2, ctx=("list", [8192, 5000])) if name.startswith("long") else \
        dict(batch=2, ctx=("list", [4096, 1000]))
    cfg = small(name, **kw)
    check_absorbed_all_steps(growing_score_inputs(cfg, period_tokens=8192 // cfg.n_splits
                                                  if name.startswith("long") else 4096 // 8,
                                                  seed=15))
