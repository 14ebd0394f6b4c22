"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties ``oracle.mla`` to an independent fact: the pure-Python brute force, a
library routine (torch's scaled-dot-product attention) on special cases, closed forms,
the equivalences the pages state (absorbed = expanded by associativity; MQA-absorb path
= GQA path over the same GQLA weights), structural invariants and the printed cache
sizes.  The last group plants mistakes in the oracle and checks that a pin catches them.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla, brute
from workloads import Config, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def small_cfg(**kw):
    base = dict(name="t", dtype="f32", batch=2, s_q=1, n_heads=8, n_wheads=8, d_c=64,
                d_rope=16, d_nope=32, d_v=24, ctx=("list", [130, 71]), n_splits=3)
    base.update(kw)
    return Config(**base)


def naive(inp, **kw):
    c = inp.cfg
    return mla.mla_decode_naive(inp.q, inp.pool_f32(), inp.page_table, inp.ctx_lens,
                                inp.w_uk, inp.w_uv, c.scale, c.page_size, c.d_c, **kw)


def rel_err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(b)))


def logical_rows(inp, b):
    """Rows of sequence b in logical order, by walking its pages one at a time."""
    c = inp.cfg
    pool = inp.pool_f32()
    out = []
    for i in range(-(-int(inp.ctx_lens[b]) // c.page_size)):
        out.append(pool[inp.page_table[b, i]])
    return np.concatenate(out, axis=0)[: int(inp.ctx_lens[b])].astype(np.float64)


def sdpa_reference(inp, K_fn, V_fn):
    """Attention through torch's scaled_dot_product_attention (float64, CPU)."""
    c = inp.cfg
    B, s_q, H = c.batch, c.s_q, c.n_heads
    group = H // c.n_wheads
    out = np.zeros((B, s_q, H, c.d_v))
    for b in range(B):
        rows = logical_rows(inp, b)
        T = rows.shape[0]
        mask = torch.zeros(s_q, T, dtype=torch.bool)
        for s in range(s_q):
            mask[s, : T - s_q + s + 1] = True
        for h in range(H):
            K = torch.from_numpy(K_fn(rows, h // group))
            V = torch.from_numpy(V_fn(rows, h // group))
            qq = torch.from_numpy(np.asarray(inp.q[b, :, h], dtype=np.float64))
            o = torch.nn.functional.scaled_dot_product_attention(
                qq[None], K[None], V[None], attn_mask=mask[None], scale=c.scale)
            out[b, :, h] = o[0].numpy()
    return out


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("s_q,Hw", [(1, 4), (2, 2), (2, 1), (1, 1)])
def test_brute_force_matches_naive(s_q, Hw):
    cfg = small_cfg(batch=2, s_q=s_q, n_heads=4, n_wheads=Hw, d_c=6, d_rope=2, d_nope=3,
                    d_v=5, page_size=4, ctx=("list", [9, 5]))
    inp = make_inputs(cfg, seed=3)
    out, _ = naive(inp)
    ref = brute.mla_decode_brute(inp.q.tolist(), inp.pool_f32().tolist(),
                                 inp.page_table.tolist(), inp.ctx_lens.tolist(),
                                 inp.w_uk.tolist(), inp.w_uv.tolist(), cfg.scale,
                                 cfg.page_size, cfg.d_c)
    assert rel_err(out, np.array(ref)) < 1e-12


# ------------------------------------------------------------ library routine

@pytest.mark.parametrize("s_q,Hw", [(1, 8), (2, 2)])
def test_naive_matches_torch_sdpa(s_q, Hw):
    cfg = small_cfg(s_q=s_q, n_wheads=Hw)
    inp = make_inputs(cfg, seed=5)
    out, _ = naive(inp)
    w_uk, w_uv = inp.w_uk.astype(np.float64), inp.w_uv.astype(np.float64)
    ref = sdpa_reference(
        inp,
        lambda rows, w: np.concatenate([rows[:, :cfg.d_c] @ w_uk[w].T, rows[:, cfg.d_c:]], 1),
        lambda rows, w: rows[:, :cfg.d_c] @ w_uv[w].T)
    assert rel_err(out, ref) < 1e-12


def test_identity_weights_reduce_to_textbook_mqa():
    """W_UK = [I | 0], W_UV = [I | 0]: keys are [c[:d_n], k^R] and values c[:d_v]."""
    cfg = small_cfg(s_q=2, n_wheads=1)
    inp = make_inputs(cfg, seed=7)
    inp.w_uk = np.eye(cfg.d_nope, cfg.d_c, dtype=np.float32)[None]
    inp.w_uv = np.eye(cfg.d_v, cfg.d_c, dtype=np.float32)[None]
    out, _ = naive(inp)
    ref = sdpa_reference(
        inp,
        lambda rows, w: np.concatenate([rows[:, :cfg.d_nope], rows[:, cfg.d_c:]], 1),
        lambda rows, w: np.ascontiguousarray(rows[:, :cfg.d_v]))
    assert rel_err(out, ref) < 1e-12


# ------------------------------------------------------------------ closed forms

def test_single_visible_token_closed_form():
    cfg = small_cfg(s_q=2, ctx=("list", [2, 1]), n_wheads=2)
    inp = make_inputs(cfg, seed=11)
    out, lse = naive(inp)
    rows0 = logical_rows(inp, 0)
    w_uk, w_uv = inp.w_uk.astype(np.float64), inp.w_uv.astype(np.float64)
    for h in range(cfg.n_heads):
        w = h // (cfg.n_heads // cfg.n_wheads)
        # row 0 of sequence 0 sees only token 0: output is that token's value exactly
        np.testing.assert_allclose(out[0, 0, h], w_uv[w] @ rows0[0, :cfg.d_c], rtol=1e-13,
                                   atol=1e-14)
        key = np.concatenate([w_uk[w] @ rows0[0, :cfg.d_c], rows0[0, cfg.d_c:]])
        assert abs(lse[0, 0, h] - cfg.scale * key @ inp.q[0, 0, h]) < 1e-12
    # sequence 1 has one token and two query rows: row 0 sees nothing
    assert np.all(out[1, 0] == 0) and np.all(np.isneginf(lse[1, 0]))


def test_zero_query_gives_mean_value():
    cfg = small_cfg(n_wheads=4)
    inp = make_inputs(cfg, seed=13)
    inp.q = np.zeros_like(inp.q)
    out, lse = naive(inp)
    for b in range(cfg.batch):
        rows = logical_rows(inp, b)
        for h in range(cfg.n_heads):
            w = h // 2
            np.testing.assert_allclose(out[b, 0, h], inp.w_uv[w].astype(np.float64)
                                       @ rows[:, :cfg.d_c].mean(0), rtol=1e-12, atol=1e-13)
            assert abs(lse[b, 0, h] - math.log(rows.shape[0])) < 1e-12


def test_softmax_rows_are_distributions():
    cfg = small_cfg(s_q=2, n_wheads=2)
    inp = make_inputs(cfg, seed=17)
    _, lse, probs = naive(inp, return_probs=True)
    for (b, s, h), p in probs.items():
        assert np.all(p >= 0) and abs(p.sum() - 1.0) < 1e-12
        assert len(p) == int(inp.ctx_lens[b]) - cfg.s_q + s + 1


def test_softmax_stats_match_scipy():
    """The oracle's softmax and log-sum-exp equal scipy's independent routines, including
    logits far outside exp's range (the max-shift must be right)."""
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(5)
    for n, spread, shift in [(1, 1.0, 0.0), (7, 3.0, 0.0), (300, 20.0, 900.0),
                             (64, 50.0, -800.0), (1000, 0.6, 0.0)]:
        z = rng.normal(shift, spread, size=n)
        p, lse = mla._softmax_stats(z)
        assert abs(lse - logsumexp(z)) <= 1e-12 * max(1.0, abs(lse))
        np.testing.assert_allclose(p, softmax(z), rtol=1e-12, atol=1e-300)


# ------------------------------------------------------------- the two equivalences

@pytest.mark.parametrize("s_q,Hw,S,split_tokens", [
    (1, 8, 1, 0), (1, 8, 3, 0), (2, 2, 5, 0), (2, 8, 4, 64), (1, 1, 7, 0)])
def test_absorbed_chain_equals_naive(s_q, Hw, S, split_tokens):
    """Absorption reassociates the products (DriveNets page, Decompression Multiplex)."""
    cfg = small_cfg(s_q=s_q, n_wheads=Hw, n_splits=S, split_tokens=split_tokens,
                    ctx=("list", [200, 65]))
    inp = make_inputs(cfg, seed=19)
    out, lse = naive(inp)
    got, got_lse = mla.mla_decode_absorbed_chain(
        inp.q, inp.pool_f32(), inp.page_table, inp.ctx_lens, inp.w_uk, inp.w_uv, cfg.scale,
        cfg.page_size, cfg.d_c, S, split_tokens)
    assert rel_err(got, out) < 1e-12
    np.testing.assert_allclose(got_lse, lse, rtol=1e-12)


@pytest.mark.parametrize("s_q", [1, 2])
def test_gqa_path_equals_mqa_absorb_path(s_q):
    """GQLA: both paths over the same weights give the same attention (GQLA abstract)."""
    cfg = small_cfg(s_q=s_q, n_heads=8, n_wheads=2, n_splits=3, ctx=("list", [150, 64]))
    inp = make_inputs(cfg, seed=23)
    k, v, kr = mla.expand_cache(inp.pool_f32(), inp.w_uk, inp.w_uv, cfg.d_c)
    op, lp = mla.gqa_split_partials(inp.q, k, v, kr, inp.page_table, inp.ctx_lens, 3,
                                    cfg.scale, cfg.page_size)
    o_gqa, lse_gqa = mla.combine_splits(op, lp)
    o_abs, lse_abs = mla.mla_decode_absorbed_chain(
        inp.q, inp.pool_f32(), inp.page_table, inp.ctx_lens, inp.w_uk, inp.w_uv, cfg.scale,
        cfg.page_size, cfg.d_c, 2)
    out, lse = naive(inp)
    assert rel_err(o_gqa, out) < 1e-12 and rel_err(o_abs, o_gqa) < 1e-12
    np.testing.assert_allclose(lse_gqa, lse, rtol=1e-12)


def test_expand_cache_identity_weights():
    cfg = small_cfg(n_wheads=2)
    inp = make_inputs(cfg, seed=29)
    eye_k = np.stack([np.eye(cfg.d_nope, cfg.d_c), 2 * np.eye(cfg.d_nope, cfg.d_c)])
    eye_v = np.stack([np.eye(cfg.d_v, cfg.d_c), -np.eye(cfg.d_v, cfg.d_c)])
    pool = np.nan_to_num(inp.pool_f32().astype(np.float64))
    k, v, kr = mla.expand_cache(pool, eye_k, eye_v, cfg.d_c)
    assert np.array_equal(k[:, :, 0], pool[..., :cfg.d_nope])
    assert np.array_equal(k[:, :, 1], 2 * pool[..., :cfg.d_nope])
    assert np.array_equal(v[:, :, 1], -pool[..., :cfg.d_v])
    assert np.array_equal(kr, pool[..., cfg.d_c:])


# --------------------------------------------------------------------- structure

def test_page_permutation_invariance():
    cfg = small_cfg(n_wheads=4, ctx=("list", [300, 129]))
    inp = make_inputs(cfg, seed=31)
    out, lse = naive(inp)
    # lay the same logical pages out in order (identity table) and decode again
    pool = inp.pool_f32()
    order = [int(p) for b in range(cfg.batch) for p in inp.page_table[b] if p >= 0]
    ident = make_inputs(cfg, seed=31)
    ident.pool = pool[order]
    tbl = np.full_like(inp.page_table, -1)
    off = 0
    for b in range(cfg.batch):
        n = int(np.sum(inp.page_table[b] >= 0))
        tbl[b, :n] = np.arange(off, off + n)
        off += n
    ident.page_table = tbl
    out2, lse2 = naive(ident)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_batch_independence():
    cfg = small_cfg(n_wheads=4)
    inp = make_inputs(cfg, seed=37)
    out, _ = naive(inp)
    inp.q[1] = -inp.q[1]
    for p in inp.page_table[1]:
        if p >= 0:
            inp.pool[p] = inp.pool[p] * 3.0
    out2, _ = naive(inp)
    assert np.array_equal(out[0], out2[0]) and not np.allclose(out[1], out2[1])


def test_split_combine_invariance_with_empty_splits():
    cfg = small_cfg(ctx=("list", [130, 20]), n_splits=6)
    inp = make_inputs(cfg, seed=41)
    q_abs = mla.absorb_query(inp.q, inp.w_uk, cfg.d_nope)
    results = []
    for S, L in [(1, 0), (2, 0), (6, 0), (9, 64), (3, 64)]:
        op, lp = mla.absorbed_split_partials(q_abs, inp.pool_f32(), inp.page_table,
                                             inp.ctx_lens, S, cfg.scale, cfg.page_size,
                                             cfg.d_c, L)
        if S >= 6:   # the 20-token sequence has empty trailing splits
            assert np.all(np.isneginf(lp[1, :, :, 1:])) and np.all(op[1, :, :, 1:] == 0)
        results.append(mla.combine_splits(op, lp))
    for o, l in results[1:]:
        assert rel_err(o, results[0][0]) < 1e-13
        np.testing.assert_allclose(l, results[0][1], rtol=1e-13)


def test_split_ranges_cover_and_align():
    for T in [0, 1, 63, 64, 65, 4096, 131072, 5000]:
        for S in [1, 3, 32]:
            r = mla.split_ranges(T, S, 64)
            assert r[0][0] == 0 and r[-1][1] == T
            assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
            assert all(lo % 64 == 0 for lo, hi in r if hi > lo)


def test_mtp_row0_equals_shorter_decode():
    cfg = small_cfg(s_q=2, n_wheads=2, ctx=("list", [100, 66]))
    inp = make_inputs(cfg, seed=43)
    out, lse = naive(inp)
    inp1 = make_inputs(cfg, seed=43)
    inp1.q = inp.q[:, :1].copy()
    inp1.ctx_lens = inp.ctx_lens - 1
    inp1.cfg = cfg.with_(s_q=1)
    out1, lse1 = naive(inp1)
    assert rel_err(out[:, 0], out1[:, 0]) < 1e-13
    np.testing.assert_allclose(lse[:, 0], lse1[:, 0], rtol=1e-13)


def test_nan_padding_never_reaches_output():
    cfg = small_cfg(s_q=2, n_wheads=2, ctx=("list", [70, 3]), dtype="bf16")
    inp = make_inputs(cfg, seed=47, extra_pages=2)
    assert np.isnan(inp.pool_f32()).any()
    out, lse = naive(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# ---------------------------------------------------------------- printed sizes

def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "cache_sizes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                ident, expr, expected, where = [x.strip() for x in line.split("|", 3)]
                rows.append((ident, expr, float(expected), where))
    return rows


@pytest.mark.parametrize("ident,expr,expected,where", _golden())
def test_printed_cache_sizes(ident, expr, expected, where):
    env = {k: getattr(mla, k) for k in dir(mla) if k.endswith("per_token")}
    assert eval(expr, {"__builtins__": {}}, env) == pytest.approx(expected, rel=1e-15)


def test_gqa_path_cache_is_gqa_level():
    """GQLA abstract: the per-group path keeps GQA-level traffic (2112 vs 2048 scalars)."""
    e = mla.gqla_expanded_cache_scalars_per_token(8, 128, 128, 64)
    g = mla.gqa_cache_scalars_per_token(8, 128)
    assert e == 2112 and 1.0 < e / g < 1.04


# ------------------------------------------------------------- planted mistakes

def _brute_vs_naive_err(seed=3):
    cfg = small_cfg(batch=2, s_q=2, n_heads=4, n_wheads=2, d_c=6, d_rope=2, d_nope=3,
                    d_v=5, page_size=4, ctx=("list", [9, 6]))
    inp = make_inputs(cfg, seed=seed)
    out, _ = naive(inp)
    ref = brute.mla_decode_brute(inp.q.tolist(), inp.pool_f32().tolist(),
                                 inp.page_table.tolist(), inp.ctx_lens.tolist(),
                                 inp.w_uk.tolist(), inp.w_uv.tolist(), cfg.scale,
                                 cfg.page_size, cfg.d_c)
    return rel_err(out, np.array(ref))


def test_planted_wrong_grouping_is_caught(monkeypatch):
    monkeypatch.setattr(mla, "weight_head_of", lambda H, Hw: np.arange(H) % Hw)
    assert _brute_vs_naive_err() > 1e-3


def test_planted_off_by_one_visibility_is_caught(monkeypatch):
    monkeypatch.setattr(mla, "visible_upto", lambda T, s_q, s: max(0, min(T, T - s_q + s)))
    assert _brute_vs_naive_err() > 1e-3


def test_planted_wrong_lse_is_caught(monkeypatch):
    def bad(z):
        e = np.exp(z - np.max(z))
        return e / e.sum(), np.log(e.sum())          # forgets the max shift
    monkeypatch.setattr(mla, "_softmax_stats", bad)
    with pytest.raises(AssertionError):
        test_single_visible_token_closed_form()


def test_planted_dropped_rope_term_is_caught(monkeypatch):
    orig = mla.gather_rows

    def no_rope(pool, row, T, P):
        r = orig(pool, row, T, P).copy()
        r[:, 64:] = 0.0
        return r
    monkeypatch.setattr(mla, "gather_rows", no_rope)
    with pytest.raises(AssertionError):
        test_identity_weights_reduce_to_textbook_mqa()
