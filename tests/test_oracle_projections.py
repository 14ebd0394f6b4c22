"""Pins of oracle/projections.py against things other than itself (CPU only).

* The fold is the associativity the Decompression Multiplex stage rests on ("How to upgrade
  GQA models to MLA...", Under the hood): projecting with the folded weights equals
  projecting, then absorbing with the already pinned ``mla.absorb_query``; on the output
  side, the folded projection equals the value up-projection (``mla.up_project_values``)
  followed by the output projection.
* Pure-Python scalar loops (with the rotation written out as complex multiplication) on
  tiny shapes tie both projections to their definitions.
* Identity weights give closed forms.
* A whole step, hidden state in and hidden state out, through the naive decode equals the
  folded chain through the absorbed split path.
* Planted mistakes (a transposed fold, an unrotated query, a wrong head group) are caught.
"""
import cmath
import math

import numpy as np
import pytest

from oracle import append, mla
from oracle import projections as pj
from workloads import Config, make_inputs, make_projection_inputs


def cfg_small(**kw):
    base = dict(name="t", dtype="f32", batch=2, s_q=2, n_heads=8, n_wheads=2, d_c=24,
                d_rope=8, d_nope=12, d_v=10, ctx=("list", [40, 9]), n_splits=3)
    base.update(kw)
    return Config(**base)


def rel_err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(b)))


def inputs(d_model=16, seed=3, **kw):
    cfg = cfg_small(**kw)
    return cfg, make_inputs(cfg, seed=seed), make_projection_inputs(cfg, d_model, seed=seed)


# ------------------------------------------------------------------ associativity

@pytest.mark.parametrize("Hw", [8, 2, 1])
def test_folded_query_equals_projection_then_absorption(Hw):
    cfg, inp, pr = inputs(n_wheads=Hw)
    q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    want = mla.absorb_query(q, inp.w_uk, cfg.d_nope)
    wqf = pj.fold_query_weights(pr.w_q, inp.w_uk, cfg.d_nope)
    assert wqf.shape == (cfg.n_heads, cfg.d_c + cfg.d_rope, pr.d_model)
    got = pj.project_query_folded(pr.x, wqf, inp.ctx_lens, cfg.s_q, cfg.d_c)
    assert rel_err(got, want) < 1e-13


@pytest.mark.parametrize("Hw", [8, 2, 1])
def test_folded_output_equals_up_projection_then_output_projection(Hw):
    cfg, inp, pr = inputs(n_wheads=Hw)
    o_lat = np.random.default_rng(8).standard_normal((cfg.batch, cfg.s_q, cfg.n_heads,
                                                      cfg.d_c))
    want = pj.output_projection(mla.up_project_values(o_lat, inp.w_uv), pr.w_o)
    wof = pj.fold_output_weights(pr.w_o, inp.w_uv, cfg.n_heads)
    assert wof.shape == (pr.d_model, cfg.n_heads * cfg.d_c)
    got = pj.output_projection_folded(o_lat, wof)
    assert rel_err(got, want) < 1e-13


# ------------------------------------------------------------- pure-Python loops

def project_query_loops(x, w_q, ctx_lens, s_q, d_nope, base=append.ROPE_BASE):
    B, _, d_model = x.shape
    H, dq, _ = w_q.shape
    d_r = dq - d_nope
    out = np.zeros((B, s_q, H, dq))
    for b in range(B):
        for s in range(s_q):
            t = int(ctx_lens[b]) - s_q + s
            for h in range(H):
                v = [sum(float(w_q[h, o, i]) * float(x[b, s, i]) for i in range(d_model))
                     for o in range(dq)]
                for o in range(d_nope):
                    out[b, s, h, o] = v[o]
                for i in range(d_r // 2):
                    z = complex(v[d_nope + 2 * i], v[d_nope + 2 * i + 1]) * \
                        cmath.rect(1.0, t * base ** (-(2.0 * i) / d_r))
                    out[b, s, h, d_nope + 2 * i] = z.real
                    out[b, s, h, d_nope + 2 * i + 1] = z.imag
    return out


def output_projection_loops(out, w_o):
    B, s_q, H, d_v = out.shape
    d_model = w_o.shape[0]
    y = np.zeros((B, s_q, d_model))
    for b in range(B):
        for s in range(s_q):
            for m in range(d_model):
                y[b, s, m] = sum(float(w_o[m, h * d_v + i]) * float(out[b, s, h, i])
                                 for h in range(H) for i in range(d_v))
    return y


def test_query_projection_matches_loops():
    cfg, inp, pr = inputs(d_model=10, n_heads=3, n_wheads=3, batch=2, ctx=("list", [5, 2]))
    got = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    want = project_query_loops(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    assert rel_err(got, want) < 1e-13


def test_output_projection_matches_loops():
    cfg, inp, pr = inputs(d_model=7, n_heads=3, n_wheads=3)
    out = np.random.default_rng(9).standard_normal((cfg.batch, cfg.s_q, cfg.n_heads,
                                                    cfg.d_v))
    assert rel_err(pj.output_projection(out, pr.w_o), output_projection_loops(out, pr.w_o)) \
        < 1e-13


def test_folded_weights_match_loops():
    """Each folded entry is the sum over the up-projection's rows, written out."""
    cfg, inp, pr = inputs(d_model=6, n_heads=4, n_wheads=2)
    wqf = pj.fold_query_weights(pr.w_q, inp.w_uk, cfg.d_nope)
    wof = pj.fold_output_weights(pr.w_o, inp.w_uv, cfg.n_heads)
    for h in range(cfg.n_heads):
        w = h // 2
        for c in range(cfg.d_c):
            for d in range(pr.d_model):
                v = sum(float(inp.w_uk[w, i, c]) * float(pr.w_q[h, i, d])
                        for i in range(cfg.d_nope))
                assert math.isclose(wqf[h, c, d], v, rel_tol=1e-12, abs_tol=1e-13)
                v = sum(float(pr.w_o[d, h * cfg.d_v + i]) * float(inp.w_uv[w, i, c])
                        for i in range(cfg.d_v))
                assert math.isclose(wof[d, h * cfg.d_c + c], v, rel_tol=1e-12, abs_tol=1e-13)
        np.testing.assert_array_equal(wqf[h, cfg.d_c:], pr.w_q[h, cfg.d_nope:])


# ------------------------------------------------------------- closed forms

def test_identity_query_weights_select_the_hidden_state():
    """W^Q[h] = [I | 0] makes q[h] the first d_nope + d_rope hidden values, with the RoPE
    part rotated at the token's position (unrotated at position 0)."""
    cfg, inp, pr = inputs(d_model=24, ctx=("list", [2, 1]))
    dq = cfg.d_nope + cfg.d_rope
    w_q = np.zeros((cfg.n_heads, dq, 24))
    w_q[:, :, :dq] = np.eye(dq)
    q = pj.project_query(pr.x, w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    x = pr.x.astype(np.float64)
    for b in range(cfg.batch):
        for s in range(cfg.s_q):
            t = int(inp.ctx_lens[b]) - cfg.s_q + s
            np.testing.assert_allclose(q[b, s, :, :cfg.d_nope],
                                       np.broadcast_to(x[b, s, :cfg.d_nope],
                                                       (cfg.n_heads, cfg.d_nope)), rtol=0)
            if t == 0:
                np.testing.assert_allclose(q[b, s, 0, cfg.d_nope:], x[b, s, cfg.d_nope:dq],
                                           rtol=0, atol=0)
            # rotation keeps each pair's length
            pair = q[b, s, 0, cfg.d_nope:].reshape(-1, 2)
            ref = x[b, s, cfg.d_nope:dq].reshape(-1, 2)
            np.testing.assert_allclose(np.hypot(pair[:, 0], pair[:, 1]),
                                       np.hypot(ref[:, 0], ref[:, 1]), rtol=1e-13)


def test_identity_output_weights_concatenate_heads():
    cfg, inp, pr = inputs(d_model=8 * 10, n_heads=8, d_v=10)
    out = np.random.default_rng(5).standard_normal((cfg.batch, cfg.s_q, 8, 10))
    y = pj.output_projection(out, np.eye(80))
    np.testing.assert_array_equal(y, out.reshape(cfg.batch, cfg.s_q, 80))


# ----------------------------------------------------------- the whole step

@pytest.mark.parametrize("Hw,S", [(8, 3), (2, 1), (1, 4)])
def test_whole_step_folded_equals_naive(Hw, S):
    """Hidden state in, hidden state out: the naive decode (keys and values decompressed per
    head) between the unfolded projections equals the folded projections around the
    absorbed split path."""
    cfg, inp, pr = inputs(d_model=20, n_wheads=Hw, n_splits=S)
    q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    out, _ = mla.mla_decode_naive(q, inp.pool_f32(), inp.page_table, inp.ctx_lens, inp.w_uk,
                                  inp.w_uv, cfg.scale, cfg.page_size, cfg.d_c)
    want = pj.output_projection(out, pr.w_o)
    q_abs = pj.project_query_folded(pr.x, pj.fold_query_weights(pr.w_q, inp.w_uk, cfg.d_nope),
                                    inp.ctx_lens, cfg.s_q, cfg.d_c)
    o_p, l_p = mla.absorbed_split_partials(q_abs, inp.pool_f32(), inp.page_table, inp.ctx_lens,
                                           S, cfg.scale, cfg.page_size, cfg.d_c)
    o_lat, _ = mla.combine_splits(o_p, l_p)
    got = pj.output_projection_folded(o_lat, pj.fold_output_weights(pr.w_o, inp.w_uv,
                                                                    cfg.n_heads))
    assert rel_err(got, want) < 1e-11


# ----------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    cfg, inp, pr = inputs(n_wheads=2)
    q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    want = mla.absorb_query(q, inp.w_uk, cfg.d_nope)
    # a wrong head group in the fold (heads reversed)
    bad = pj.fold_query_weights(pr.w_q[::-1].copy(), inp.w_uk, cfg.d_nope)[::-1]
    got = pj.project_query_folded(pr.x, bad, inp.ctx_lens, cfg.s_q, cfg.d_c)
    assert rel_err(got, want) > 1e-3
    # the query's RoPE part left unrotated
    monkeypatch.setattr(pj, "rope", lambda x, pos, base=None: np.asarray(x, np.float64))
    got = pj.project_query_folded(pr.x, pj.fold_query_weights(pr.w_q, inp.w_uk, cfg.d_nope),
                                  inp.ctx_lens, cfg.s_q, cfg.d_c)
    assert rel_err(got, want) > 1e-3
    monkeypatch.undo()
    # the output fold with its head blocks shifted by one head
    o_lat = np.random.default_rng(8).standard_normal((cfg.batch, cfg.s_q, cfg.n_heads,
                                                      cfg.d_c))
    want_y = pj.output_projection(mla.up_project_values(o_lat, inp.w_uv), pr.w_o)
    wof = pj.fold_output_weights(pr.w_o, inp.w_uv, cfg.n_heads)
    assert rel_err(pj.output_projection_folded(o_lat, np.roll(wof, cfg.d_c, axis=1)),
                   want_y) > 1e-3


def test_planted_transposed_fold_is_caught():
    """With a square up-projection (d_nope = d_c) a fold that forgets to transpose W_UK has
    the right shape; the associativity pin must still reject it."""
    cfg, inp, pr = inputs(d_c=12, d_nope=12)
    q = pj.project_query(pr.x, pr.w_q, inp.ctx_lens, cfg.s_q, cfg.d_nope)
    want = mla.absorb_query(q, inp.w_uk, cfg.d_nope)
    w_uk = np.asarray(inp.w_uk, np.float64)
    widx = mla.weight_head_of(cfg.n_heads, cfg.n_wheads)
    lat = np.einsum("hci,hid->hcd", w_uk[widx], np.asarray(pr.w_q, np.float64)[:, :12])
    bad = np.concatenate([lat, np.asarray(pr.w_q, np.float64)[:, 12:]], axis=1)
    got = pj.project_query_folded(pr.x, bad, inp.ctx_lens, cfg.s_q, cfg.d_c)
    assert rel_err(got, want) > 1e-3
