"""Pins of the cache-append oracle against things other than itself (CPU only).

``oracle.append.rope`` is tied to the rotation's group properties (identity at position
0, norm preservation, composition of positions, dot products that depend on the position
difference only), to an independent complex-number formulation and to pure-Python loops;
``append_rows`` / ``cache_append`` to closed forms (identity projections) and to the
positions the decode path's causal visibility rule fixes.  The last group plants
mistakes and checks that a pin catches each.
"""
import cmath
import math

import numpy as np
import pytest

from oracle import append, mla

RNG = np.random.default_rng(1234)


def rope_complex(x, position, base=append.ROPE_BASE):
    """Independent route: pair (x_{2i}, x_{2i+1}) as the complex number x_{2i} + i x_{2i+1},
    multiplied by e^{i * position * base^(-2i/d)}."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.exp(-np.log(base) * np.arange(d // 2) * 2.0 / d)
    z = z * np.exp(1j * np.asarray(position, np.float64)[..., None] * theta)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def rope_loops(x, position, base=append.ROPE_BASE):
    """Pure-Python scalar loops with cmath.rect, one vector at a time."""
    d = len(x)
    out = [0.0] * d
    for i in range(d // 2):
        w = cmath.rect(1.0, position * base ** (-(2.0 * i) / d))
        z = complex(x[2 * i], x[2 * i + 1]) * w
        out[2 * i], out[2 * i + 1] = z.real, z.imag
    return out


# ------------------------------------------------------------------ the rotation

def test_rope_at_position_zero_is_identity():
    x = RNG.standard_normal((5, 64))
    assert np.array_equal(append.rope(x, np.zeros(5)), x)


def test_rope_preserves_norms_of_every_pair():
    x = RNG.standard_normal((7, 64))
    pos = RNG.integers(0, 200000, size=7)
    y = append.rope(x, pos)
    nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=0)


def test_rope_positions_compose():
    x = RNG.standard_normal((4, 64))
    m, n = np.array([3, 1000, 65535, 7]), np.array([9, 24, 1, 131000])
    assert np.allclose(append.rope(append.rope(x, m), n), append.rope(x, m + n),
                       rtol=0, atol=1e-9)


def test_rope_dot_products_depend_on_the_position_difference_only():
    a, b = RNG.standard_normal(64), RNG.standard_normal(64)
    ref = float(append.rope(a, 1000) @ append.rope(b, 990))
    for k in (0, 1, 77, 65536, 131061):
        got = float(append.rope(a, 1000 + k) @ append.rope(b, 990 + k))
        assert abs(got - ref) < 1e-9 * max(1.0, abs(ref))


def test_rope_matches_complex_formulation_and_loops():
    x = RNG.standard_normal((6, 16))
    pos = np.array([0, 1, 2, 63, 4096, 131071])
    y = append.rope(x, pos)
    assert np.allclose(y, rope_complex(x, pos), rtol=0, atol=1e-10)
    for i in range(6):
        assert np.allclose(y[i], rope_loops(list(x[i]), int(pos[i])), rtol=0, atol=1e-10)


def test_rope_pair_angles_closed_form():
    """The unit vector of pair i at position 1 turns by exactly base^(-2i/d) radians,
    measured with atan2; the first pair turns by 1 radian; pairs never mix."""
    d = 64
    for i in range(d // 2):
        e = np.zeros(d)
        e[2 * i] = 1.0
        y = append.rope(e, 1)
        ang = math.atan2(y[2 * i + 1], y[2 * i])
        assert abs(ang - 10000.0 ** (-2.0 * i / d)) < 1e-14
        rest = np.delete(y, [2 * i, 2 * i + 1])
        assert np.all(rest == 0.0)
    e = np.zeros(2)
    e[0] = 1.0
    assert np.allclose(append.rope(e, 2.5), [math.cos(2.5), math.sin(2.5)], atol=1e-15)


# ------------------------------------------------------------------ projection and write

def small_case(B=3, s_q=2, d_model=40, d_c=12, d_r=8, P=4, ctx=(1, 6, 9)):
    h = RNG.standard_normal((B, s_q, d_model))
    w_dkv = RNG.standard_normal((d_c, d_model)) / np.sqrt(d_model)
    w_kr = RNG.standard_normal((d_r, d_model)) / np.sqrt(d_model)
    ctx = np.asarray(ctx, np.int32)
    n_pages = [(int(t) + P - 1) // P for t in ctx]
    perm = RNG.permutation(sum(n_pages))
    mp = max(n_pages)
    table = np.full((B, mp), -1, np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = perm[off:off + n]
        off += n
    pool = RNG.standard_normal((sum(n_pages), P, d_c + d_r))
    return h, w_dkv, w_kr, ctx, table, pool, P


def test_identity_projections_give_the_hidden_state():
    """W_DKV = [I 0] copies h into the latent unrotated; W_KR = [0 I] puts the next d_R
    components of h into the RoPE key, rotated to the token's position."""
    B, s_q, d_model, d_c, d_r = 2, 2, 30, 12, 8
    h = RNG.standard_normal((B, s_q, d_model))
    w_dkv = np.eye(d_c, d_model)
    w_kr = np.eye(d_r, d_model, k=d_c)
    pos = append.new_token_positions([5, 70], s_q)
    rows = append.append_rows(h, w_dkv, w_kr, pos)
    assert np.array_equal(rows[..., :d_c], h[..., :d_c])
    for b in range(B):
        for s in range(s_q):
            want = rope_loops(list(h[b, s, d_c:d_c + d_r]), int(pos[b, s]))
            assert np.allclose(rows[b, s, d_c:], want, rtol=0, atol=1e-12)


def test_new_token_positions_follow_the_visibility_rule():
    """The new token of query row s is the last token row s may see."""
    ctx, s_q = [1, 5, 64], 3
    pos = append.new_token_positions(ctx, s_q)
    for b, T in enumerate(ctx):
        for s in range(s_q):
            assert pos[b, s] == mla.visible_upto(T, s_q, s) - 1 or pos[b, s] < 0


def test_cache_append_writes_exactly_the_new_rows():
    h, w_dkv, w_kr, ctx, table, pool, P = small_case()
    s_q = h.shape[1]
    before = pool.copy()
    out = append.cache_append(pool, table, ctx, h, w_dkv, w_kr, s_q, P)
    assert np.array_equal(pool, before)     # the input pool is not modified
    pos = np.maximum(append.new_token_positions(ctx, s_q), 0)
    rows = append.append_rows(h, w_dkv, w_kr, pos)
    written = np.zeros(pool.shape[:2], bool)
    for b, T in enumerate(ctx):
        for s in range(s_q):
            t = int(T) - s_q + s
            if t < 0:                       # sequence 0 holds one token: row s = 0 has none
                continue
            page = table[b, t // P]
            assert np.array_equal(out[page, t % P], rows[b, s])
            written[page, t % P] = True
    assert written.sum() == 5               # 1 + 2 + 2 new rows, the t < 0 one skipped
    assert np.array_equal(out[~written], pool[~written])


def test_unmapped_pages_are_not_written():
    h, w_dkv, w_kr, ctx, table, pool, P = small_case()
    table = table.copy()
    table[2, :] = -1
    out = append.cache_append(pool, table, ctx, h, w_dkv, w_kr, h.shape[1], P)
    for b in (0, 1):
        t = int(ctx[b]) - 1
        assert not np.array_equal(out[table[b, t // P], t % P], pool[table[b, t // P], t % P])
    changed = np.any(out != pool, axis=-1)
    assert changed.sum() == 3               # sequences 0 and 1 only


# ------------------------------------------------------------------ planted mistakes

def _rope_halves(x, position, base=append.ROPE_BASE):
    """Mistake: rotate (x_i, x_{i + d/2}) instead of consecutive pairs."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return append.rope(x[..., inv], position, base)[..., perm]


@pytest.mark.parametrize("mistake", ["halves", "position+1", "base 1e4 -> 1e6"])
def test_planted_mistakes_are_caught(mistake):
    x = RNG.standard_normal((3, 16))
    pos = np.array([1, 5, 300])
    if mistake == "halves":
        got = _rope_halves(x, pos)
    elif mistake == "position+1":
        got = append.rope(x, pos + 1)
    else:
        got = append.rope(x, pos, base=1e6)
    assert not np.allclose(got, rope_complex(x, pos), rtol=0, atol=1e-6)
