"""Plain float64 definition of the cache-append step (test infrastructure only).

The write side of the decode path: each new token's hidden state is projected down to
the latent and to the decoupled RoPE key, the RoPE key is rotated to the token's
position, and the row [c_t | k^R_t] is written into the paged cache.

Page references (each names the page's title and the section on it):

[MLA-GRPO]   "MLA and GRPO architecture" - section 2 "Multi-Head Latent Attention (MLA)",
             subsections "The Mathematics of MLA" (down-projection of the hidden state to
             the latent) and "Decoupled Rotary Position Embeddings (RoPE)" (a dedicated
             RoPE key, the only rotated part; the cached state per token is the latent and
             that key).

Readings where the pages are silent (each one also listed in the design notes):
  * The RoPE key is a linear projection of the hidden state, k^R_t = RoPE_t(W_KR h_t):
    the pages name the key and say RoPE is applied to it alone, but give no formula for
    where it comes from; a projection of h_t, like the latent, is the plain reading.
  * The rotation is the rotary embedding's own definition: consecutive pairs
    (x_{2i}, x_{2i+1}) rotated by the angle t * base^(-2i / d_R), base 10000.  The pages
    give no convention.
  * A new token's position is its index in the sequence: the s_q new tokens of a step are
    the last s_q of the T_b cached ones (t = T_b - s_q + s), the same rule the decode
    path's causal visibility uses.

Array conventions (float arrays are converted to float64 on entry):
  h          [B, s_q, d_model]    hidden states of the new tokens
  w_dkv      [d_c, d_model]       latent down-projection
  w_kr       [d_rope, d_model]    RoPE-key projection
  pool       [num_pages, P, d_c + d_rope]
  page_table [B, max_pages] int;  ctx_lens [B] int (new tokens included)
"""
import numpy as np

ROPE_BASE = 10000.0


def rope(x, position, base=ROPE_BASE):
    """Rotate consecutive pairs of the last axis of x by position * base^(-2i / d).

    [MLA-GRPO] "Decoupled Rotary Position Embeddings (RoPE)": the rotation applies to
    the small RoPE key only.  ``position`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE width must be even")
    freq = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)           # [d / 2]
    ang = np.asarray(position, dtype=np.float64)[..., None] * freq       # [..., d / 2]
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def new_token_positions(ctx_lens, s_q):
    """[B, s_q] positions t = T_b - s_q + s of the step's new tokens (may be < 0 when a
    sequence holds fewer than s_q tokens; such tokens are not written)."""
    T = np.asarray(ctx_lens, dtype=np.int64)[:, None]
    return T - s_q + np.arange(s_q, dtype=np.int64)[None, :]


def append_rows(h, w_dkv, w_kr, positions, base=ROPE_BASE):
    """Cache rows [c_t | k^R_t] of the new tokens: [B, s_q, d_c + d_rope].

    [MLA-GRPO] "The Mathematics of MLA": c_t = W_DKV h_t; "Decoupled RoPE": the dedicated
    key is rotated, the latent is not.
    """
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, dtype=np.float64).T
    kr = rope(h @ np.asarray(w_kr, dtype=np.float64).T, positions, base)
    return np.concatenate([c, kr], axis=-1)


def cache_append(pool, page_table, ctx_lens, h, w_dkv, w_kr, s_q, page_size,
                 base=ROPE_BASE):
    """The pool after writing the step's new rows (a float64 copy; the input is untouched).

    Token (b, s) goes to row t % P of physical page page_table[b, t // P]; tokens with
    t < 0 or an unmapped page (entry < 0) are not written.
    """
    out = np.array(pool, dtype=np.float64, copy=True)
    pos = new_token_positions(ctx_lens, s_q)
    rows = append_rows(h, w_dkv, w_kr, np.maximum(pos, 0), base)
    for b in range(pos.shape[0]):
        for s in range(s_q):
            t = int(pos[b, s])
            if t < 0 or t // page_size >= page_table.shape[1]:
                continue
            page = int(page_table[b, t // page_size])
            if page < 0:
                continue
            out[page, t % page_size] = rows[b, s]
    return out
