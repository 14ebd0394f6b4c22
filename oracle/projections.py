"""Plain float64 definitions of the projections around the decode path, in the unfolded
form and with the up-projections folded into them offline (test infrastructure only).

Page references (each names the page's title and the section on it):

[DRIVENETS]  "How to upgrade GQA models to MLA for massive KV Cache Savings" - section
             "Under the hood: how offline conversion works", the Decompression Multiplex
             stage: matrix products are associative, so the key up-projection can be
             multiplied into the query weights W^Q ahead of time; the query then lands in
             the latent space directly and the keys are never decompressed.
[MLA-GRPO]   "MLA and GRPO architecture" - section 2, "The Mathematics of MLA" (k = W_UK c,
             v = W_UV c) and "Decoupled Rotary Position Embeddings (RoPE)" (only the
             dedicated RoPE part is rotated).
[CLARITY]    "MLA's 512-Scalar KV Latent Cuts Cache 98%..." - the shapes MLA is described
             on: a 5120-wide hidden state, 128 heads of 128, a 512-wide latent.

Readings where the pages are silent (each one also listed in the design notes):
  * W^Q maps the hidden state straight to every head's query, q[h] = W^Q[h] x with W^Q[h]
    of shape [d_nope + d_rope, d_model], no-position rows first: the pages name W^Q and the
    hidden size, not a query latent.
  * The query's RoPE part is rotated at the query token's own position t = T_b - s_q + s,
    with the same rotation as the cache's RoPE key (append.rope).
  * The output projection W^O maps the concatenated head outputs back to the hidden state,
    y = sum_h W^O[:, h] out[h] with W^O of shape [d_model, H * d_v].  The pages do not name
    it; folding W_UV into it is the same associativity the page states for the key side.

Array conventions (float arrays are converted to float64 on entry):
  x      [B, s_q, d_model]             hidden states of the step's new tokens
  w_q    [H, d_nope + d_rope, d_model] query weights, no-position rows first
  w_uk   [H_w, d_nope, d_c];  w_uv [H_w, d_v, d_c]   (as in mla.py)
  w_o    [d_model, H * d_v]            output projection
"""
import numpy as np

from .append import ROPE_BASE, new_token_positions, rope
from .mla import weight_head_of


def project_query(x, w_q, ctx_lens, s_q, d_nope, base=ROPE_BASE):
    """q[b,s,h] = [W^Q_nope[h] x ; RoPE_t(W^Q_rope[h] x)], t = T_b - s_q + s: the query the
    absorbed path takes ([MLA-GRPO] "Decoupled RoPE": the no-position part unrotated)."""
    x = np.asarray(x, dtype=np.float64)
    w_q = np.asarray(w_q, dtype=np.float64)
    q = np.einsum("hod,bsd->bsho", w_q, x)
    pos = new_token_positions(ctx_lens, s_q)                    # [B, s_q]
    q[..., d_nope:] = rope(q[..., d_nope:], pos[:, :, None])
    return q


def fold_query_weights(w_q, w_uk, d_nope):
    """[DRIVENETS] Decompression Multiplex, done once offline: per head h the latent rows
    W_UK[w(h)]^T W^Q_nope[h] ([d_c, d_model]) followed by the RoPE rows W^Q_rope[h]
    unchanged: [H, d_c + d_rope, d_model]."""
    w_q = np.asarray(w_q, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    widx = weight_head_of(w_q.shape[0], w_uk.shape[0])
    lat = np.einsum("hic,hid->hcd", w_uk[widx], w_q[:, :d_nope])
    return np.concatenate([lat, w_q[:, d_nope:]], axis=1)


def project_query_folded(x, w_qf, ctx_lens, s_q, d_c, base=ROPE_BASE):
    """q_abs[b,s,h] = [W~^Q_lat[h] x ; RoPE_t(W^Q_rope[h] x)]: the absorbed query straight
    from the hidden state, with no runtime absorption step."""
    x = np.asarray(x, dtype=np.float64)
    w_qf = np.asarray(w_qf, dtype=np.float64)
    q = np.einsum("hod,bsd->bsho", w_qf, x)
    pos = new_token_positions(ctx_lens, s_q)
    q[..., d_c:] = rope(q[..., d_c:], pos[:, :, None])
    return q


def output_projection(out, w_o):
    """y[b,s] = sum_h W^O[:, h d_v:(h+1) d_v] out[b,s,h] (out from the value up-projection)."""
    out = np.asarray(out, dtype=np.float64)
    B, s_q, H, d_v = out.shape
    return out.reshape(B, s_q, H * d_v) @ np.asarray(w_o, dtype=np.float64).T


def fold_output_weights(w_o, w_uv, n_heads):
    """The value-side fold, done once offline: block h of W~^O is W^O[:, h] W_UV[w(h)]
    ([d_model, d_c]); [d_model, H * d_c]."""
    w_o = np.asarray(w_o, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    H_w, d_v, d_c = w_uv.shape
    widx = weight_head_of(n_heads, H_w)
    blocks = [w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[widx[h]] for h in range(n_heads)]
    return np.concatenate(blocks, axis=1)


def output_projection_folded(o_lat, w_of):
    """y[b,s] = sum_h W~^O[:, h d_c:(h+1) d_c] o_lat[b,s,h]: the hidden-state output straight
    from the merged latent outputs, with no runtime value up-projection."""
    o_lat = np.asarray(o_lat, dtype=np.float64)
    B, s_q, H, d_c = o_lat.shape
    return o_lat.reshape(B, s_q, H * d_c) @ np.asarray(w_of, dtype=np.float64).T
