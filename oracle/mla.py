"""Plain float64 definitions of single-step MLA / GQLA decode (test infrastructure only).

Page references used below (each names the page's title and the section on it):

[MLA-GRPO]   "MLA and GRPO architecture" - section 1 "The Bottleneck: The KV Cache Crisis
             in Autoregressive LLMs"; section 2 "Multi-Head Latent Attention (MLA)":
             subsections "The Mathematics of MLA", "Decoupled Rotary Position Embeddings
             (RoPE)" and the table "Memory Footprint Comparison".
[DRIVENETS]  "How to upgrade GQA models to MLA for massive KV Cache Savings" - section
             "Under the hood: how offline conversion works" (the "Decompression
             Multiplex" stage) and section "Real-world results".
[CLARITY]    "MLA's 512-Scalar KV Latent Cuts Cache 98%, Enabling 512 Concurrent 128k
             Streams" (single article body).
[GQLA-ABS]   "GQLA: Group-Query Latent Attention for Hardware-Adaptive Large Language
             Model Decoding" - abstract.
[GQLA-RADIO] "GQLA: Group-Query Latent Attention for Hardware-Adaptive Decoding" (AI
             Radio episode) - "Key concepts", the paper abstract, and the transcript
             part "The paper's summary".

Array conventions (all float arrays are converted to float64 on entry):
  q          [B, s_q, H, d_nope + d_rope]   query; no-position part first, the RoPE part
                                            already rotated
  w_uk       [H_w, d_nope, d_c]             key up-projection, one slice per weight head
  w_uv       [H_w, d_v, d_c]                value up-projection, one slice per weight head
  pool       [num_pages, P, d_c + d_rope]   paged latent cache, one row [c_t | k^R_t] per token
  page_table [B, max_pages] int             logical page -> physical page
  ctx_lens   [B] int                        cached tokens per sequence, new tokens included
Query head h uses weight head w(h) = h // (H // H_w): H_w = H is MLA, H_w = G is GQLA.
Query row s (0 <= s < s_q) sees the cached tokens t <= T_b - s_q + s.
"""
import numpy as np


# --------------------------------------------------------------------------- helpers

def weight_head_of(n_heads, n_wheads):
    """Weight-head index w(h) for every query head h (contiguous groups).

    [GQLA-RADIO] paper abstract and "The paper's summary": GQLA indexes the
    up-projections by g groups instead of replicating them across the query heads; the
    MLA case is one group per head.  Contiguous grouping is the plain reading.
    """
    if n_heads % n_wheads != 0:
        raise ValueError("n_heads must be a multiple of n_wheads")
    return np.arange(n_heads) // (n_heads // n_wheads)


def visible_upto(T, s_q, s):
    """Number of cached tokens query row s may attend to: tokens 0 .. T - s_q + s.

    [MLA-GRPO] section 1: token t+1 attends over all prior tokens; the s_q new tokens
    are already in the cache and attend causally among themselves.
    """
    return max(0, min(T, T - s_q + s + 1))


def split_ranges(T, n_splits, page_size, split_tokens=0):
    """Token ranges [lo, hi) of the n_splits chunks of a T-token sequence.

    Even mode (split_tokens == 0): every chunk has L = ceil(ceil(T / S) / P) * P tokens
    (page aligned), the last ones may be short or empty.  Fixed mode: L = split_tokens.
    This chunking is the split-KV decomposition of the decode step; the pages do not
    describe it, so any chunking whose combine gives back the full softmax is valid.
    """
    if split_tokens > 0:
        L = split_tokens
    else:
        per = -(-T // n_splits)
        L = -(-per // page_size) * page_size
    return [(min(u * L, T), min((u + 1) * L, T)) for u in range(n_splits)]


def gather_rows(pool, page_table_row, T, page_size):
    """Logical cache rows 0..T-1 of one sequence, read through its page table."""
    t = np.arange(T)
    pages = np.asarray(page_table_row)[t // page_size]
    return np.asarray(pool[pages, t % page_size], dtype=np.float64)


def _softmax_stats(z):
    """Return (p, lse) of a logit vector: p = exp(z - max) / sum, lse = log sum exp z."""
    m = np.max(z)
    e = np.exp(z - m)
    l = np.sum(e)
    return e / l, m + np.log(l)


# --------------------------------------------------------------- the plain definition

def mla_decode_naive(q, pool, page_table, ctx_lens, w_uk, w_uv, scale, page_size,
                     d_c, batches=None, heads=None, return_probs=False):
    """Naive, non-absorbed MLA decode: materialise per-head K and V, then softmax attention.

    For each sequence b, query row s and head h (weight head w = w(h)):
      c_t, k^R_t = the cached row of token t, split at d_c           [MLA-GRPO] "Decoupled
                                                                     RoPE": cached state is
                                                                     [c_t^KV, k_t^R]
      K_h[t] = [W_UK[w] c_t ; k^R_t],  V_h[t] = W_UV[w] c_t           [MLA-GRPO] "The
                                                                     Mathematics of MLA"
      z_t = scale * <q[b,s,h], K_h[t]>  for visible t
      out[b,s,h] = sum_t softmax(z)_t V_h[t],  lse = log sum_t exp z_t
    A row with no visible token gives out = 0 and lse = -inf.
    ``batches`` / ``heads`` restrict the work to a subset; other entries stay NaN.
    Returns (out [B,s_q,H,d_v], lse [B,s_q,H]) and, if asked, {(b,s,h): p}.
    """
    q = np.asarray(q, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, s_q, H, dq = q.shape
    H_w, d_n, _ = w_uk.shape
    d_v = w_uv.shape[1]
    widx = weight_head_of(H, H_w)
    out = np.full((B, s_q, H, d_v), np.nan)
    lse = np.full((B, s_q, H), np.nan)
    probs = {}
    for b in (range(B) if batches is None else batches):
        T = int(ctx_lens[b])
        rows = gather_rows(pool, page_table[b], T, page_size)
        c, kr = rows[:, :d_c], rows[:, d_c:]
        for h in (range(H) if heads is None else heads):
            w = widx[h]
            K = np.concatenate([c @ w_uk[w].T, kr], axis=1)     # [T, d_n + d_rope]
            V = c @ w_uv[w].T                                    # [T, d_v]
            for s in range(s_q):
                n = visible_upto(T, s_q, s)
                if n == 0:
                    out[b, s, h], lse[b, s, h] = 0.0, -np.inf
                    continue
                z = scale * (K[:n] @ q[b, s, h])
                p, lse[b, s, h] = _softmax_stats(z)
                out[b, s, h] = p @ V[:n]
                if return_probs:
                    probs[(b, s, h)] = p
    if return_probs:
        return out, lse, probs
    return out, lse


# ----------------------------------------------------- steps of the absorbed (MQA) path

def absorb_query(q, w_uk, d_nope):
    """Query absorption: q_abs[b,s,h] = [W_UK[w(h)]^T q_nope ; q_rope].

    [DRIVENETS] "Under the hood", Decompression Multiplex: matrix products are
    associative, so the key up-projection moves onto the query and the query is
    projected into the latent space; keys are never decompressed.  [GQLA-RADIO] "Key
    concepts": on the MQA-absorb path the latent serves as the shared key.  The RoPE
    part bypasses W_UK ([MLA-GRPO] "Decoupled RoPE"; [CLARITY]: the rotation does not
    commute with the up-projection).
    """
    q = np.asarray(q, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    H = q.shape[2]
    widx = weight_head_of(H, w_uk.shape[0])
    q_lat = np.einsum("bshi,hic->bshc", q[..., :d_nope], w_uk[widx])
    return np.concatenate([q_lat, q[..., d_nope:]], axis=-1)


def absorbed_split_partials(q_abs, pool, page_table, ctx_lens, n_splits, scale,
                            page_size, d_c, split_tokens=0, batches=None):
    """Per-split softmax partials of absorbed attention over the latent cache.

    For split u of sequence b and query row (s, h), over the visible tokens t of u:
      z_t = scale * <q_abs[b,s,h], [c_t ; k^R_t]>
      o_u = sum_t softmax_u(z)_t c_t      (the latent is the value: [GQLA-RADIO] "Key
                                           concepts", MQA-absorb path)
      lse_u = log sum_t exp z_t
    An empty split gives o_u = 0, lse_u = -inf.
    Returns o_part [B,s_q,H,S,d_c], lse_part [B,s_q,H,S].
    """
    q_abs = np.asarray(q_abs, dtype=np.float64)
    B, s_q, H, D = q_abs.shape
    o_part = np.full((B, s_q, H, n_splits, d_c), np.nan)
    lse_part = np.full((B, s_q, H, n_splits), np.nan)
    for b in (range(B) if batches is None else batches):
        T = int(ctx_lens[b])
        rows = gather_rows(pool, page_table[b], T, page_size)
        for u, (lo, hi) in enumerate(split_ranges(T, n_splits, page_size, split_tokens)):
            for s in range(s_q):
                top = min(hi, visible_upto(T, s_q, s))
                if top <= lo:
                    o_part[b, s, :, u], lse_part[b, s, :, u] = 0.0, -np.inf
                    continue
                R = rows[lo:top]
                for h in range(H):
                    z = scale * (R @ q_abs[b, s, h])
                    p, lse_part[b, s, h, u] = _softmax_stats(z)
                    o_part[b, s, h, u] = p @ R[:, :d_c]
    return o_part, lse_part


def combine_splits(o_part, lse_part):
    """Merge split partials: lse = log sum_u exp lse_u, o = sum_u exp(lse_u - lse) o_u.

    This is the log-sum-exp identity of softmax over a union of disjoint token sets.
    Rows whose splits are all empty give o = 0, lse = -inf.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = np.max(lse_part, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    wts = np.exp(lse_part - m_safe)                          # exp(-inf) = 0
    tot = np.sum(wts, axis=-1, keepdims=True)
    tot_safe = np.where(empty, 1.0, tot)
    o = np.sum((wts / tot_safe)[..., None] * np.where(wts[..., None] > 0, o_part, 0.0),
               axis=-2)
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))[..., 0]
    o = np.where(empty, 0.0, o)
    return o, lse


def up_project_values(o_lat, w_uv):
    """Value up-projection after the latent reduction: out[b,s,h] = W_UV[w(h)] o_lat[b,s,h].

    [MLA-GRPO] "The Mathematics of MLA": v_t = W_UV c_t; by associativity
    sum_t p_t W_UV c_t = W_UV sum_t p_t c_t ([DRIVENETS] "Under the hood").
    """
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    widx = weight_head_of(o_lat.shape[2], w_uv.shape[0])
    return np.einsum("hvc,bshc->bshv", w_uv[widx], o_lat)


def mla_decode_absorbed_chain(q, pool, page_table, ctx_lens, w_uk, w_uv, scale, page_size,
                              d_c, n_splits, split_tokens=0):
    """The absorbed step written as the four plain steps above, for tests."""
    d_nope = np.asarray(w_uk).shape[1]
    q_abs = absorb_query(q, w_uk, d_nope)
    o_part, lse_part = absorbed_split_partials(q_abs, pool, page_table, ctx_lens, n_splits,
                                               scale, page_size, d_c, split_tokens)
    o_lat, lse = combine_splits(o_part, lse_part)
    return up_project_values(o_lat, w_uv), lse


# -------------------------------------------------------------------- GQLA GQA path

def expand_cache(pool, w_uk, w_uv, d_c):
    """Per-group expanded cache of the GQLA GQA path from the latent cache.

    [GQLA-RADIO] "The paper's summary": the GQA path caches per-group K and V plus the
    shared RoPE key.  With [MLA-GRPO] "The Mathematics of MLA":
      k[p, r, j] = W_UK[j] c,   v[p, r, j] = W_UV[j] c,   kr[p, r] = k^R
    for the row (p, r) = [c | k^R] of the latent pool.  Returns float64 arrays
    k [num_pages, P, G, d_nope], v [num_pages, P, G, d_v], kr [num_pages, P, d_rope].
    """
    pool = np.asarray(pool, dtype=np.float64)
    c, kr = pool[..., :d_c], pool[..., d_c:]
    k = np.einsum("jnc,prc->prjn", np.asarray(w_uk, dtype=np.float64), c)
    v = np.einsum("jvc,prc->prjv", np.asarray(w_uv, dtype=np.float64), c)
    return k, v, kr.copy()


def gqa_split_partials(q, k_pool, v_pool, kr_pool, page_table, ctx_lens, n_splits, scale,
                       page_size, split_tokens=0, batches=None, heads=None):
    """Per-split partials of the GQA path over the per-group expanded cache.

    Head h belongs to group j = w(h) and attends with
      z_t = scale * (<q_nope, K[t, j]> + <q_rope, k^R[t]>),  o_u = sum_t softmax_u(z)_t V[t, j]
    ([GQLA-ABS] abstract: a GQA path with a per-group expanded cache; [GQLA-RADIO] "The
    paper's summary": per-group K and V plus the shared RoPE key).
    Returns o_part [B,s_q,H,S,d_v], lse_part [B,s_q,H,S].
    """
    q = np.asarray(q, dtype=np.float64)
    B, s_q, H, _ = q.shape
    G, d_n = k_pool.shape[2], k_pool.shape[3]
    d_v = v_pool.shape[3]
    widx = weight_head_of(H, G)
    o_part = np.full((B, s_q, H, n_splits, d_v), np.nan)
    lse_part = np.full((B, s_q, H, n_splits), np.nan)
    for b in (range(B) if batches is None else batches):
        T = int(ctx_lens[b])
        t = np.arange(T)
        pages = np.asarray(page_table[b])[t // page_size]
        K_all = np.asarray(k_pool[pages, t % page_size], dtype=np.float64)   # [T, G, d_n]
        V_all = np.asarray(v_pool[pages, t % page_size], dtype=np.float64)   # [T, G, d_v]
        KR = np.asarray(kr_pool[pages, t % page_size], dtype=np.float64)     # [T, d_r]
        for u, (lo, hi) in enumerate(split_ranges(T, n_splits, page_size, split_tokens)):
            for s in range(s_q):
                top = min(hi, visible_upto(T, s_q, s))
                for h in (range(H) if heads is None else heads):
                    if top <= lo:
                        o_part[b, s, h, u], lse_part[b, s, h, u] = 0.0, -np.inf
                        continue
                    j = widx[h]
                    z = scale * (K_all[lo:top, j] @ q[b, s, h, :d_n]
                                 + KR[lo:top] @ q[b, s, h, d_n:])
                    p, lse_part[b, s, h, u] = _softmax_stats(z)
                    o_part[b, s, h, u] = p @ V_all[lo:top, j]
    return o_part, lse_part


# --------------------------------------------------------------- cache-size arithmetic

def mha_cache_scalars_per_token(n_heads, d_head):
    """One key and one value per head: 2 * n_h * d_h scalars per token per layer.

    [MLA-GRPO] section 1 formula and "Memory Footprint Comparison" table; [CLARITY]:
    32,768 scalars per token for 128 heads of dimension 128.
    """
    return 2 * n_heads * d_head


def gqa_cache_scalars_per_token(n_kv_heads, d_head):
    """GQA caches one K and one V per KV head: 2 * n_kv * d_h ([GQLA-ABS]: 2*8*128)."""
    return 2 * n_kv_heads * d_head


def mla_cache_scalars_per_token(d_c, d_rope):
    """MLA caches [c_t ; k^R_t]: d_c + d_R scalars per token per layer.

    [MLA-GRPO] "Decoupled RoPE" (cached state) and the "Memory Footprint Comparison"
    table; [GQLA-ABS]: the MQA-absorb path caches the latent plus the shared RoPE key.
    """
    return d_c + d_rope


def gqla_expanded_cache_scalars_per_token(n_groups, d_nope, d_v, d_rope):
    """The GQA path caches per-group K and V plus one shared RoPE key:
    G * (d_nope + d_v) + d_rope ([GQLA-RADIO] "The paper's summary")."""
    return n_groups * (d_nope + d_v) + d_rope


def kv_cache_bytes_per_token(n_layers, n_kv_heads, d_head, bytes_per_scalar):
    """Whole-model KV bytes per token: 2 * layers * heads * d_head * bytes ([MLA-GRPO] s.1)."""
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_scalar
