"""Seeded synthetic inputs for MLA / GQLA decode (random draws and encodings only).

Recipe (seed s, numpy ``SeedSequence(s).spawn(7)`` streams in this order):
  0 q        ~ N(0, 1)                         [B, s_q, H, d_nope + d_rope]
  1 c_kv     ~ N(0, 1)                         latent part of every pool row
  2 k_rope   ~ N(0, 1)                         RoPE part of every pool row (already rotated)
  3 W_UK     ~ N(0, 1) / sqrt(d_c)             [H_w, d_nope, d_c]
  4 W_UV     ~ N(0, 1) / sqrt(d_c)             [H_w, d_v, d_c]
  5 ctx_lens fixed, or integer-uniform in [lo, hi] inclusive
  6 page permutation of all used pages
The cache-append step's inputs (hidden states, W_DKV, W_KR) come from
``make_append_inputs`` with streams of their own.
Values are drawn in float32; for bf16 workloads they are rounded to bf16
(round-to-nearest-even) and those bf16 values ARE the inputs.  The pool is generated in
physical page order; sequence b owns ceil(T_b / P) pages whose physical ids are
``perm[off_b : off_b + n_b]`` (``page_table[b, i]``); unused table entries are -1 and the
rows past T_b in a sequence's last page are NaN, so a kernel that reads them poisons its
output.
"""
import numpy as np

from .configs import Config

_CHUNK_PAGES = 2048


# ------------------------------------------------------------------ bf16 encoding

def bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), rounded)


def bf16_decode(bits):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x):
    """float32 values rounded to the nearest bf16 value (returned as float32)."""
    return bf16_decode(bf16_bits(x))


class Bf16View:
    """Read-only float32 view of a bf16-bit array: indexing decodes only what it reads."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_decode(self.bits[idx])


# ------------------------------------------------------------------ the inputs

class Inputs:
    """One seeded workload instance.

    q, w_uk, w_uv: float32 (bf16-exact when cfg.dtype == "bf16").
    pool: float32 [num_pages, P, D] for f32 workloads, uint16 bf16 bits for bf16 ones.
    """

    def __init__(self, cfg, q, w_uk, w_uv, pool, page_table, ctx_lens):
        self.cfg = cfg
        self.q, self.w_uk, self.w_uv = q, w_uk, w_uv
        self.pool = pool
        self.page_table = page_table
        self.ctx_lens = ctx_lens
        self.num_pages = pool.shape[0]
        self.max_pages = page_table.shape[1]

    @property
    def is_bf16(self):
        return self.cfg.dtype == "bf16"

    def pool_view(self):
        """Array-like float32 view of the pool (decodes bf16 lazily)."""
        return Bf16View(self.pool) if self.is_bf16 else self.pool

    def pool_f32(self):
        return bf16_decode(self.pool) if self.is_bf16 else self.pool

    @property
    def total_tokens(self):
        return int(np.sum(self.ctx_lens, dtype=np.int64))


def _ctx_lens(cfg, rng):
    kind = cfg.ctx[0]
    if kind == "fixed":
        return np.full(cfg.batch, cfg.ctx[1], dtype=np.int32)
    if kind == "uniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    if kind == "list":
        return np.asarray(cfg.ctx[1], dtype=np.int32)
    raise ValueError(f"unknown ctx rule {cfg.ctx}")


def _normal(rng, shape, bf16):
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_round(x) if bf16 else x


def make_inputs(cfg: Config, seed=None, identity_table=False, extra_pages=0,
                max_pages=None):
    """Build the seeded inputs of ``cfg`` (seed defaults to cfg.seed).

    identity_table: page i of the concatenated sequences is physical page i (no
    permutation).  extra_pages: unused physical pages appended to the pool (filled with
    NaN).  max_pages: page-table row stride (default: the largest sequence's page count).
    """
    seed = cfg.seed if seed is None else seed
    streams = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(7)]
    bf16 = cfg.dtype == "bf16"
    B, s_q, H, Hw = cfg.batch, cfg.s_q, cfg.n_heads, cfg.n_wheads
    P, d_c, d_r = cfg.page_size, cfg.d_c, cfg.d_rope

    q = _normal(streams[0], (B, s_q, H, cfg.d_nope + d_r), bf16)
    ctx = _ctx_lens(cfg, streams[5])
    n_pages_b = (ctx.astype(np.int64) + P - 1) // P
    n_used = int(n_pages_b.sum())
    num_pages = n_used + extra_pages
    inv = np.float32(1.0 / np.sqrt(d_c))
    w_uk = _normal(streams[3], (Hw, cfg.d_nope, d_c), False) * inv
    w_uv = _normal(streams[4], (Hw, cfg.d_v, d_c), False) * inv
    if bf16:
        w_uk, w_uv = bf16_round(w_uk), bf16_round(w_uv)

    # pool rows in physical order, generated in chunks of pages
    D = d_c + d_r
    pool = np.empty((num_pages, P, D), dtype=np.uint16 if bf16 else np.float32)
    for p0 in range(0, num_pages, _CHUNK_PAGES):
        p1 = min(num_pages, p0 + _CHUNK_PAGES)
        c = streams[1].standard_normal(((p1 - p0) * P, d_c), dtype=np.float32)
        r = streams[2].standard_normal(((p1 - p0) * P, d_r), dtype=np.float32)
        blk = np.concatenate([c, r], axis=1).reshape(p1 - p0, P, D)
        pool[p0:p1] = bf16_bits(blk) if bf16 else blk
    nan = np.uint16(0x7FC0) if bf16 else np.float32(np.nan)
    if extra_pages:
        pool[n_used:] = nan

    perm = (np.arange(n_used, dtype=np.int64) if identity_table
            else streams[6].permutation(n_used))
    mp = int(n_pages_b.max()) if max_pages is None else int(max_pages)
    if mp < int(n_pages_b.max()):
        raise ValueError("max_pages smaller than the longest sequence")
    table = np.full((B, mp), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(n_pages_b[b])
        table[b, :n] = perm[off:off + n]
        tail = int(ctx[b]) - (n - 1) * P          # valid rows in the last page
        if n > 0 and tail < P:
            pool[perm[off + n - 1], tail:] = nan
        off += n
    return Inputs(cfg, q, w_uk, w_uv, pool, table, ctx)


class AppendInputs:
    """Inputs of the cache-append step for one workload: the new tokens' hidden states
    and the two down-projections (float32; bf16-exact for bf16 workloads)."""

    def __init__(self, h, w_dkv, w_kr):
        self.h, self.w_dkv, self.w_kr = h, w_dkv, w_kr
        self.d_model = h.shape[-1]


def make_append_inputs(cfg: Config, d_model=5120, seed=None):
    """Seeded inputs of the cache-append step, from streams of their own
    (``SeedSequence([seed, 1]).spawn(3)``) so the decode inputs of the same seed are
    unchanged:  0 h ~ N(0, 1) [B, s_q, d_model];  1 W_DKV ~ N(0, 1) / sqrt(d_model)
    [d_c, d_model];  2 W_KR ~ N(0, 1) / sqrt(d_model) [d_rope, d_model].  The
    projections then have unit variance, like the drawn cache rows."""
    seed = cfg.seed if seed is None else seed
    streams = [np.random.default_rng(x) for x in np.random.SeedSequence([seed, 1]).spawn(3)]
    bf16 = cfg.dtype == "bf16"
    inv = np.float32(1.0 / np.sqrt(d_model))
    h = _normal(streams[0], (cfg.batch, cfg.s_q, d_model), bf16)
    w_dkv = _normal(streams[1], (cfg.d_c, d_model), False) * inv
    w_kr = _normal(streams[2], (cfg.d_rope, d_model), False) * inv
    if bf16:
        w_dkv, w_kr = bf16_round(w_dkv), bf16_round(w_kr)
    return AppendInputs(h, w_dkv, w_kr)


class ProjectionInputs:
    """Inputs of the projections around the decode path: the new tokens' hidden states, the
    query weights and the output projection (float32; bf16-exact for bf16 workloads)."""

    def __init__(self, x, w_q, w_o):
        self.x, self.w_q, self.w_o = x, w_q, w_o
        self.d_model = x.shape[-1]


def make_projection_inputs(cfg: Config, d_model=5120, seed=None):
    """Seeded inputs of the query and output projections, from streams of their own
    (``SeedSequence([seed, 2]).spawn(3)``) so the decode inputs of the same seed are
    unchanged:  0 x ~ N(0, 1) [B, s_q, d_model];  1 W^Q ~ N(0, 1) / sqrt(d_model)
    [H, d_nope + d_rope, d_model], so the query has unit variance like the drawn q;
    2 W^O ~ N(0, 1) / sqrt(H d_v) [d_model, H d_v]."""
    seed = cfg.seed if seed is None else seed
    streams = [np.random.default_rng(x) for x in np.random.SeedSequence([seed, 2]).spawn(3)]
    bf16 = cfg.dtype == "bf16"
    x = _normal(streams[0], (cfg.batch, cfg.s_q, d_model), bf16)
    w_q = _normal(streams[1], (cfg.n_heads, cfg.d_nope + cfg.d_rope, d_model), False)
    w_q *= np.float32(1.0 / np.sqrt(d_model))
    w_o = _normal(streams[2], (d_model, cfg.n_heads * cfg.d_v), False)
    w_o *= np.float32(1.0 / np.sqrt(cfg.n_heads * cfg.d_v))
    if bf16:
        w_q, w_o = bf16_round(w_q), bf16_round(w_o)
    return ProjectionInputs(x, w_q, w_o)


def growing_score_inputs(cfg: Config, period_tokens, q_value=40.0, step=16.0, seed=None):
    """A workload whose scores climb on every 32-token tile (the rows' softmax reference must
    move on each one): q is zero except its first RoPE coordinate (q_value), and the first
    RoPE coordinate of the cached token at logical position t is step * ((t % period) // 32).
    With q_value 40, step 16 and the 1/sqrt(576) scale the score rises by 26.7 nats (38.5 log2
    units) per tile and restarts every ``period_tokens`` tokens (one split chunk).  The values
    are exact in bf16 while (period / 32 - 1) < 256."""
    inp = make_inputs(cfg, seed=seed)
    inp.q[...] = 0.0
    inp.q[..., cfg.d_nope] = q_value
    pool = inp.pool_f32().copy()
    for b in range(cfg.batch):
        T = int(inp.ctx_lens[b])
        for i in range(-(-T // cfg.page_size)):
            page = inp.page_table[b, i]
            t = i * cfg.page_size + np.arange(cfg.page_size)
            vals = (((t % period_tokens) // 32) * step).astype(np.float32)
            live = t < T
            pool[page, live, cfg.d_c] = vals[live]
    inp.pool = bf16_bits(pool) if cfg.dtype == "bf16" else pool
    return inp
