"""The decode workloads, by name.

Shapes follow the pages' models: DeepSeek-style MLA (128 heads, latent 512, RoPE key 64,
no-position/value head dim 128; "MLA's 512-Scalar KV Latent Cuts Cache 98%...") and a
LLaMA-3-8B-shaped GQLA model (32 query heads in 8 groups, head dim 128; "GQLA:
Group-Query Latent Attention..." abstract).  Context lengths stand in for the pages'
long-context streams (128k) and for GQLA's 8K-64K inputs.
"""
from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str              # "f32" or "bf16": dtype of q, weights and caches
    batch: int
    s_q: int                # new query tokens per sequence
    n_heads: int            # query heads H
    n_wheads: int           # weight heads H_w (H for MLA, G for GQLA)
    d_c: int                # latent width
    d_rope: int             # decoupled RoPE key width
    d_nope: int             # no-position query/key head width
    d_v: int                # value head width
    ctx: tuple              # ("fixed", T) or ("uniform", lo, hi) inclusive
    n_splits: int           # split-KV chunks per sequence
    page_size: int = 64
    split_tokens: int = 0   # 0: even page-aligned chunks; >0: fixed chunk length
    seed: int = 0

    @property
    def D(self):
        return self.d_c + self.d_rope

    @property
    def scale(self):
        # softmax scale 1/sqrt(d_c + d_rope): the pages state none; the width of the
        # absorbed dot product is the plain reading (1/sqrt(576) for the MLA shapes).
        return 1.0 / math.sqrt(self.d_c + self.d_rope)

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    # tiny fp32: absorbed vs naive expanded equality at 1e-4
    "tiny-f32": Config("tiny-f32", "f32", 2, 1, 8, 8, 64, 16, 32, 32, ("fixed", 256), 4),
    # DeepSeek-V2-shaped absorbed decode, batch 16 x 4096 (8 chunks, tuned over 4-16: 256
    # workgroups, one per CU)
    "dsv2-b16-t4096": Config("dsv2-b16-t4096", "bf16", 16, 1, 128, 128, 512, 64, 128, 128,
                             ("fixed", 4096), 8),
    # long-context paged decode, batch 4 x 131072, split-KV over 32 chunks
    "long-b4-t131072": Config("long-b4-t131072", "bf16", 4, 1, 128, 128, 512, 64, 128, 128,
                              ("fixed", 131072), 32),
    # ragged MTP decode: s_q = 2, lengths uniform in [1024, 32768]; every sequence cut into
    # 6 page-aligned chunks (tuned: 0.85 ms per step against 0.87-0.98 ms for 4, 8, 10 or 12
    # chunks and 1.28 ms for fixed 2048-token chunks)
    "mtp-b64-ragged": Config("mtp-b64-ragged", "bf16", 64, 2, 128, 128, 512, 64, 128, 128,
                             ("uniform", 1024, 32768), 6),
    # GQLA LLaMA-3-8B-shaped: 32 heads in 8 groups, contexts swept 8192..65536 (8 chunks at
    # 8192 and 65536, tuned for the absorbed path; the GQA path is within 2 % for 2-32)
    "gqla-b32-t8192": Config("gqla-b32-t8192", "bf16", 32, 1, 32, 8, 512, 64, 128, 128,
                             ("fixed", 8192), 8),
    "gqla-b32-t16384": Config("gqla-b32-t16384", "bf16", 32, 1, 32, 8, 512, 64, 128, 128,
                              ("fixed", 16384), 8),
    "gqla-b32-t32768": Config("gqla-b32-t32768", "bf16", 32, 1, 32, 8, 512, 64, 128, 128,
                              ("fixed", 32768), 8),
    "gqla-b32-t65536": Config("gqla-b32-t65536", "bf16", 32, 1, 32, 8, 512, 64, 128, 128,
                              ("fixed", 65536), 8),
    # the same model decoding two tokens per step (MTP, s_q = 2), the pairing the pages
    # give for the GQA path on H20
    "gqla-mtp-b32-t65536": Config("gqla-mtp-b32-t65536", "bf16", 32, 2, 32, 8, 512, 64, 128,
                                  128, ("fixed", 65536), 8),
    # one rank's share of the GQA path under 8-way tensor parallelism over the groups:
    # one group (its K, V and a replica of the RoPE key) and its 4 query heads
    "gqla-shard-b32-t65536": Config("gqla-shard-b32-t65536", "bf16", 32, 1, 4, 1, 512, 64,
                                    128, 128, ("fixed", 65536), 16),
}


def get_config(name, **overrides):
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg
