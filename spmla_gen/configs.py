"""Workload recipes for the sparse paged MLA decode step.

Each recipe fixes the shapes, storage formats, seed and value distributions
of one synthetic workload.  The workloads follow the decode setting that the
pages describe: DSA-style Top-k token selection over an MLA compressed latent
cache shared by all heads (Kuaishou Wanqing inference article, 6aiq.com,
sections 5.1.1-5.1.2), paged through a block table (deepseekmodel.com engine
guide, "PagedAttention's two primitives"), stored in bf16 or in FP8 e4m3 with
a per-token scale (Workers AI KV-quantisation article, section 1).  Numeric
sizes (heads, latent and rope dims, indexer heads, k, lengths) are workload
choices, not values stated on the pages.
"""
from dataclasses import dataclass, field, replace
import math

F32, BF16, FP8 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3"}


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    lens: tuple            # ("fixed", (L0, L1, ...)) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    n_heads: int
    d_latent: int
    d_rope: int
    page_size: int
    cache_dtype: int       # F32 / BF16 / FP8
    q_dtype: int           # F32 / BF16 (query and indexer query)
    topk: int
    seed: int
    idx_heads: int = 0     # 0: no indexer (dense attention over every token)
    idx_dim: int = 0
    idx_dtype: int = BF16
    w_dist: str = "uniform"  # "uniform" U(0,1) or "normal" N(0,1) indexer head weights
    pool_factor: float = 1.0  # physical pool pages / needed pages
    sm_scale: float = 0.0     # 0: 1/sqrt(d_latent + d_rope)

    @property
    def dim(self):
        return self.d_latent + self.d_rope

    @property
    def softmax_scale(self):
        return self.sm_scale if self.sm_scale else 1.0 / math.sqrt(self.dim)

    @property
    def dense(self):
        return self.idx_heads == 0

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    # Tiny oracle case.
    "c1": Config("c1", 2, ("fixed", (37, 100)), 8, 64, 16, 16, F32, F32, 32, seed=1,
                 idx_heads=2, idx_dim=16, idx_dtype=F32, w_dist="normal", sm_scale=1.0 / math.sqrt(80.0)),
    # Dense MLA decode, bf16 cache, every token attended.
    "c2": Config("c2", 32, ("uniform", 1024, 8192), 128, 512, 64, 64, BF16, BF16, 0, seed=2),
    # Sparse DSA + MLA decode, bf16 cache and indexer keys.
    "c3": Config("c3", 64, ("uniform", 32768, 131072), 128, 512, 64, 64, BF16, BF16, 2048, seed=3,
                 idx_heads=64, idx_dim=128, idx_dtype=BF16),
    # The same draws as c3 with the latent cache and indexer keys stored FP8 e4m3 + per-token scale.
    "c3f": Config("c3f", 64, ("uniform", 32768, 131072), 128, 512, 64, 64, FP8, BF16, 2048, seed=3,
                  idx_heads=64, idx_dim=128, idx_dtype=FP8),
    # Continuous-batching mix, FP8 cache, pages scattered over a 1.25x pool.
    "c4": Config("c4", 128, ("lognormal", 8192, 1.0, 512, 65536), 128, 512, 64, 64, FP8, BF16, 2048, seed=4,
                 idx_heads=64, idx_dim=128, idx_dtype=FP8, pool_factor=1.25),
    # Million-token contexts.
    "c5": Config("c5", 4, ("fixed", (1048576,) * 4), 128, 512, 64, 64, FP8, BF16, 2048, seed=5,
                 idx_heads=64, idx_dim=128, idx_dtype=FP8),
}
