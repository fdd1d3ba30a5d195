"""Seeded synthetic inputs for the sparse paged MLA decode step.

This module only draws numbers and lays them out (lengths, page tables,
queries, cache rows, indexer keys and weights).  It holds none of the
attention method's arithmetic and is shared by the HIP path's tests and bench
and by the oracle's tests.  The heavy lifting is in gen.c (SplitMix64
counter-based draws, Box-Muller normals, bf16 / FP8 e4m3fn storage encoders).

Tensor ids of the draw streams: 0 lengths, 1 page permutation, 2 q,
3 latent rows, 4 indexer queries, 5 indexer head weights, 6 indexer keys,
7 filler for pool pages that no request maps.
"""
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import CONFIGS, Config, F32, BF16, FP8, DTYPE_NAMES  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspmla_gen.so")
_lib = None

(T_LENS, T_PERM, T_Q, T_KV, T_QIDX, T_W, T_KIDX, T_FILL, T_NEW_KV, T_NEW_KIDX, T_MQ_Q, T_MQ_QIDX, T_MQ_W,
 T_CHUNK_Q) = range(14)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.spmla_gen_stream_key.restype = u64
    lib.spmla_gen_stream_key.argtypes = [u64, u64, u64]
    lib.spmla_gen_normal_f32.argtypes = [u64, u64, i64, vp]
    lib.spmla_gen_uniform_f64.argtypes = [u64, u64, i64, vp]
    lib.spmla_gen_normal_f64.argtypes = [u64, u64, i64, vp]
    lib.spmla_gen_f32_to_bf16.argtypes = [vp, i64, vp]
    lib.spmla_gen_rows_to_fp8.argtypes = [vp, i64, i32, vp, vp]
    lib.spmla_gen_fill_pool.restype = ctypes.c_int
    lib.spmla_gen_fill_pool.argtypes = [u64, u64, i32, vp, i32, i32, vp, i32, i32, vp, vp, i32]
    lib.spmla_gen_fill_garbage.argtypes = [u64, i64, i32, vp, i32]
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def stream_key(seed, tensor_id, sub=0):
    return _load().spmla_gen_stream_key(seed, tensor_id, sub)


def uniforms(seed, tensor_id, sub, n, start=0):
    out = np.empty(n, np.float64)
    _load().spmla_gen_uniform_f64(stream_key(seed, tensor_id, sub), start, n, _ptr(out))
    return out


def normals64(seed, tensor_id, sub, n, start=0):
    out = np.empty(n, np.float64)
    _load().spmla_gen_normal_f64(stream_key(seed, tensor_id, sub), start, n, _ptr(out))
    return out


def normals32(seed, tensor_id, sub, n, start=0):
    out = np.empty(n, np.float32)
    _load().spmla_gen_normal_f32(stream_key(seed, tensor_id, sub), start, n, _ptr(out))
    return out


def to_bf16_bits(x):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().spmla_gen_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def to_fp8_rows(x):
    """fp32 [rows, dim] -> (uint8 e4m3fn codes [rows, dim], fp32 scale [rows]) with scale absmax/448."""
    x = np.ascontiguousarray(x, np.float32)
    rows, dim = x.shape
    out = np.empty((rows, dim), np.uint8)
    sc = np.empty(rows, np.float32)
    _load().spmla_gen_rows_to_fp8(_ptr(x), rows, dim, _ptr(out), _ptr(sc))
    return out, sc


def bf16_bits_to_f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_lengths(cfg: Config):
    kind = cfg.lens[0]
    if kind == "fixed":
        lens = np.array(cfg.lens[1], np.int64)
        assert len(lens) == cfg.batch
    elif kind == "uniform":
        lo, hi = cfg.lens[1], cfg.lens[2]
        u = uniforms(cfg.seed, T_LENS, 0, cfg.batch)
        lens = lo + np.floor(u * (hi - lo + 1)).astype(np.int64)
        lens = np.minimum(lens, hi)
    elif kind == "lognormal":
        median, sigma, lo, hi = cfg.lens[1:5]
        z = normals64(cfg.seed, T_LENS, 0, cfg.batch)
        lens = np.rint(median * np.exp(sigma * z)).astype(np.int64)
        lens = np.clip(lens, lo, hi)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def permutation(seed, tensor_id, n):
    """Fisher-Yates shuffle of range(n) driven by the counter-based uniforms."""
    u = uniforms(seed, tensor_id, 0, max(n - 1, 0))
    perm = np.arange(n, dtype=np.int64)
    j = np.floor(u * np.arange(n, 1, -1)).astype(np.int64)  # j_i in [0, i] for i = n-1 .. 1
    for step, i in enumerate(range(n - 1, 0, -1)):
        k = j[step]
        perm[i], perm[k] = perm[k], perm[i]
    return perm


@dataclass
class Inputs:
    cfg: Config
    lens: np.ndarray            # int32 [B]
    block_table: np.ndarray     # int32 [B, bt_stride], -1 past a request's pages
    num_pages: int
    max_len: int
    score_stride: int
    q: np.ndarray               # [B, H, D] float32 or uint16 (bf16 bits)
    kv: np.ndarray              # [num_pages, P, D] float32 / uint16 / uint8
    kv_scale: Optional[np.ndarray]   # float32 [num_pages, P] iff FP8
    q_idx: Optional[np.ndarray] = None   # [B, H_I, d_I] float32 / uint16
    w: Optional[np.ndarray] = None       # float32 [B, H_I]
    k_idx: Optional[np.ndarray] = None   # [num_pages, P, d_I]
    k_idx_scale: Optional[np.ndarray] = None

    @property
    def bt_stride(self):
        return self.block_table.shape[1]


_NP_STORAGE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}


def _dense_rows(cfg_dtype, rows_f32):
    if cfg_dtype == F32:
        return rows_f32
    if cfg_dtype == BF16:
        return to_bf16_bits(rows_f32)
    raise ValueError("queries are fp32 or bf16")


def _fill_pool(cfg, lens, bt, num_pages, dim, tensor_id, dtype, poison_tail, unassigned):
    P = cfg.page_size
    pool = np.empty((num_pages, P, dim), _NP_STORAGE[dtype])
    scale = np.empty((num_pages, P), np.float32) if dtype == FP8 else None
    lib = _load()
    if len(unassigned):
        for pg in unassigned:
            key = stream_key(cfg.seed, T_FILL, (tensor_id << 32) | int(pg))
            lib.spmla_gen_fill_garbage(ctypes.c_uint64(key), P * dim, dtype,
                                       ctypes.c_void_p(pool[pg].ctypes.data), int(poison_tail))
            if scale is not None:
                scale[pg] = np.nan if poison_tail else 1.0
    lens32 = np.ascontiguousarray(lens, np.int32)
    bt32 = np.ascontiguousarray(bt, np.int32)
    rc = lib.spmla_gen_fill_pool(cfg.seed, tensor_id, cfg.batch, _ptr(lens32), P, dim, _ptr(bt32),
                                 bt32.shape[1], dtype, _ptr(pool), _ptr(scale), int(poison_tail))
    if rc != 0:
        raise ValueError("generator: unsupported pool shape")
    return pool, scale


def make_inputs(cfg, poison_tail=False, lens=None, shuffle=True):
    """Draw every input of one workload.  `cfg` is a Config or a key of CONFIGS.

    lens: optional explicit context lengths (overrides the recipe's draw).
    poison_tail: fill cache slots that no token maps to with NaN instead of
    plausible draws (a reader that strays past a context length then shows).
    shuffle: False lays every request's pages out contiguously in order
    (block_table[b][j] = first page of b + j), which lets a check read the
    logical rows straight out of the pool.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    lens = draw_lengths(cfg) if lens is None else np.asarray(lens, np.int32)
    assert lens.shape == (cfg.batch,) and lens.min() >= 0
    P = cfg.page_size
    n_pages = (lens.astype(np.int64) + P - 1) // P
    needed = int(n_pages.sum())
    num_pages = needed if cfg.pool_factor == 1.0 else int(math.ceil(cfg.pool_factor * needed))
    num_pages = max(num_pages, 1)
    perm = permutation(cfg.seed, T_PERM, num_pages) if shuffle else np.arange(num_pages, dtype=np.int64)
    bt_stride = max(int(n_pages.max()), 1)
    bt = np.full((cfg.batch, bt_stride), -1, np.int32)
    off = 0
    for b in range(cfg.batch):
        n = int(n_pages[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    unassigned = np.sort(perm[needed:]) if num_pages > needed else np.array([], np.int64)
    max_len = int(lens.max())
    score_stride = max(64, (max_len + 63) // 64 * 64)

    D = cfg.dim
    q32 = np.empty((cfg.batch, cfg.n_heads, D), np.float32)
    for b in range(cfg.batch):
        q32[b] = normals32(cfg.seed, T_Q, b, cfg.n_heads * D).reshape(cfg.n_heads, D)
    q = _dense_rows(cfg.q_dtype, q32)
    kv, kv_scale = _fill_pool(cfg, lens, bt, num_pages, D, T_KV, cfg.cache_dtype, poison_tail, unassigned)
    inp = Inputs(cfg, lens, bt, num_pages, max_len, score_stride, q, kv, kv_scale)
    if not cfg.dense:
        HI, dI = cfg.idx_heads, cfg.idx_dim
        qi = np.empty((cfg.batch, HI, dI), np.float32)
        w = np.empty((cfg.batch, HI), np.float32)
        for b in range(cfg.batch):
            qi[b] = normals32(cfg.seed, T_QIDX, b, HI * dI).reshape(HI, dI)
            if cfg.w_dist == "normal":
                w[b] = normals32(cfg.seed, T_W, b, HI)
            else:
                w[b] = uniforms(cfg.seed, T_W, b, HI).astype(np.float32)
        inp.q_idx = _dense_rows(cfg.q_dtype, qi)
        inp.w = w
        inp.k_idx, inp.k_idx_scale = _fill_pool(cfg, lens, bt, num_pages, dI, T_KIDX, cfg.idx_dtype,
                                                poison_tail, unassigned)
    return inp


def make_mq_queries(inp, n_q):
    """Queries of n_q new tokens per request for a multi-query step: query
    n_q - 1 (the newest position) is the workload's own q / q_idx / w, the
    earlier ones are drawn from sub-stream b * n_q + i of their own tensor
    ids.  Returns (q [B, n_q, H, D], q_idx [B, n_q, H_I, d_I], w [B, n_q, H_I])
    in the workload's storage types."""
    cfg = inp.cfg
    B, H, D = cfg.batch, cfg.n_heads, cfg.dim
    HI, dI = cfg.idx_heads, cfg.idx_dim
    q = np.empty((B, n_q) + inp.q.shape[1:], inp.q.dtype)
    qi = np.empty((B, n_q) + inp.q_idx.shape[1:], inp.q_idx.dtype)
    w = np.empty((B, n_q, HI), np.float32)
    for b in range(B):
        for i in range(n_q):
            if i == n_q - 1:
                q[b, i], qi[b, i], w[b, i] = inp.q[b], inp.q_idx[b], inp.w[b]
                continue
            sub = b * n_q + i
            q[b, i] = _dense_rows(cfg.q_dtype, normals32(cfg.seed, T_MQ_Q, sub, H * D).reshape(1, H, D))[0]
            qi[b, i] = _dense_rows(cfg.q_dtype, normals32(cfg.seed, T_MQ_QIDX, sub, HI * dI).reshape(1, HI, dI))[0]
            if cfg.w_dist == "normal":
                w[b, i] = normals32(cfg.seed, T_MQ_W, sub, HI)
            else:
                w[b, i] = uniforms(cfg.seed, T_MQ_W, sub, HI).astype(np.float32)
    return q, qi, w


def make_chunk_queries(inp, n_req, n_q):
    """Queries of a prefill chunk: n_q new tokens for each of the first n_req
    requests, query (b, i) from sub-stream b * n_q + i of its own tensor id,
    in the workload's query type.  Returns q [n_req, n_q, H, D]."""
    cfg = inp.cfg
    H, D = cfg.n_heads, cfg.dim
    q = np.empty((n_req, n_q, H, D), np.float32)
    for b in range(n_req):
        for i in range(n_q):
            q[b, i] = normals32(cfg.seed, T_CHUNK_Q, b * n_q + i, H * D).reshape(H, D)
    return _dense_rows(cfg.q_dtype, q.reshape(n_req * n_q, H, D)).reshape(n_req, n_q, H, D)
