"""ctypes binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the bench's CPU
baseline may import this package.  It shares no code with the HIP library.

Storage formats are taken from the numpy dtype of each array: float32 is
fp32, uint16 is bf16 bit patterns, uint8 is FP8 e4m3fn codes (which then need
an fp32 per-token scale array).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPMLA_ORACLE_LIB names another build of oracle.c (the sanitizer test's).
_LIB_PATH = os.environ.get("SPMLA_ORACLE_LIB") or os.path.join(_HERE, "liboracle_spmla.so")
_lib = None

BAD_PAGE, BAD_LEN, BAD_INDEX, BAD_TAG = 1, 2, 4, 8


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_fp8_e4m3_value.restype = d
    lib.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_value.restype = d
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_fp8_e4m3_encode_array.restype = None
    lib.oracle_fp8_e4m3_encode_array.argtypes = [vp, i64, vp]
    lib.oracle_bf16_encode_array.restype = None
    lib.oracle_bf16_encode_array.argtypes = [vp, i64, vp]
    lib.oracle_page_check.restype = ctypes.c_int
    lib.oracle_page_check.argtypes = [vp, vp, i32, vp, i32, i64, vp, i32, i32, vp]
    lib.oracle_cache_append.restype = ctypes.c_int
    lib.oracle_cache_append.argtypes = [vp, ctypes.c_int, i32, i32, vp, vp, ctypes.c_int, i32, i32, vp, i32, vp, vp]
    lib.oracle_indexer_scores.restype = ctypes.c_int
    lib.oracle_indexer_scores.argtypes = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i32, i32, vp, i32, vp, i32,
                                          i64, i32, i32, vp, vp, i64, vp]
    lib.oracle_indexer_scores_at.restype = ctypes.c_int
    lib.oracle_indexer_scores_at.argtypes = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i32, i32, vp, i32, i32, i32,
                                             vp, vp, i64, vp, vp]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [vp, i64, vp, i32, i32, vp]
    lib.oracle_mla_attention.restype = ctypes.c_int
    lib.oracle_mla_attention.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, i32, i32, vp, i32, vp, i32, i64,
                                         vp, i32, i32, i32, i32, d, vp, vp, vp]
    lib.oracle_lse_merge.restype = ctypes.c_int
    lib.oracle_lse_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    lib.oracle_kv_bytes_per_token.restype = d
    lib.oracle_kv_bytes_per_token.argtypes = [i32, i32, i32, d]
    lib.oracle_mla_bytes_per_token.restype = d
    lib.oracle_mla_bytes_per_token.argtypes = [i32, i32, d, d]
    _lib = lib
    return lib


_FMT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.uint8): 2}


def _fmt(a):
    return _FMT[np.asarray(a).dtype]


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype))
    return a


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def fp8_e4m3_value(code):
    return _load().oracle_fp8_e4m3_value(int(code))


def bf16_value(bits):
    return _load().oracle_bf16_value(int(bits))


def indexer_scores(q_idx, w, k_pool, k_scale, block_table, lens, max_len=None, score_stride=None):
    """fp64 scores [B, score_stride] (NaN-free only where t < lens[b]), magnitudes, status."""
    q_idx, w = _c(q_idx), _c(w, np.float32)
    k_pool, k_scale = _c(k_pool), _c(k_scale, np.float32)
    bt, lens = _c(block_table, np.int32), _c(lens, np.int32)
    B, H, d = q_idx.shape
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    max_len = int(lens.max()) if max_len is None else int(max_len)
    stride = max(int(lens.max()), 1) if score_stride is None else int(score_stride)
    scores = np.full((B, stride), np.nan)
    mags = np.full((B, stride), np.nan)
    status = np.zeros(B, np.int32)
    rc = _load().oracle_indexer_scores(_p(q_idx), _fmt(q_idx), _p(w), _p(k_pool), _p(k_scale), _fmt(k_pool),
                                       num_pages, P, _p(bt), bt.shape[1], _p(lens), B, max_len, H, d,
                                       _p(scores), _p(mags), stride, _p(status))
    assert rc == 0
    return scores, mags, status


def indexer_scores_at(q_idx, w, k_pool, k_scale, block_table, sample_b, sample_t):
    """fp64 scores and magnitudes at sampled (request, token) positions."""
    q_idx, w = _c(q_idx), _c(w, np.float32)
    k_pool, k_scale = _c(k_pool), _c(k_scale, np.float32)
    bt = _c(block_table, np.int32)
    sb, st = _c(sample_b, np.int32), _c(sample_t, np.int64)
    B, H, d = q_idx.shape
    n = sb.shape[0]
    s = np.empty(n)
    a = np.empty(n)
    rc = _load().oracle_indexer_scores_at(_p(q_idx), _fmt(q_idx), _p(w), _p(k_pool), _p(k_scale), _fmt(k_pool),
                                          k_pool.shape[0], k_pool.shape[1], _p(bt), bt.shape[1], H, d,
                                          _p(sb), _p(st), n, _p(s), _p(a))
    assert rc == 0
    return s, a


def topk(scores, lens, k):
    """Indices [B, k] ascending, -1 padded; scores may be any float array [B, stride]."""
    sc = _c(scores, np.float64)
    lens = _c(lens, np.int32)
    B = sc.shape[0]
    out = np.empty((B, k), np.int32)
    rc = _load().oracle_topk(_p(sc), sc.shape[1], _p(lens), B, k, _p(out))
    assert rc == 0
    return out


def mla_attention(q, kv, kv_scale, block_table, lens, indices, n_heads, d_latent, d_rope, sm_scale,
                  max_len=None):
    """fp64 o [B, H, d_latent], lse [B, H], status [B]; indices None = every token t < L_b."""
    q, kv, kv_scale = _c(q), _c(kv), _c(kv_scale, np.float32)
    bt, lens = _c(block_table, np.int32), _c(lens, np.int32)
    idx = _c(indices, np.int32)
    B = q.shape[0]
    k = 0 if idx is None else idx.shape[1]
    max_len = int(lens.max()) if max_len is None else int(max_len)
    o = np.empty((B, n_heads, d_latent))
    lse = np.empty((B, n_heads))
    status = np.zeros(B, np.int32)
    rc = _load().oracle_mla_attention(_p(q), _fmt(q), _p(kv), _p(kv_scale), _fmt(kv), kv.shape[0], kv.shape[1],
                                      _p(bt), bt.shape[1], _p(lens), B, max_len, _p(idx), k,
                                      n_heads, d_latent, d_rope, float(sm_scale), _p(o), _p(lse), _p(status))
    assert rc == 0
    return o, lse, status


def lse_merge(o_part, lse_part):
    """Merge partials o_part [B, S, H, d], lse_part [B, S, H] -> o [B, H, d], lse [B, H] (fp64)."""
    op = _c(o_part, np.float64)
    lp = _c(lse_part, np.float64)
    B, S, H, d = op.shape
    o = np.empty((B, H, d))
    lse = np.empty((B, H))
    rc = _load().oracle_lse_merge(_p(op), _p(lp), B, S, H, d, _p(o), _p(lse))
    assert rc == 0
    return o, lse


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem):
    return _load().oracle_kv_bytes_per_token(layers, kv_heads, head_dim, float(bytes_per_elem))


def mla_bytes_per_token(d_latent, d_rope, bytes_per_elem, scale_bytes=0.0):
    return _load().oracle_mla_bytes_per_token(d_latent, d_rope, float(bytes_per_elem), float(scale_bytes))


def decode_step(inp, k=None, splits=None):
    """Whole step on one generator `Inputs`: indexer -> top-k -> attention (fp64).

    Returns dict(scores, idx, o, lse, status).  Dense workloads (no indexer)
    attend every token."""
    cfg = inp.cfg
    out = {}
    if cfg.dense:
        idx = None
    else:
        scores, _, st = indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table, inp.lens,
                                       score_stride=inp.score_stride)
        idx = topk(scores, inp.lens, cfg.topk if k is None else k)
        out["scores"] = scores
        out["idx"] = idx
    o, lse, st = mla_attention(inp.q, inp.kv, inp.kv_scale, inp.block_table, inp.lens, idx, cfg.n_heads,
                               cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    out.update(o=o, lse=lse, status=st)
    return out


def fp8_e4m3_encode(q):
    """float32 array -> uint8 e4m3fn codes (nearest, ties to even, saturating)."""
    q = np.ascontiguousarray(q, np.float32)
    out = np.empty(q.shape, np.uint8)
    _load().oracle_fp8_e4m3_encode_array(_p(q), q.size, _p(out))
    return out


def bf16_encode(x):
    """float32 array -> uint16 bf16 bit patterns (nearest, ties to even)."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_bf16_encode_array(_p(x), x.size, _p(out))
    return out


def cache_append(rows, pool, pool_scale, block_table, positions):
    """Write row b of `rows` ([B, dim] float32, or uint16 bf16 bits) to slot
    positions[b] of request b in `pool` ([num_pages, P, dim] float32 / uint16
    bf16 / uint8 FP8 codes, with `pool_scale` [num_pages, P] float32 when FP8),
    in place.  Returns the per-request status bits."""
    rows = np.ascontiguousarray(rows)
    B, dim = rows.shape
    assert pool.flags.c_contiguous and pool.shape[2] == dim
    num_pages, P = pool.shape[0], pool.shape[1]
    pdt = _fmt(pool)
    if pdt == 2:
        assert pool_scale is not None and pool_scale.flags.c_contiguous and pool_scale.dtype == np.float32
    bt = _c(block_table, np.int32)
    pos = _c(positions, np.int32)
    status = np.zeros(B, np.int32)
    rc = _load().oracle_cache_append(_p(rows), _fmt(rows), B, dim, _p(pool), _p(pool_scale) if pdt == 2 else None,
                                     pdt, num_pages, P, _p(bt), bt.shape[1], _p(pos), _p(status))
    assert rc == 0
    return status


def page_check(block_table, bt_tags, lens, page_tags, page_size, max_len=None):
    """Per-request status bits of the page-integrity check (BAD_LEN, BAD_PAGE, BAD_TAG)."""
    bt = _c(block_table, np.int32)
    tags = _c(bt_tags, np.uint64)
    assert tags.shape == bt.shape
    lens = _c(lens, np.int32)
    pt = _c(page_tags, np.uint64)
    B = lens.shape[0]
    max_len = int(lens.max()) if max_len is None and B else int(max_len or 0)
    status = np.zeros(B, np.int32)
    assert _load().oracle_page_check(_p(bt), _p(tags), bt.shape[1], _p(lens), B, max_len, _p(pt), pt.shape[0],
                                     int(page_size), _p(status)) == 0
    return status


def multi_query_step(q, q_idx, w, kv, kv_scale, k_pool, k_scale, block_table, lens, k, n_heads, d_latent, d_rope,
                     sm_scale, score_stride=None):
    """Multi-query verification step [EG, "Speculative Decoding"; KW 5.3].

    Q new tokens per request are already in the cache, at positions
    L-Q .. L-1.  Query i has the causal limit L - Q + 1 + i (it sees itself
    and every earlier token), and gets its own indexer scores, its own top-k
    over that limit and its own attention over the selected tokens.

    q [B, Q, H, D], q_idx [B, Q, H_I, d_I], w [B, Q, H_I]; a request with
    L < Q is flagged BAD_LEN and its outputs are NaN.  Returns dict(scores
    [B, Q, stride], idx [B, Q, k], o [B, Q, H, d_latent], lse [B, Q, H],
    status [B], vis [B, Q])."""
    B, Q = q.shape[0], q.shape[1]
    lens = np.asarray(lens, np.int64)
    bad = lens < Q
    vis = np.where(bad[:, None], 0, lens[:, None] - Q + 1 + np.arange(Q)[None, :]).astype(np.int32)
    stride = max(int(lens.max()), 1) if score_stride is None else int(score_stride)
    scores = np.full((B, Q, stride), np.nan)
    idx = np.full((B, Q, k), -1, np.int32)
    o = np.full((B, Q, n_heads, d_latent), np.nan)
    lse = np.full((B, Q, n_heads), np.nan)
    status = np.where(bad, BAD_LEN, 0).astype(np.int32)
    ok = ~bad
    if ok.any():
        for i in range(Q):
            s, _, st = indexer_scores(q_idx[ok, i], w[ok, i], k_pool, k_scale, block_table[ok], vis[ok, i],
                                      max_len=int(lens.max()), score_stride=stride)
            sel = topk(s, vis[ok, i], k)
            oi, li, st2 = mla_attention(q[ok, i], kv, kv_scale, block_table[ok], vis[ok, i], sel, n_heads, d_latent,
                                        d_rope, sm_scale, max_len=int(lens.max()))
            scores[ok, i], idx[ok, i], o[ok, i], lse[ok, i] = s, sel, oi, li
            status[ok] |= st | st2
    return dict(scores=scores, idx=idx, o=o, lse=lse, status=status, vis=vis)


def prefill_chunk_attention(q, kv, kv_scale, block_table, lens, n_heads, d_latent, d_rope, sm_scale, blocks=None):
    """Dense causal attention of n_q new tokens per request (positions
    L-n_q .. L-1, already cached): query i attends to every t < L - n_q + 1 + i.
    With `blocks`, the context of each query is cut into that many equal
    blocks, each attended alone, and the block partials are merged with the
    online-softmax state, as a ring pass computes it block by block [KW
    5.2.2]; without, in one piece.  Returns o [B, n_q, H, d_latent], lse
    [B, n_q, H], status [B]."""
    B, Q = q.shape[0], q.shape[1]
    lens = np.asarray(lens, np.int64)
    bad = lens < Q
    o = np.full((B, Q, n_heads, d_latent), np.nan)
    lse = np.full((B, Q, n_heads), np.nan)
    status = np.where(bad, BAD_LEN, 0).astype(np.int32)
    ok = np.nonzero(~bad)[0]
    for i in range(Q):
        for b in ok:
            vis = int(lens[b] - Q + 1 + i)
            if blocks is None:
                oi, li, st = mla_attention(q[b:b + 1, i], kv, kv_scale, block_table[b:b + 1], [vis], None, n_heads,
                                           d_latent, d_rope, sm_scale, max_len=int(lens.max()))
            else:
                edges = [vis * j // blocks for j in range(blocks + 1)]
                parts = [mla_attention(q[b:b + 1, i], kv, kv_scale, block_table[b:b + 1], [vis],
                                       np.arange(edges[j], edges[j + 1], dtype=np.int32)[None, :]
                                       if edges[j + 1] > edges[j] else np.full((1, 1), -1, np.int32),
                                       n_heads, d_latent, d_rope, sm_scale, max_len=int(lens.max()))
                         for j in range(blocks)]
                oi, li = lse_merge(np.stack([p[0] for p in parts], 1), np.stack([p[1] for p in parts], 1))
                st = np.zeros(1, np.int32)
                for p in parts:
                    st |= p[2]
            o[b, i], lse[b, i] = oi[0], li[0]
            status[b] |= st[0]
    return o, lse, status
