"""Python binding of libsparse_mla.so (sparse paged MLA decode for gfx950).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, reads their shapes and pointers, and calls the C entry point
of the same name on the current torch stream.  All arithmetic happens in the
library's HIP kernels; there is no fallback.  If the library is not built
(python -m sparse_paged_mla_amd.build) every call raises.

The C header include/sparse_mla.h documents each operation, its layouts and
its error behaviour.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_mla.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
BAD_PAGE, BAD_LEN, BAD_INDEX, BAD_TAG = 1, 2, 4, 8
STATUS_NAMES = {0: "SPMLA_OK", -1: "SPMLA_EINVAL", -2: "SPMLA_EUNSUPPORTED", -3: "SPMLA_ELAUNCH",
                -4: "SPMLA_EWORKSPACE"}

_lib = None


class SparseMLAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def load_library():
    """Load libsparse_mla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_paged_mla_amd.build`")
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(lib):
    """Set the C signatures of every exported call on a loaded library handle."""
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.dsa_indexer_scores.restype = ctypes.c_int
    lib.dsa_indexer_scores.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, i32, vp, i32, i64, i32, i32, vp, i64,
                                       vp, vp]
    lib.dsa_indexer_scores_mq.restype = ctypes.c_int
    lib.dsa_indexer_scores_mq.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, i32, vp, i32, i64, i32, i32, i32,
                                          vp, i64, vp, vp]
    lib.topk_workspace_bytes.restype = ctypes.c_size_t
    lib.topk_workspace_bytes.argtypes = [i32, i64, i32]
    lib.topk_select.restype = ctypes.c_int
    lib.topk_select.argtypes = [vp, i64, vp, i32, i64, i32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.topk_select_noalloc.restype = ctypes.c_int
    lib.topk_select_noalloc.argtypes = [vp, i64, vp, i32, i64, i32, vp, vp, vp]
    lib.mla_paged_decode.restype = ctypes.c_int
    lib.mla_paged_decode.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, i32, vp, i32, i64, vp, i32, i32, i32, i32,
                                     f32, i32, i32, vp, vp, vp, vp]
    lib.kv_cache_append.restype = ctypes.c_int
    lib.kv_cache_append.argtypes = [vp, i32, i32, i32, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.kv_cache_append_pair.restype = ctypes.c_int
    lib.kv_cache_append_pair.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.kv_page_check.restype = ctypes.c_int
    lib.kv_page_check.argtypes = [vp, vp, i32, vp, i32, i64, vp, i32, i32, vp, vp]
    lib.mq_expand_requests.restype = ctypes.c_int
    lib.mq_expand_requests.argtypes = [vp, i32, vp, i32, i32, vp, vp, vp]
    lib.lse_merge.restype = ctypes.c_int
    lib.lse_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.spmla_last_error.restype = ctypes.c_char_p
    lib.spmla_last_error.argtypes = []
    return lib


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc):
    if rc != 0:
        raise SparseMLAError(rc, load_library().spmla_last_error().decode())


def dsa_indexer_scores(q_idx, weights, k_pool, k_scale, block_table, context_lens, max_len, scores,
                       req_status=None, stream=None):
    """scores[b, t] = sum_h w[b,h] * relu(q_idx[b,h] . key(b,t)) for t < context_lens[b]."""
    lib = load_library()
    B, H, d = q_idx.shape
    num_pages, page_size = k_pool.shape[0], k_pool.shape[1]
    _check(lib.dsa_indexer_scores(_ptr(q_idx), _dtype_code(q_idx), _ptr(weights), _ptr(k_pool), _ptr(k_scale),
                                  _dtype_code(k_pool), num_pages, page_size, _ptr(block_table),
                                  block_table.shape[1], _ptr(context_lens), B, int(max_len), H, d, _ptr(scores),
                                  scores.stride(0), _ptr(req_status), _stream(stream)))


def dsa_indexer_scores_mq(q_idx, weights, k_pool, k_scale, block_table, context_lens, max_len, scores,
                          req_status=None, stream=None):
    """Multi-query indexer: q_idx [B, n_q, H, d], weights [B, n_q, H] -> scores
    [B * n_q, stride] (row b * n_q + i: query i, every t < context_lens[b])."""
    lib = load_library()
    B, n_q, H, d = q_idx.shape
    num_pages, page_size = k_pool.shape[0], k_pool.shape[1]
    _check(lib.dsa_indexer_scores_mq(_ptr(q_idx), _dtype_code(q_idx), _ptr(weights), _ptr(k_pool), _ptr(k_scale),
                                     _dtype_code(k_pool), num_pages, page_size, _ptr(block_table),
                                     block_table.shape[1], _ptr(context_lens), B, int(max_len), n_q, H, d,
                                     _ptr(scores), scores.stride(0), _ptr(req_status), _stream(stream)))


def topk_workspace_bytes(batch, max_len, k):
    return int(load_library().topk_workspace_bytes(int(batch), int(max_len), int(k)))


def topk_select(scores, context_lens, max_len, k, out_idx, workspace, req_status=None, stream=None):
    """out_idx[b] = the min(k, L_b) best-scoring token indices, ascending, -1 padded."""
    lib = load_library()
    B = context_lens.shape[0]
    _check(lib.topk_select(_ptr(scores), scores.stride(0), _ptr(context_lens), B, int(max_len), int(k),
                           _ptr(out_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _ptr(req_status), _stream(stream)))


def topk_select_noalloc(scores, context_lens, max_len, k, out_idx, req_status=None, stream=None):
    """topk_select with the library's static device workspace instead of a caller buffer."""
    lib = load_library()
    B = context_lens.shape[0]
    _check(lib.topk_select_noalloc(_ptr(scores), scores.stride(0), _ptr(context_lens), B, int(max_len), int(k),
                                   _ptr(out_idx), _ptr(req_status), _stream(stream)))


def mla_paged_decode(q, kv_pool, kv_scale, block_table, context_lens, max_len, indices, d_latent, sm_scale,
                     o_part, lse_part, req_status=None, stream=None, split_tokens=0):
    """Split-KV attention over indices[b] (or every token when indices is None).

    o_part [B, S, H, d_latent] and lse_part [B, S, H] fix the number of splits S;
    split_tokens > 0 fixes the split length instead of dividing each request by S."""
    lib = load_library()
    B, H, D = q.shape
    num_pages, page_size = kv_pool.shape[0], kv_pool.shape[1]
    S = o_part.shape[1]
    k = 0 if indices is None else indices.shape[1]
    _check(lib.mla_paged_decode(_ptr(q), _dtype_code(q), _ptr(kv_pool), _ptr(kv_scale), _dtype_code(kv_pool),
                                num_pages, page_size, _ptr(block_table), block_table.shape[1], _ptr(context_lens), B,
                                int(max_len), _ptr(indices), k, H, int(d_latent), D - int(d_latent),
                                float(sm_scale), S, int(split_tokens), _ptr(o_part), _ptr(lse_part), _ptr(req_status),
                                _stream(stream)))


def lse_merge(o_part, lse_part, o, lse, stream=None):
    """o, lse = merge of the split partials o_part [B, S, H, d], lse_part [B, S, H]."""
    lib = load_library()
    B, S, H, d = o_part.shape
    _check(lib.lse_merge(_ptr(o_part), _ptr(lse_part), B, S, H, d, _ptr(o), _ptr(lse), _stream(stream)))


def kv_cache_append(rows, pool, pool_scale, block_table, positions, req_status=None, stream=None):
    """Write rows[b] ([B, dim] fp32/bf16) to slot positions[b] of request b in
    pool ([num_pages, P, dim] fp32/bf16/FP8; FP8 quantises with a per-token
    scale written to pool_scale [num_pages, P])."""
    lib = load_library()
    B, dim = rows.shape
    num_pages, page_size = pool.shape[0], pool.shape[1]
    if pool.shape[2] != dim:
        raise ValueError("pool row length differs from the rows'")
    _check(lib.kv_cache_append(_ptr(rows), _dtype_code(rows), B, dim, _ptr(pool), _ptr(pool_scale),
                               _dtype_code(pool), num_pages, page_size, _ptr(block_table), block_table.shape[1],
                               _ptr(positions), _ptr(req_status), _stream(stream)))


def kv_page_check(block_table, bt_tags, context_lens, max_len, page_tags, page_size, req_status, stream=None):
    """OR BAD_PAGE / BAD_TAG / BAD_LEN into req_status for every request whose
    covered block-table entries have a bad page id or a tag (int64 [B,
    bt_stride], the page's tag when it was given out) other than the page's
    current tag (page_tags int64 [num_pages])."""
    lib = load_library()
    B = context_lens.shape[0]
    if bt_tags.shape != block_table.shape:
        raise ValueError("bt_tags must have the block table's shape")
    _check(lib.kv_page_check(_ptr(block_table), _ptr(bt_tags), block_table.shape[1], _ptr(context_lens), B,
                             int(max_len), _ptr(page_tags), page_tags.shape[0], int(page_size), _ptr(req_status),
                             _stream(stream)))


def mq_expand_requests(block_table, context_lens, n_q, out_block_table, out_lens, stream=None):
    """Expanded batch of a multi-query step: request b * n_q + i is query i of
    request b (same block-table row, length L_b - n_q + 1 + i)."""
    lib = load_library()
    B = context_lens.shape[0]
    if out_block_table.shape != (B * n_q, block_table.shape[1]) or out_lens.shape != (B * n_q,):
        raise ValueError("output shapes must be [B * n_q, bt_stride] and [B * n_q]")
    _check(lib.mq_expand_requests(_ptr(block_table), block_table.shape[1], _ptr(context_lens), B, int(n_q),
                                  _ptr(out_block_table), _ptr(out_lens), _stream(stream)))


def kv_cache_append_pair(kv_rows, kv_pool, kv_scale, idx_rows, idx_pool, idx_scale, block_table, positions,
                         req_status=None, stream=None):
    """kv_cache_append of the latent rows and the indexer keys of the same new
    tokens in one launch (the pools share page ids)."""
    lib = load_library()
    B = kv_rows.shape[0]
    if idx_rows.shape[0] != B or _dtype_code(kv_rows) != _dtype_code(idx_rows):
        raise ValueError("both row arrays need the same batch and dtype")
    if _dtype_code(kv_pool) != _dtype_code(idx_pool) or kv_pool.shape[:2] != idx_pool.shape[:2]:
        raise ValueError("both pools need the same dtype, page count and page size")
    if kv_pool.shape[2] != kv_rows.shape[1] or idx_pool.shape[2] != idx_rows.shape[1]:
        raise ValueError("pool row lengths differ from the rows'")
    _check(lib.kv_cache_append_pair(_ptr(kv_rows), kv_rows.shape[1], _ptr(kv_pool), _ptr(kv_scale), _ptr(idx_rows),
                                    idx_rows.shape[1], _ptr(idx_pool), _ptr(idx_scale), _dtype_code(kv_rows),
                                    _dtype_code(kv_pool), B, kv_pool.shape[0], kv_pool.shape[1], _ptr(block_table),
                                    block_table.shape[1], _ptr(positions), _ptr(req_status), _stream(stream)))
