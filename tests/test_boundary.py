"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host with the documented
status codes before anything is enqueued (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")
LIB = os.path.join(ROOT, "sparse_paged_mla_amd", "libsparse_mla.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EWORKSPACE = 0, -1, -2, -3, -4
F32, BF16, FP8 = 0, 1, 2


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)))


# SPMLA_BOUNDARY_LIB names a host-only build of the same validation layer
# with the launchers stubbed out (the sanitizer test's); it also exports
# spmla_stub_launches(), the number of calls that got past validation.
STUB_LIB = os.environ.get("SPMLA_BOUNDARY_LIB")


@pytest.fixture(scope="module")
def lib():
    import sparse_paged_mla_amd as spm
    if STUB_LIB:
        return spm.declare(ctypes.CDLL(STUB_LIB))
    if not os.path.exists(LIB):
        pytest.fail("libsparse_mla.so is not built (run __graft_entry__.build())")
    return spm.load_library()


def test_header_declares_the_four_operations():
    names = _declared()
    for n in ("dsa_indexer_scores", "topk_select", "mla_paged_decode", "lse_merge", "topk_workspace_bytes",
              "kv_cache_append", "kv_cache_append_pair", "kv_page_check", "mq_expand_requests", "spmla_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), f"{n} not exported"


def _launches(lib):
    f = lib.spmla_stub_launches
    f.restype = ctypes.c_int
    return f()


def test_product_never_loads_the_oracle():
    for dirpath, _, files in os.walk(os.path.join(ROOT, "sparse_paged_mla_amd")):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f), errors="ignore").read()
                assert "oracle" not in text.replace("oracle-free", ""), f"{f} mentions the oracle"


FAKE = ctypes.c_void_p(0x1000)   # a non-null 16-byte-aligned value; never dereferenced by rejected calls
MIS = ctypes.c_void_p(0x1004)    # misaligned


def _idx(lib, **kw):
    a = dict(q_idx=FAKE, q_dtype=BF16, w=FAKE, k_pool=FAKE, k_scale=FAKE, k_dtype=FP8, num_pages=10, page_size=64,
             bt=FAKE, bt_stride=4, lens=FAKE, batch=2, max_len=256, n_heads=64, d=128, scores=FAKE,
             score_stride=256, status=None, stream=None)
    a.update(kw)
    return lib.dsa_indexer_scores(*a.values())


def _dec(lib, **kw):
    a = dict(q=FAKE, q_dtype=BF16, kv=FAKE, kv_scale=FAKE, kv_dtype=FP8, num_pages=10, page_size=64, bt=FAKE,
             bt_stride=4, lens=FAKE, batch=2, max_len=256, indices=FAKE, k=2048, n_heads=128, d_latent=512,
             d_rope=64, sm_scale=1 / 24, splits=1, split_tokens=0, o_part=FAKE, lse_part=FAKE, status=None,
             stream=None)
    a.update(kw)
    return lib.mla_paged_decode(*a.values())


def test_indexer_rejects(lib):
    assert _idx(lib, page_size=48) == EUNSUPPORTED
    assert _idx(lib, q_dtype=FP8) == EUNSUPPORTED
    assert _idx(lib, q_dtype=BF16, k_dtype=F32) == EUNSUPPORTED
    assert _idx(lib, k_dtype=7) == EINVAL
    assert _idx(lib, n_heads=129) == EUNSUPPORTED
    assert _idx(lib, d=96) == EUNSUPPORTED
    assert _idx(lib, q_dtype=BF16, d=16) == EUNSUPPORTED
    assert _idx(lib, score_stride=255) == EINVAL
    assert b"score_stride" in lib.spmla_last_error()
    assert _idx(lib, q_idx=None) == EINVAL
    assert _idx(lib, k_scale=None) == EINVAL
    assert _idx(lib, k_pool=MIS) == EINVAL
    assert _idx(lib, batch=-1) == EINVAL
    assert _idx(lib, num_pages=0) == EINVAL
    assert _idx(lib, max_len=-5) == EINVAL
    assert _idx(lib, batch=0, q_idx=None, scores=None) == OK  # empty batch: nothing to do
    assert _idx(lib, score_stride=258) == EINVAL              # rows not 16-byte aligned
    assert _idx(lib, scores=MIS) == EINVAL


def test_topk_rejects(lib):
    lib.topk_workspace_bytes.restype = ctypes.c_size_t
    need = lib.topk_workspace_bytes(4, 1000, 2048)
    assert need >= 4 * 1000 * 8
    assert lib.topk_workspace_bytes(4, 1000, 5000) == 0
    assert lib.topk_workspace_bytes(-1, 1000, 8) == 0
    f = lib.topk_select
    assert f(FAKE, 1000, FAKE, 4, 1000, 0, FAKE, FAKE, need, None, None) == EUNSUPPORTED
    assert f(FAKE, 1000, FAKE, 4, 1000, 4097, FAKE, FAKE, need, None, None) == EUNSUPPORTED
    assert f(FAKE, 999, FAKE, 4, 1000, 2048, FAKE, FAKE, need, None, None) == EINVAL
    assert f(FAKE, 1000, FAKE, 4, 1000, 2048, FAKE, FAKE, need - 1, None, None) == EWORKSPACE
    assert f(FAKE, 1000, FAKE, 4, 1000, 2048, FAKE, None, need, None, None) == EWORKSPACE
    assert f(FAKE, 1000, FAKE, 4, 1000, 2048, FAKE, ctypes.c_void_p(0x1010), need, None, None) == EINVAL
    assert f(None, 1000, FAKE, 4, 1000, 2048, FAKE, FAKE, need, None, None) == EINVAL
    assert f(FAKE, 1000, FAKE, 4, 1000, 2048, FAKE, FAKE, 0, None, None) == EWORKSPACE
    assert b"workspace" in lib.spmla_last_error()
    assert f(None, 1000, None, 0, 1000, 2048, None, None, 0, None, None) == OK


def test_topk_noalloc_rejects(lib):
    """The static-workspace form checks the same arguments, and sizes whose
    workspace exceeds its 32 MiB array, before any HIP call."""
    f = lib.topk_select_noalloc
    assert f(FAKE, 1000, FAKE, 4, 1000, 0, FAKE, None, None) == EUNSUPPORTED
    assert f(FAKE, 1000, FAKE, 4, 1000, 4097, FAKE, None, None) == EUNSUPPORTED
    assert f(FAKE, 999, FAKE, 4, 1000, 2048, FAKE, None, None) == EINVAL
    assert f(None, 1000, FAKE, 4, 1000, 2048, FAKE, None, None) == EINVAL
    assert f(FAKE, 1000, FAKE, -1, 1000, 2048, FAKE, None, None) == EINVAL
    assert f(None, 1000, None, 0, 1000, 2048, None, None, None) == OK
    big = 1 << 20
    assert lib.topk_workspace_bytes(1024, big, 2048) > 32 << 20
    assert f(FAKE, big, FAKE, 1024, big, 2048, FAKE, None, None) == EWORKSPACE
    assert b"static scratch" in lib.spmla_last_error()


def test_decode_rejects(lib):
    lib.mla_paged_decode.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert _dec(lib, d_latent=260) == EUNSUPPORTED          # widths must be multiples of 8
    assert _dec(lib, d_rope=12) == EUNSUPPORTED
    assert _dec(lib, d_latent=0) == EINVAL
    assert _dec(lib, d_latent=1024, d_rope=8) == EUNSUPPORTED  # latent + rope <= 1024
    assert _dec(lib, q_dtype=FP8) == EUNSUPPORTED
    assert _dec(lib, kv_dtype=F32) == EUNSUPPORTED          # bf16 queries need a bf16/FP8 cache
    assert _dec(lib, splits=0) == EUNSUPPORTED
    assert _dec(lib, splits=65) == EUNSUPPORTED
    assert _dec(lib, split_tokens=-32) == EINVAL
    assert _dec(lib, split_tokens=48) == EINVAL             # a split length is whole 32-token tiles
    assert _dec(lib, sm_scale=0.0) == EINVAL
    assert _dec(lib, sm_scale=float("nan")) == EINVAL
    assert _dec(lib, n_heads=0) == EUNSUPPORTED
    assert _dec(lib, k=70000) == EUNSUPPORTED
    assert _dec(lib, kv_scale=None) == EINVAL
    assert _dec(lib, o_part=None) == EINVAL
    assert _dec(lib, q=MIS) == EINVAL
    assert _dec(lib, page_size=8) == EUNSUPPORTED
    assert _dec(lib, bt=None) == EINVAL
    assert _dec(lib, batch=0) == OK


def test_merge_rejects(lib):
    f = lib.lse_merge
    assert f(FAKE, FAKE, 2, 0, 4, 512, FAKE, FAKE, None) == EUNSUPPORTED
    assert f(FAKE, FAKE, 2, 65, 4, 512, FAKE, FAKE, None) == EUNSUPPORTED
    assert f(FAKE, FAKE, 2, 4, 4, 510, FAKE, FAKE, None) == EUNSUPPORTED
    assert f(None, FAKE, 2, 4, 4, 512, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, FAKE, 2, 4, 4, 512, MIS, FAKE, None) == EINVAL
    assert f(FAKE, FAKE, -2, 4, 4, 512, FAKE, FAKE, None) == EINVAL
    assert f(None, None, 0, 4, 4, 512, None, None, None) == OK


def _app(lib, rows=FAKE, row_dtype=1, batch=4, dim=576, pool=FAKE, scale=FAKE, pool_dtype=2, num_pages=10, P=64,
         bt=FAKE, bt_stride=4, pos=FAKE):
    return lib.kv_cache_append(rows, row_dtype, batch, dim, pool, scale, pool_dtype, num_pages, P, bt, bt_stride, pos,
                               None, None)


def test_append_rejects(lib):
    assert _app(lib, row_dtype=2) == EUNSUPPORTED      # FP8 rows in
    assert _app(lib, pool_dtype=3) == EINVAL
    assert _app(lib, dim=20) == EUNSUPPORTED
    assert _app(lib, dim=4104) == EUNSUPPORTED
    assert _app(lib, P=48) == EUNSUPPORTED
    assert _app(lib, num_pages=0) == EINVAL
    assert _app(lib, bt_stride=0) == EINVAL
    assert _app(lib, batch=-1) == EINVAL
    assert _app(lib, scale=None) == EINVAL             # an FP8 pool needs its scales
    assert _app(lib, rows=None) == EINVAL
    assert _app(lib, pos=None) == EINVAL
    assert _app(lib, pool=MIS) == EINVAL
    assert "16-byte" in lib.spmla_last_error().decode()
    assert _app(lib, batch=0, rows=None, pool=None, bt=None, pos=None) == OK


def test_page_check_rejects(lib):
    f = lib.kv_page_check
    assert f(FAKE, FAKE, 4, FAKE, 2, 100, FAKE, 10, 48, FAKE, None) == EUNSUPPORTED
    assert f(FAKE, FAKE, 0, FAKE, 2, 100, FAKE, 10, 64, FAKE, None) == EINVAL
    assert f(FAKE, FAKE, 4, FAKE, 2, 100, FAKE, 0, 64, FAKE, None) == EINVAL
    assert f(FAKE, None, 4, FAKE, 2, 100, FAKE, 10, 64, FAKE, None) == EINVAL
    assert f(FAKE, FAKE, 4, FAKE, 2, 100, None, 10, 64, FAKE, None) == EINVAL
    assert f(FAKE, FAKE, 4, FAKE, 2, 100, FAKE, 10, 64, None, None) == EINVAL   # status is the output
    assert f(FAKE, MIS, 4, FAKE, 2, 100, FAKE, 10, 64, FAKE, None) == EINVAL
    assert f(None, None, 4, None, 0, 0, None, 10, 64, None, None) == OK


def test_mq_expand_rejects(lib):
    f = lib.mq_expand_requests
    assert f(FAKE, 4, FAKE, 2, 0, FAKE, FAKE, None) == EUNSUPPORTED
    assert f(FAKE, 4, FAKE, 2, 65537, FAKE, FAKE, None) == EUNSUPPORTED
    assert f(FAKE, 0, FAKE, 2, 2, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, FAKE, -1, 2, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, FAKE, 2, 2, None, FAKE, None) == EINVAL
    assert f(None, 4, None, 0, 2, None, None, None) == OK


def test_indexer_mq_rejects(lib):
    f = lib.dsa_indexer_scores_mq

    def call(n_q=2, n_heads=64, q_dtype=BF16, d=128, score_stride=256, scores=FAKE):
        return f(FAKE, q_dtype, FAKE, FAKE, FAKE, FP8, 10, 64, FAKE, 4, FAKE, 2, 256, n_q, n_heads, d, scores,
                 score_stride, None, None)
    assert call(n_q=3) == EUNSUPPORTED
    assert call(n_q=0) == EUNSUPPORTED
    assert call(n_heads=48) == EUNSUPPORTED
    assert call(q_dtype=F32) == EUNSUPPORTED
    assert call(d=96) == EUNSUPPORTED
    assert call(score_stride=258) == EINVAL
    assert call(scores=MIS) == EINVAL


def test_append_pair_rejects(lib):
    f = lib.kv_cache_append_pair

    def call(kv_dim=576, idx_dim=128, kv_scale=FAKE, idx_rows=FAKE, idx_pool=FAKE, row_dtype=1, pool_dtype=2, P=64):
        return f(FAKE, kv_dim, FAKE, kv_scale, idx_rows, idx_dim, idx_pool, FAKE, row_dtype, pool_dtype, 4, 10, P,
                 FAKE, 4, FAKE, None, None)
    assert call(idx_dim=12) == EUNSUPPORTED
    assert call(kv_dim=4104) == EUNSUPPORTED
    assert call(row_dtype=2) == EUNSUPPORTED
    assert call(P=48) == EUNSUPPORTED
    assert call(kv_scale=None) == EINVAL
    assert call(idx_rows=None) == EINVAL
    assert call(idx_pool=MIS) == EINVAL


@pytest.mark.skipif(not STUB_LIB, reason="needs the host-only build with stubbed launchers")
def test_valid_calls_reach_the_launcher_and_rejected_ones_do_not(lib):
    """With the launchers stubbed, every call that passes validation reaches
    its launcher exactly once and every rejected call reaches none."""
    n0 = _launches(lib)
    assert _idx(lib) == OK
    assert _dec(lib) == OK
    assert lib.lse_merge(FAKE, FAKE, 2, 4, 4, 512, FAKE, FAKE, None) == OK
    assert _app(lib) == OK
    assert lib.kv_page_check(FAKE, FAKE, 4, FAKE, 2, 100, FAKE, 10, 64, FAKE, None) == OK
    assert lib.mq_expand_requests(FAKE, 4, FAKE, 2, 2, FAKE, FAKE, None) == OK
    need = lib.topk_workspace_bytes(4, 100000, 2048)
    assert lib.topk_select(FAKE, 100000, FAKE, 4, 100000, 2048, FAKE, ctypes.c_void_p(0x100000), need, None,
                           None) == OK
    assert lib.topk_select_noalloc(FAKE, 100000, FAKE, 4, 100000, 2048, FAKE, None, None) == OK
    assert lib.spmla_last_error() == b""
    assert _launches(lib) == n0 + 8
    assert _idx(lib, d=96) == EUNSUPPORTED
    assert _dec(lib, splits=0) == EUNSUPPORTED
    assert lib.topk_select(FAKE, 100000, FAKE, 4, 100000, 2048, FAKE, ctypes.c_void_p(0x100000), need - 1, None,
                           None) == EWORKSPACE
    assert lib.topk_select_noalloc(FAKE, 1 << 20, FAKE, 1024, 1 << 20, 2048, FAKE, None, None) == EWORKSPACE
    assert _launches(lib) == n0 + 8
