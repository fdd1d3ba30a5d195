"""GPU parity of the multi-query verification step (n_q new tokens per
request, causal per query) against the oracle, stage by stage."""
import numpy as np
import pytest
import torch

import oracle
import spmla_gen as gen
from spmla_gen.torch_io import device_batch, tensor
from tests import parity

pytestmark = pytest.mark.gpu


def _lib():
    import sparse_paged_mla_amd as spm
    spm.load_library()
    return spm


def _run_mq(cfg, lens, n_q, splits):
    from sparse_paged_mla_amd.step import MultiQueryStep
    inp = gen.make_inputs(cfg, lens=lens)
    q, qi, w = gen.make_mq_queries(inp, n_q)
    db = device_batch(inp)
    st = MultiQueryStep(db, tensor(q, "cuda"), tensor(qi, "cuda"), torch.from_numpy(w).cuda(), num_splits=splits)
    st.run()
    torch.cuda.synchronize()
    return inp, q, qi, w, st


def _check(cfg, lens, n_q, splits, what):
    print(f"[mq] {what} lens={lens} n_q={n_q} splits={splits}", flush=True)
    inp, q, qi, w, st = _run_mq(cfg, lens, n_q, splits)
    B = cfg.batch
    lens = np.asarray(lens)
    vis = np.where(lens[:, None] >= n_q, lens[:, None] - n_q + 1 + np.arange(n_q)[None, :], -1)
    np.testing.assert_array_equal(st.lens.cpu().numpy().reshape(B, n_q), vis)
    np.testing.assert_array_equal(st.bt.cpu().numpy(), np.repeat(inp.block_table, n_q, axis=0))
    status = st.status.cpu().numpy()
    assert not status[lens >= n_q].any()
    assert (status[lens < n_q] & oracle.BAD_LEN).all()
    ok = lens >= n_q
    s_gpu = st.scores.cpu().numpy()
    idx = st.idx.cpu().numpy()
    o, lse = st.o.cpu().numpy(), st.lse.cpu().numpy()
    for i in range(n_q):
        sub = np.nonzero(ok)[0]
        vi = vis[sub, i].astype(np.int32)
        s_ref, mags, _ = oracle.indexer_scores(qi[sub, i], w[sub, i], inp.k_idx, inp.k_idx_scale,
                                               inp.block_table[sub], vi, max_len=inp.max_len,
                                               score_stride=inp.score_stride)
        for r, b in enumerate(sub):
            parity.check_scores(s_gpu[b, i, :vi[r]], s_ref[r, :vi[r]], mags[r, :vi[r]], f"{what} scores b={b} q={i}")
        parity.check_topk_exact(idx[sub, i], s_gpu[sub, i], vi, cfg.topk, f"{what} q={i}")
        o_ref, lse_ref, st_ref = oracle.mla_attention(q[sub, i], inp.kv, inp.kv_scale, inp.block_table[sub], vi,
                                                      idx[sub, i], cfg.n_heads, cfg.d_latent, cfg.d_rope,
                                                      cfg.softmax_scale, max_len=inp.max_len)
        assert not st_ref.any()
        parity.check_attention(o[sub, i], lse[sub, i], o_ref, lse_ref, f"{what} q={i}")
    if (~ok).any():
        assert (idx[~ok] == -1).all() and np.isnan(o[~ok]).all()
    return inp, st


@pytest.mark.parametrize("splits", [1, 2])
def test_mq_tiny(splits):
    """Three queries per request; a request of 2 tokens is shorter than n_q."""
    _lib()
    _check(gen.CONFIGS["c1"].with_(batch=3), [37, 5, 2], 3, splits, "c1 mq")


@pytest.mark.parametrize("n_q", [2, 4])
def test_mq_fp8(n_q):
    """The c3f shapes (FP8 latent rows and indexer keys, top-k 2048) with a
    request below k, one just above and a long one."""
    _lib()
    _check(gen.CONFIGS["c3f"].with_(batch=3), [2049, 70, 9000], n_q, 2, "c3f mq")


def test_mq_one_query_equals_single_step():
    """n_q = 1 is the ordinary step, bit for bit."""
    _lib()
    from sparse_paged_mla_amd.step import DecodeStep
    cfg = gen.CONFIGS["c3f"].with_(batch=2)
    inp, st = _check(cfg, [5000, 3000], 1, 2, "c3f n_q=1")
    single = DecodeStep(device_batch(inp), num_splits=2)
    single.run()
    torch.cuda.synchronize()
    assert torch.equal(single.idx, st.idx[:, 0]) and torch.equal(single.o, st.o[:, 0])
    assert torch.equal(single.lse, st.lse[:, 0])


MQ_INDEXER_CASES = [
    ("c3f", {}),                                   # FP8 keys, 64 heads, page 64
    ("c3", {}),                                    # bf16 keys
    ("c3f", {"idx_heads": 32}),
    ("c3f", {"idx_heads": 16}),
    ("c3f", {"page_size": 16}),
    ("c3", {"idx_heads": 32}),
    ("c3", {"page_size": 16}),                     # bf16 keys, pages shorter than a step
    ("c3", {"page_size": 128}),                    # steps starting inside a page
    ("c3f", {"page_size": 32, "idx_heads": 16}),   # two pages per step
]


@pytest.mark.parametrize("name,kw", MQ_INDEXER_CASES, ids=lambda v: str(v))
def test_mq_indexer_against_one_query_at_a_time(name, kw):
    """Two queries scored per key read, over ragged lengths with an empty
    request, partial pages and several runs per workgroup.  With bf16 keys
    each query gets, bit for bit, the scores and status the one-query
    indexer gives it alone (same arithmetic in the same order); with FP8
    keys the pair runs the scaled FP8 MFMA, so each query's scores are
    checked against the oracle's and the status words must agree."""
    spm = _lib()
    lens = [0, 1, 63, 65, 3000, 9000, 20000, 70]
    cfg = gen.CONFIGS[name].with_(batch=len(lens), **kw)
    print(f"[mq-indexer] {name} {kw} lens={lens}", flush=True)
    inp = gen.make_inputs(cfg, lens=lens)
    _, qi, w = gen.make_mq_queries(inp, 2)
    db = device_batch(inp)
    B, S = cfg.batch, inp.score_stride
    qi_d, w_d = tensor(qi, "cuda"), torch.from_numpy(w).cuda()
    both = torch.full((B * 2, S), float("nan"), device="cuda")
    st_both = torch.zeros(B * 2, dtype=torch.int32, device="cuda")
    spm.dsa_indexer_scores_mq(qi_d, w_d, db.k_idx, db.k_idx_scale, db.block_table, db.lens, db.max_len, both,
                              req_status=st_both)
    torch.cuda.synchronize()
    for i in range(2):
        one = torch.full((B, S), float("nan"), device="cuda")
        st_one = torch.zeros(B, dtype=torch.int32, device="cuda")
        spm.dsa_indexer_scores(qi_d[:, i].contiguous(), w_d[:, i].contiguous(), db.k_idx, db.k_idx_scale,
                               db.block_table, db.lens, db.max_len, one, req_status=st_one)
        torch.cuda.synchronize()
        a = both.view(B, 2, S)[:, i].cpu().numpy()
        np.testing.assert_array_equal(st_both.view(B, 2)[:, i].cpu().numpy(), st_one.cpu().numpy())
        if cfg.idx_dtype != gen.FP8:
            b = one.cpu().numpy()
            for r, n in enumerate(lens):
                np.testing.assert_array_equal(a[r, :n].view(np.uint32), b[r, :n].view(np.uint32),
                                              err_msg=f"request {r} query {i}")
            continue
        s_ref, mags, _ = oracle.indexer_scores(qi[:, i], w[:, i], inp.k_idx, inp.k_idx_scale, inp.block_table,
                                               inp.lens, max_len=inp.max_len, score_stride=S)
        for r, n in enumerate(lens):
            parity.check_scores(a[r, :n], s_ref[r, :n], mags[r, :n], f"pair scores b={r} q={i}")


def test_mq_indexer_flags_bad_length_when_max_len_is_zero():
    """The two-query indexer with max_len 0 and a request of length 5: both
    of its queries are flagged, the empty request's are not."""
    spm = _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=2)
    inp = gen.make_inputs(cfg, lens=[0, 5])
    _, qi, w = gen.make_mq_queries(inp, 2)
    db = device_batch(inp)
    scores = torch.zeros(4, 64, dtype=torch.float32, device="cuda")
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    spm.dsa_indexer_scores_mq(tensor(qi, "cuda"), torch.from_numpy(w).cuda(), db.k_idx, db.k_idx_scale,
                              db.block_table, db.lens, 0, scores, req_status=st)
    torch.cuda.synchronize()
    assert list(st.cpu().numpy()) == [0, 0, spm.BAD_LEN, spm.BAD_LEN]


@pytest.mark.parametrize("name", ["c3", "c3f"])
def test_mq_indexer_bad_pages(name):
    """Block-table entries out of range (negative, and past the pool) in two
    requests: the two-query indexer flags both queries of those requests and
    leaves their tokens on the bad pages NaN, like the one-query indexer;
    every other score and status is untouched (bit for bit with bf16 keys)."""
    spm = _lib()
    lens = [3000, 700, 5000]
    cfg = gen.CONFIGS[name].with_(batch=3)
    inp = gen.make_inputs(cfg, lens=lens)
    P = cfg.page_size
    bt = inp.block_table.copy()
    bt[0, 5] = -3
    bt[2, (5000 - 1) // P] = inp.k_idx.shape[0] + 7
    _, qi, w = gen.make_mq_queries(inp, 2)
    db = device_batch(inp)
    bt_d = tensor(bt, "cuda")
    B, S = 3, inp.score_stride
    qi_d, w_d = tensor(qi, "cuda"), torch.from_numpy(w).cuda()
    both = torch.full((B * 2, S), float("nan"), device="cuda")
    st_both = torch.zeros(B * 2, dtype=torch.int32, device="cuda")
    spm.dsa_indexer_scores_mq(qi_d, w_d, db.k_idx, db.k_idx_scale, bt_d, db.lens, db.max_len, both,
                              req_status=st_both)
    torch.cuda.synchronize()
    assert list(st_both.cpu().numpy()) == [spm.BAD_PAGE] * 2 + [0] * 2 + [spm.BAD_PAGE] * 2
    a = both.view(B, 2, S).cpu().numpy()
    for i in range(2):
        one = torch.full((B, S), float("nan"), device="cuda")
        st_one = torch.zeros(B, dtype=torch.int32, device="cuda")
        spm.dsa_indexer_scores(qi_d[:, i].contiguous(), w_d[:, i].contiguous(), db.k_idx, db.k_idx_scale, bt_d,
                               db.lens, db.max_len, one, req_status=st_one)
        torch.cuda.synchronize()
        b = one.cpu().numpy()
        np.testing.assert_array_equal(st_one.cpu().numpy(), st_both.view(B, 2)[:, i].cpu().numpy())
        for r, n in enumerate(lens):
            np.testing.assert_array_equal(np.isnan(a[r, i, :n]), np.isnan(b[r, :n]), err_msg=f"request {r} query {i}")
            if cfg.idx_dtype != gen.FP8:
                np.testing.assert_array_equal(a[r, i, :n].view(np.uint32), b[r, :n].view(np.uint32))
    assert np.isnan(a[0, :, 5 * P:6 * P]).all() and not np.isnan(a[0, :, :5 * P]).any()
    last = (5000 - 1) // P * P
    assert np.isnan(a[2, :, last:5000]).all() and not np.isnan(a[2, :, :last]).any()
    assert not np.isnan(a[1, :, :700]).any()
