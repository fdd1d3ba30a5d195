"""GPU parity at the full sizes of every workload, in the launch
configuration the benchmark times (its default KV splits): the whole step
runs on the device; the oracle checks indexer scores at sampled (request,
token) positions, the top-k of every request exactly against the GPU's own
scores, and the attention output and log-sum-exp of sampled requests over
the GPU-selected tokens.  Inputs are seeded (spmla_gen); nothing here is
stored."""
import numpy as np
import pytest
import torch

import oracle
import spmla_gen as gen
from spmla_gen.torch_io import device_batch
from tests import parity

pytestmark = pytest.mark.gpu

N_SCORE_SAMPLES = 512
N_ATTN_REQUESTS = 3


def _say(msg):
    print(f"[fullsize] {msg}", flush=True)


@pytest.mark.parametrize("name", ["c2", "c3", "c3f", "c4", "c5"])
def test_full_size_step(name):
    import sparse_paged_mla_amd as spm
    from sparse_paged_mla_amd.step import DecodeStep, default_splits
    spm.load_library()
    _say(f"{name}: generating inputs")
    inp = gen.make_inputs(name)
    cfg = inp.cfg
    splits, split_tokens = default_splits(name, inp.lens, cfg.n_heads)
    db = device_batch(inp)
    step = DecodeStep(db, num_splits=splits, split_tokens=split_tokens)
    _say(f"{name}: B={cfg.batch} sum L={int(inp.lens.sum())} max_len={inp.max_len} splits={splits} "
         f"split_tokens={split_tokens}: running the step")
    step.run()
    torch.cuda.synchronize()
    status = step.status.cpu().numpy()
    assert not status.any(), status
    rng = np.random.default_rng(1000 + cfg.seed)
    idx = None
    if not cfg.dense:
        s_gpu = step.scores.cpu().numpy()
        # Indexer: sampled positions, every request represented.
        sb = rng.integers(0, cfg.batch, N_SCORE_SAMPLES).astype(np.int32)
        sb[: cfg.batch] = np.arange(min(cfg.batch, N_SCORE_SAMPLES))
        st = (rng.random(N_SCORE_SAMPLES) * inp.lens[sb]).astype(np.int64)
        st[::7] = inp.lens[sb[::7]] - 1  # the last token of a request
        s_ref, mags = oracle.indexer_scores_at(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table,
                                               sb, st)
        parity.check_scores(s_gpu[sb, st], s_ref, mags, f"{name} sampled scores")
        _say(f"{name}: {N_SCORE_SAMPLES} sampled scores match")
        # Top-k: exact on the GPU's own scores, every request.
        idx = step.idx.cpu().numpy()
        parity.check_topk_exact(idx, s_gpu, inp.lens, cfg.topk, f"{name} top-k")
        _say(f"{name}: top-k of all {cfg.batch} requests exact")
    # Attention: sampled requests (the longest, the shortest, one more).
    L = inp.lens
    reqs = sorted({int(np.argmax(L)), int(np.argmin(L)), int(rng.integers(0, cfg.batch))})[:N_ATTN_REQUESTS]
    sel = np.array(reqs, np.int32)
    o_ref, lse_ref, st_ref = oracle.mla_attention(inp.q[sel], inp.kv, inp.kv_scale, inp.block_table[sel], L[sel],
                                                  None if idx is None else idx[sel], cfg.n_heads, cfg.d_latent,
                                                  cfg.d_rope, cfg.softmax_scale, max_len=inp.max_len)
    assert not st_ref.any()
    o_gpu = step.o.cpu().numpy()
    d_o = parity.check_attention(o_gpu[sel], step.lse.cpu().numpy()[sel], o_ref, lse_ref,
                                 f"{name} attention requests {reqs}")
    _say(f"{name}: attention of requests {reqs} matches (max |do| {d_o:.2e}, "
         f"relative RMS {parity.rel_rms(o_gpu[sel], o_ref):.2e})")
    if not cfg.dense and name != "c5":
        # Diagnostic: the oracle's own fp64 scores and top-k for the shortest
        # request, against what the GPU selected and produced.
        b = np.array([int(np.argmin(L))], np.int32)
        s_full, _, _ = oracle.indexer_scores(inp.q_idx[b], inp.w[b], inp.k_idx, inp.k_idx_scale,
                                             inp.block_table[b], L[b], max_len=inp.max_len,
                                             score_stride=int(L[b][0]))

        def att(ix):
            o, l, _ = oracle.mla_attention(inp.q[b], inp.kv, inp.kv_scale, inp.block_table[b], L[b], ix,
                                           cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.softmax_scale,
                                           max_len=inp.max_len)
            return o, l
        e2e = parity.end_to_end(idx[b], o_gpu[b], s_full, L[b], cfg.topk, att)
        _say(f"{name}: end to end (request {int(b[0])}, L={int(L[b][0])}): {e2e['swaps']} of {e2e['selected']} "
             f"selected tokens differ from the fp64 ranking; max |do| {e2e['max_abs_do']:.2e}, "
             f"relative RMS {e2e['rel_rms_o']:.2e}")


def test_full_size_multi_query_c3f():
    """The two-query verification step at the c3f size, as the benchmark
    times it (two queries per key read in the indexer): sampled scores of
    both queries, every query's top-k exactly against the GPU's scores with
    its causal length, attention of sampled requests."""
    import sparse_paged_mla_amd as spm
    from spmla_gen.torch_io import tensor
    from sparse_paged_mla_amd.step import DEFAULT_SPLITS, MultiQueryStep
    spm.load_library()
    n_q = 2
    inp = gen.make_inputs("c3f")
    cfg = inp.cfg
    q, qi, w = gen.make_mq_queries(inp, n_q)
    st = MultiQueryStep(device_batch(inp), tensor(q, "cuda"), tensor(qi, "cuda"), torch.from_numpy(w).cuda(),
                        num_splits=DEFAULT_SPLITS["c3f"])
    assert st.two_query_indexer
    _say("c3f n_q=2: running the multi-query step")
    st.run()
    torch.cuda.synchronize()
    assert not st.status.cpu().numpy().any()
    s_gpu, idx = st.scores.cpu().numpy(), st.idx.cpu().numpy()
    vis = inp.lens[:, None] - n_q + 1 + np.arange(n_q)[None, :]
    rng = np.random.default_rng(77)
    for i in range(n_q):
        sb = rng.integers(0, cfg.batch, 256).astype(np.int32)
        tt = (rng.random(256) * vis[sb, i]).astype(np.int64)
        tt[::5] = vis[sb[::5], i] - 1
        s_ref, mags = oracle.indexer_scores_at(qi[:, i], w[:, i], inp.k_idx, inp.k_idx_scale, inp.block_table, sb, tt)
        parity.check_scores(s_gpu[sb, i, tt], s_ref, mags, f"mq scores q={i}")
        parity.check_topk_exact(idx[:, i], s_gpu[:, i], vis[:, i], cfg.topk, f"mq top-k q={i}")
        sel = np.array(sorted({int(np.argmax(inp.lens)), int(rng.integers(0, cfg.batch))}), np.int32)
        o_ref, lse_ref, _ = oracle.mla_attention(q[sel, i], inp.kv, inp.kv_scale, inp.block_table[sel],
                                                 vis[sel, i].astype(np.int32), idx[sel, i], cfg.n_heads,
                                                 cfg.d_latent, cfg.d_rope, cfg.softmax_scale, max_len=inp.max_len)
        parity.check_attention(st.o.cpu().numpy()[sel, i], st.lse.cpu().numpy()[sel, i], o_ref, lse_ref,
                               f"mq attention q={i} requests {list(sel)}")
    _say("c3f n_q=2: sampled scores, all top-k and sampled attention match")


def test_full_size_prefill_chunk_sampled():
    """The prefill chunk as the benchmark times it (64 new tokens on each of
    the first two c3f requests, 2 KV blocks): the newest query of the first
    request and the oldest of the second against the oracle's dense causal
    attention (each one is tens of GFLOP in the fp64 oracle)."""
    import sparse_paged_mla_amd as spm
    from spmla_gen.torch_io import tensor
    from sparse_paged_mla_amd.step import PrefillChunkStep
    spm.load_library()
    inp = gen.make_inputs("c3f")
    cfg = inp.cfg
    n_req, n_q = 2, 64
    q = gen.make_chunk_queries(inp, n_req, n_q)
    db = device_batch(inp)
    import dataclasses
    sub = dataclasses.replace(db, q=db.q[:n_req], block_table=db.block_table[:n_req], lens=db.lens[:n_req])
    st = PrefillChunkStep(sub, tensor(q, "cuda"), num_blocks=2)
    _say("c3f prefill chunk: running")
    st.run()
    torch.cuda.synchronize()
    assert not st.status.cpu().numpy().any()
    o, lse = st.o.cpu().numpy(), st.lse.cpu().numpy()
    for b, i in ((0, n_q - 1), (1, 0)):
        vis = int(inp.lens[b]) - n_q + 1 + i
        o_ref, lse_ref, _ = oracle.mla_attention(q[b:b + 1, i], inp.kv, inp.kv_scale, inp.block_table[b:b + 1],
                                                 np.array([vis], np.int32), None, cfg.n_heads, cfg.d_latent,
                                                 cfg.d_rope, cfg.softmax_scale, max_len=inp.max_len)
        parity.check_attention(o[b:b + 1, i], lse[b:b + 1, i], o_ref, lse_ref, f"prefill b={b} q={i}")
    _say("c3f prefill chunk: sampled queries match")
