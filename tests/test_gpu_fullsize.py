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
    from sparse_paged_mla_amd.step import DEFAULT_SPLITS, DecodeStep
    spm.load_library()
    _say(f"{name}: generating inputs")
    inp = gen.make_inputs(name)
    cfg = inp.cfg
    splits = DEFAULT_SPLITS[name]
    db = device_batch(inp)
    step = DecodeStep(db, num_splits=splits)
    _say(f"{name}: B={cfg.batch} sum L={int(inp.lens.sum())} max_len={inp.max_len} splits={splits}: running the step")
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
    parity.check_attention(step.o.cpu().numpy()[sel], step.lse.cpu().numpy()[sel], o_ref, lse_ref,
                           f"{name} attention requests {reqs}")
    _say(f"{name}: attention of requests {reqs} matches")
