"""GPU parity of the prefill chunk attention (dense, causal, KV blocks merged
with the online-softmax algebra) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import spmla_gen as gen
from spmla_gen.torch_io import device_batch, tensor
from tests import parity
from tests.test_gpu_parity import SPLIT_LSE_ATOL, SPLIT_O_ATOL

pytestmark = pytest.mark.gpu


def _run(cfg, lens, n_q, blocks, seed=21):
    import sparse_paged_mla_amd as spm
    from sparse_paged_mla_amd.step import PrefillChunkStep
    spm.load_library()
    inp = gen.make_inputs(cfg, lens=lens)
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((cfg.batch, n_q, cfg.n_heads, cfg.dim)).astype(np.float32)
    q = gen.to_bf16_bits(q32) if cfg.q_dtype == gen.BF16 else q32
    st = PrefillChunkStep(device_batch(inp), tensor(q, "cuda"), num_blocks=blocks)
    st.run()
    torch.cuda.synchronize()
    return inp, q, st


@pytest.mark.parametrize("blocks", [1, 3])
def test_prefill_chunk_bf16(blocks):
    cfg = gen.CONFIGS["c2"].with_(batch=2)
    print(f"[prefill] bf16 blocks={blocks}", flush=True)
    inp, q, st = _run(cfg, [700, 1500], 16, blocks)
    assert not st.status.cpu().numpy().any()
    o_ref, l_ref, s_ref = oracle.prefill_chunk_attention(q, inp.kv, inp.kv_scale, inp.block_table, inp.lens,
                                                         cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    assert not s_ref.any()
    parity.check_attention(st.o.cpu().numpy().reshape(-1, cfg.n_heads, cfg.d_latent),
                           st.lse.cpu().numpy().reshape(-1, cfg.n_heads),
                           o_ref.reshape(-1, cfg.n_heads, cfg.d_latent), l_ref.reshape(-1, cfg.n_heads),
                           f"prefill bf16 blocks={blocks}")


def test_prefill_chunk_fp8_and_short_request():
    """FP8 cache; a request shorter than the chunk is flagged, its outputs NaN."""
    cfg = gen.CONFIGS["c3f"].with_(batch=3)
    print("[prefill] fp8", flush=True)
    inp, q, st = _run(cfg, [2000, 300, 5], 8, 2)
    status = st.status.cpu().numpy()
    assert not status[:2].any() and (status[2] & oracle.BAD_LEN).all()
    o_ref, l_ref, _ = oracle.prefill_chunk_attention(q[:2], inp.kv, inp.kv_scale, inp.block_table[:2], inp.lens[:2],
                                                     cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    o, lse = st.o.cpu().numpy(), st.lse.cpu().numpy()
    parity.check_attention(o[:2].reshape(-1, cfg.n_heads, cfg.d_latent), lse[:2].reshape(-1, cfg.n_heads),
                           o_ref.reshape(-1, cfg.n_heads, cfg.d_latent), l_ref.reshape(-1, cfg.n_heads), "prefill fp8")
    assert np.isnan(o[2]).all()


def test_prefill_blocks_agree():
    """Cutting the context into 1, 4 or 7 blocks changes only rounding."""
    cfg = gen.CONFIGS["c2"].with_(batch=2)
    outs = [_run(cfg, [3000, 1200], 12, nb)[2] for nb in (1, 4, 7)]
    for st in outs[1:]:
        assert np.abs(st.o.cpu().numpy() - outs[0].o.cpu().numpy()).max() < SPLIT_O_ATOL
        assert np.abs(st.lse.cpu().numpy() - outs[0].lse.cpu().numpy()).max() < SPLIT_LSE_ATOL
