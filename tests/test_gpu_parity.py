"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Stage by stage, so one stage's error cannot hide
another's: indexer scores; top-k on the GPU's own scores; attention on the
GPU-selected tokens; merge.  Tolerances are in tests/parity.py."""
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


def _step(inp, splits=1, split_tokens=0):
    from sparse_paged_mla_amd.step import DecodeStep
    db = device_batch(inp)
    st = DecodeStep(db, num_splits=splits, split_tokens=split_tokens)
    st.run()
    torch.cuda.synchronize()
    return db, st


def _check_full(inp, splits=1, what="", split_tokens=0):
    print(f"[parity] {what} B={inp.cfg.batch} lens={list(inp.lens[:8])} splits={splits} split_tokens={split_tokens}",
          flush=True)
    cfg = inp.cfg
    db, st = _step(inp, splits, split_tokens)
    status = st.status.cpu().numpy()
    assert not status.any(), status
    idx = None
    if not cfg.dense:
        s_gpu = st.scores.cpu().numpy()
        s_ref, mags, _ = oracle.indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table,
                                               inp.lens, score_stride=inp.score_stride)
        for b in range(cfg.batch):
            L = inp.lens[b]
            parity.check_scores(s_gpu[b, :L], s_ref[b, :L], mags[b, :L], f"{what} scores b={b}")
        idx = st.idx.cpu().numpy()
        parity.check_topk_exact(idx, s_gpu, inp.lens, cfg.topk, what)
    o_ref, lse_ref, st_ref = oracle.mla_attention(inp.q, inp.kv, inp.kv_scale, inp.block_table, inp.lens, idx,
                                                  cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    assert not st_ref.any()
    parity.check_attention(st.o.cpu().numpy(), st.lse.cpu().numpy(), o_ref, lse_ref, what)
    return db, st


# ---------------------------------------------------------------- whole steps

@pytest.mark.parametrize("splits", [1, 2, 3])
def test_c1_tiny_full_step(splits):
    _lib()
    _check_full(gen.make_inputs("c1"), splits, "c1")


def test_c1_dense_attention():
    _lib()
    inp = gen.make_inputs(gen.CONFIGS["c1"].with_(idx_heads=0, topk=0))
    _check_full(inp, 2, "c1 dense")


SMALL_SPARSE = [
    ("bf16", gen.CONFIGS["c3"].with_(batch=3), [70, 1000, 5000]),
    ("fp8", gen.CONFIGS["c3f"].with_(batch=4), [1, 300, 3000, 9000]),
    ("fp8-p16", gen.CONFIGS["c4"].with_(batch=3, page_size=16, pool_factor=1.25), [2049, 17, 4100]),
]


@pytest.mark.parametrize("name,cfg,lens", SMALL_SPARSE, ids=[s[0] for s in SMALL_SPARSE])
@pytest.mark.parametrize("splits", [1, 4])
def test_small_sparse_step(name, cfg, lens, splits):
    _lib()
    _check_full(gen.make_inputs(cfg, lens=lens), splits, name)


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_small_dense_bf16(splits):
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=3)
    _check_full(gen.make_inputs(cfg, lens=[33, 700, 2500]), splits, "dense bf16")


def test_poisoned_tails_are_never_read():
    _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=3)
    _check_full(gen.make_inputs(cfg, lens=[65, 2100, 3001], poison_tail=True), 2, "poisoned fp8")
    cfg = gen.CONFIGS["c2"].with_(batch=2)
    _check_full(gen.make_inputs(cfg, lens=[31, 1000], poison_tail=True), 3, "poisoned dense")


# ----------------------------------------------------------------- top-k only

def _gpu_topk(scores, lens, k, max_len=None, form="single"):
    """form "single": 16-byte aligned score rows, which rows of up to 256K keys
    send through the one-launch kernel; "launches": a row stride that is not
    a multiple of 4 floats, which always takes the three-launch form."""
    spm = _lib()
    B, stride = scores.shape
    if max_len is None:
        max_len = int(max(lens)) if len(lens) else 0
    if form == "launches":
        pad = 5 - stride % 4                        # stride + pad is 1 mod 4
        s = torch.from_numpy(np.pad(np.ascontiguousarray(scores, np.float32), ((0, 0), (0, pad)))).cuda()
        assert s.stride(0) % 4 != 0                 # padding past the rows' keys is never read
    else:
        s = torch.from_numpy(np.ascontiguousarray(scores, np.float32)).cuda()
        assert s.stride(0) % 4 == 0 and s.data_ptr() % 16 == 0
    l = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(spm.topk_workspace_bytes(B, max_len, k), 256), dtype=torch.uint8, device="cuda")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    spm.topk_select(s, l, max_len, k, out, ws, st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st.cpu().numpy()


FORMS = pytest.mark.parametrize("form", ["single", "launches"])


@FORMS
@pytest.mark.parametrize("k", [1, 32, 2048, 4096])
def test_topk_ties_nan_negzero(k, form):
    rng = np.random.default_rng(k)
    lens = [0, 1, 31, 2048, 5000, 70000]
    S = np.zeros((len(lens), 70016), np.float32)
    S[:] = np.round(rng.standard_normal(S.shape) * 4).astype(np.float32)  # heavy ties
    S[1, 0] = np.nan
    S[2, :31] = np.where(rng.random(31) < 0.3, np.float32(-0.0), S[2, :31])
    S[3, ::7] = np.nan
    S[4, :] = 1.25                                                         # all equal
    S[5, ::3] = -0.0
    idx, st = _gpu_topk(S, lens, k, form=form)
    assert not st.any()
    parity.check_topk_exact(idx, S, np.array(lens), k, f"ties k={k} {form}")


@FORMS
@pytest.mark.parametrize("long_len", [300000, 65536])
def test_topk_large_continuous(long_len, form):
    """Rows past and at the one-launch kernel's 64K limit (the first go
    through the three launches whatever the stride)."""
    rng = np.random.default_rng(11)
    lens = [long_len, long_len // 2 + 1, 2047, 2049]
    S = rng.standard_normal((4, long_len + 32)).astype(np.float32) * 30 + 144
    idx, st = _gpu_topk(S, lens, 2048, form=form)
    parity.check_topk_exact(idx, S, np.array(lens), 2048, f"continuous {long_len} {form}")


@FORMS
@pytest.mark.parametrize("max_len", [None, 300000])
def test_topk_big_tie_groups(max_len, form):
    """Tie groups larger than what a workgroup holds on chip (every key equal;
    two values with the k-th falling inside ~15000 equal ones), plus a plain
    row; max_len 300000 sends the same rows through the multi-workgroup
    path."""
    rng = np.random.default_rng(5)
    lens = [40000, 30000, 20000]
    S = np.zeros((3, 300032 if max_len else 40064), np.float32)
    S[0, :] = 1.25
    S[1, :] = (rng.random(S.shape[1]) < 0.5).astype(np.float32)
    S[2, :] = rng.standard_normal(S.shape[1]).astype(np.float32)
    idx, st = _gpu_topk(S, lens, 2048, max_len, form=form)
    assert not st.any()
    parity.check_topk_exact(idx, S, np.array(lens), 2048, f"big ties max_len={max_len} {form}")


@FORMS
@pytest.mark.parametrize("lens", [[100000, 250000, 90000, 90000], [60000, 65536, 50000, 50000]])
def test_topk_sample_miss_falls_back(form, lens):
    """Rows whose sampled positions hold the largest keys: the threshold from
    the sample then admits fewer than k keys, and the finish must select over
    the whole request.  The sample positions are the top-k kernel's own (16
    runs of 256 keys starting evenly over [0, L - 256]); also a row sorted in
    decreasing order and one sorted in increasing order."""
    rng = np.random.default_rng(23)
    S = rng.random((4, max(lens) + 48)).astype(np.float32)
    for r in (0, 1):
        L = lens[r]
        for run in range(16):
            t0 = run * (L - 256) // 15
            S[r, t0:t0 + 256] = 10.0 + rng.random(256).astype(np.float32)
    S[2, :lens[2]] = np.sort(S[2, :lens[2]])[::-1]  # all candidates in the first segment
    S[3, :lens[3]] = np.sort(S[3, :lens[3]])
    for k in (2048, 32):
        idx, st = _gpu_topk(S, lens, k, form=form)
        assert not st.any()
        parity.check_topk_exact(idx, S, np.array(lens), k, f"sample miss k={k} {form}")


@FORMS
def test_topk_clustered_candidates(form):
    """The largest keys (distinct) packed into the first 3000 tokens: the
    sample's first run sits inside the cluster, so about 2600 keys reach the
    threshold, all in the first of the one-launch kernel's 16 segments (more
    than its 1024-entry region: the whole-row selection takes over); also the
    cluster in the middle of the row, and a row of ordinary keys."""
    rng = np.random.default_rng(41)
    lens = [50000, 50000, 50000]
    S = rng.random((3, 50048)).astype(np.float32)
    S[0, :3000] += 10.0
    S[1, 20000:23000] += 10.0
    idx, st = _gpu_topk(S, lens, 2048, form=form)
    assert not st.any()
    parity.check_topk_exact(idx, S, np.array(lens), 2048, f"clustered {form}")


def test_topk_bad_len_flags_request():
    S = np.random.default_rng(0).standard_normal((3, 256)).astype(np.float32)
    spm = _lib()
    s = torch.from_numpy(S).cuda()
    l = torch.tensor([10, 300, -1], dtype=torch.int32, device="cuda")  # 300 > max_len 256, -1 < 0
    out = torch.empty((3, 8), dtype=torch.int32, device="cuda")
    ws = torch.empty(spm.topk_workspace_bytes(3, 256, 8), dtype=torch.uint8, device="cuda")
    st = torch.zeros(3, dtype=torch.int32, device="cuda")
    spm.topk_select(s, l, 256, 8, out, ws, st)
    torch.cuda.synchronize()
    assert list(st.cpu().numpy()) == [0, spm.BAD_LEN, spm.BAD_LEN]
    o = out.cpu().numpy()
    assert np.all(o[1:] == -1)
    parity.check_topk_exact(o[:1], S[:1], np.array([10]), 8, "bad-len neighbour")


def test_scores_growing_along_the_context():
    """Logits that grow steadily along the tokens: later tiles exceed the first
    tile's max by far more than the kernel's fixed-reference headroom, which
    forces its recompute path; results must still match the oracle."""
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=2)
    inp = gen.make_inputs(cfg, lens=[3000, 777])
    D = cfg.dim
    u = gen.normals32(11, 0, 0, D)
    u /= np.linalg.norm(u)
    q = np.broadcast_to(u * 6.0, (2, cfg.n_heads, D)).astype(np.float32)
    q[:, 1::2] *= -1.0                                  # half the heads see decreasing logits
    inp.q = gen.to_bf16_bits(q)
    P = cfg.page_size
    kv = gen.bf16_bits_to_f32(inp.kv).reshape(-1, D)
    for b in range(2):
        for t in range(int(inp.lens[b])):
            row = int(inp.block_table[b, t // P]) * P + t % P
            kv[row] = u * (t / 40.0) + 0.05 * kv[row]
    inp.kv = gen.to_bf16_bits(kv).reshape(inp.kv.shape)
    for splits in (1, 3):
        _check_full(inp, splits, "growing logits")


def test_fp8_growing_logits_recompute():
    """The same growing logits on an FP8 cache: the FP8-cache kernel's own
    recompute pass (with the segment table kept from the first pass when the
    split has one segment, rebuilt when it has several)."""
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=2, cache_dtype=gen.FP8)
    inp = gen.make_inputs(cfg, lens=[3000, 777])
    D = cfg.dim
    u = gen.normals32(11, 0, 0, D)
    u /= np.linalg.norm(u)
    q = np.broadcast_to(u * 6.0, (2, cfg.n_heads, D)).astype(np.float32)
    q[:, 1::2] *= -1.0
    inp.q = gen.to_bf16_bits(q)
    P = cfg.page_size
    rows = np.zeros((inp.num_pages * P, D), np.float32)
    for b in range(2):
        for t in range(int(inp.lens[b])):
            row = int(inp.block_table[b, t // P]) * P + t % P
            rows[row] = u * (t / 40.0) + 0.05 * gen.normals32(12, b, t, D)
    codes, scales = gen.to_fp8_rows(rows)
    inp.kv = codes.reshape(inp.kv.shape)
    inp.kv_scale = scales.reshape(inp.kv_scale.shape)
    for splits in (1, 2, 3):   # 3000 tokens: 3, 2 and 1 segments of 1024 per split
        _check_full(inp, splits, "growing logits fp8")


# The two role-specialised decode kernels: FP8 cache (c3f) and bf16 cache (c3).
SPARSE_CACHES = [pytest.param("c3f", id="fp8"), pytest.param("c3", id="bf16")]


@pytest.mark.parametrize("name", SPARSE_CACHES)
@pytest.mark.parametrize("n_heads", [8, 40, 72])
def test_partial_head_groups(name, n_heads):
    """Head counts that leave waves, and lanes within a wave, without a head."""
    _lib()
    cfg = gen.CONFIGS[name].with_(batch=3, n_heads=n_heads)
    _check_full(gen.make_inputs(cfg, lens=[70, 2500, 5000]), 3, f"{name} {n_heads} heads")


GENERIC_SHAPES = [
    pytest.param(dict(d_latent=40, d_rope=24, q_dtype=gen.BF16, cache_dtype=gen.FP8), id="40+24-bf16q-fp8"),
    pytest.param(dict(d_latent=96, d_rope=0, q_dtype=gen.F32, cache_dtype=gen.BF16), id="96+0-f32q-bf16"),
    pytest.param(dict(d_latent=256, d_rope=32, q_dtype=gen.BF16, cache_dtype=gen.BF16), id="256+32-bf16"),
    pytest.param(dict(d_latent=512, d_rope=64, q_dtype=gen.F32, cache_dtype=gen.FP8), id="512+64-f32q-fp8"),
    pytest.param(dict(d_latent=8, d_rope=8, q_dtype=gen.F32, cache_dtype=gen.F32), id="8+8-f32"),
    pytest.param(dict(d_latent=1000, d_rope=24, q_dtype=gen.BF16, cache_dtype=gen.BF16), id="1000+24-bf16"),
]


@pytest.mark.parametrize("shape", GENERIC_SHAPES)
@pytest.mark.parametrize("splits", [1, 3])
def test_generic_shapes_dense(shape, splits):
    """Latent and rope widths outside the two tuned shapes (any multiples of
    8): dense attention over pages of 16, 24 heads (a partial group of 16)."""
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=3, n_heads=24, page_size=16, **shape)
    _check_full(gen.make_inputs(cfg, lens=[5, 300, 777]), splits, f"generic dense {shape}")


@pytest.mark.parametrize("shape", GENERIC_SHAPES[:3])
def test_generic_shapes_sparse(shape):
    """The same shapes behind an indexer and top-k (k below and above L)."""
    _lib()
    cfg = gen.CONFIGS["c3"].with_(batch=2, n_heads=24, topk=64, idx_heads=8, idx_dim=32, **shape)
    _check_full(gen.make_inputs(cfg, lens=[40, 900]), 2, f"generic sparse {shape}")


@pytest.mark.parametrize("n_heads", [72, 128])
def test_fp8_many_pairs_64_head_groups(n_heads):
    """The FP8 kernel's 64-head workgroups at a size the oracle checks whole:
    66 requests x 2 splits are enough (request, split) pairs to fill a
    256-CU GPU with 64-head groups, so the 32-head form is not taken (the
    smaller cases above take it)."""
    _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=66, n_heads=n_heads, topk=256)
    lens = 40 + (np.arange(66) * 97) % 560
    _check_full(gen.make_inputs(cfg, lens=lens), 2, f"fp8 64-head groups, {n_heads} heads")


@pytest.mark.parametrize("cache", [pytest.param(gen.FP8, id="fp8"), pytest.param(gen.BF16, id="bf16")])
@pytest.mark.parametrize("splits", [1, 2, 5])
def test_dense_multi_segment(cache, splits):
    """Dense attention: splits longer than one segment table (1024
    positions) and a ragged last tile."""
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=2, cache_dtype=cache)
    _check_full(gen.make_inputs(cfg, lens=[2500, 4133]), splits, f"dense cache {cache}")


@pytest.mark.parametrize("name", SPARSE_CACHES)
def test_empty_splits(name):
    """A small top-k spread over many splits leaves whole splits empty."""
    _lib()
    cfg = gen.CONFIGS[name].with_(batch=2, topk=32)
    _check_full(gen.make_inputs(cfg, lens=[40, 3000]), 4, f"{name} empty splits")


# A fixed split length (split_tokens): long requests take more splits than
# short ones, splits past a request's end carry lse -inf only, and the last
# split takes everything from its start on.  Dense and sparse, on every decode
# kernel (FP8 and bf16 role-specialised, fp32 small shapes, generic shapes).
FIXED_SPLITS = [
    pytest.param("c2", dict(), [100, 3000, 777, 5000], 6, 1024, id="bf16-dense"),
    pytest.param("c2", dict(), [100, 3000, 777, 5000], 2, 1024, id="bf16-dense-last-takes-rest"),
    pytest.param("c2", dict(cache_dtype=gen.FP8), [2100, 65, 4000], 5, 1024, id="fp8-dense"),
    pytest.param("c3f", dict(), [3000, 70, 9000], 4, 512, id="fp8-sparse"),
    pytest.param("c3", dict(), [3000, 5000], 3, 1024, id="bf16-sparse"),
    pytest.param("c1", dict(idx_heads=0, topk=0), [37, 100], 3, 32, id="f32-small-dense"),
    pytest.param("c2", dict(d_latent=256, d_rope=32), [900, 3000], 4, 800, id="generic-dense"),
]


@pytest.mark.parametrize("name,over,lens,splits,split_tokens", FIXED_SPLITS)
def test_fixed_split_length(name, over, lens, splits, split_tokens):
    _lib()
    cfg = gen.CONFIGS[name].with_(batch=len(lens), **over)
    _check_full(gen.make_inputs(cfg, lens=lens), splits, f"{name} fixed split", split_tokens=split_tokens)


def test_balanced_splits_on_a_ragged_batch():
    """The step's balanced policy on a small ragged dense batch, and the
    partials it leaves: splits past a request's end have lse -inf."""
    from sparse_paged_mla_amd.step import balanced_splits
    _lib()
    cfg = gen.CONFIGS["c2"].with_(batch=5)
    lens = [300, 6000, 1500, 9000, 64]
    S, c = balanced_splits(lens, cfg.n_heads)
    assert c % 32 == 0 and S == max(-(-L // c) for L in lens)
    _, st = _check_full(gen.make_inputs(cfg, lens=lens), S, "balanced", split_tokens=c)
    lse_p = st.lse_part.cpu().numpy()
    for b, L in enumerate(lens):
        for s in range(S):
            live = s * c < L
            assert np.isfinite(lse_p[b, s]).all() == live, (b, s)


# ------------------------------------------------------------ fault handling

@pytest.mark.parametrize("name", SPARSE_CACHES)
def test_device_faults_flag_only_the_offending_request(name):
    spm = _lib()
    cfg = gen.CONFIGS[name].with_(batch=4)
    inp = gen.make_inputs(cfg, lens=[500, 600, 700, 800])
    bt = inp.block_table.copy()
    bt[1, 2] = inp.num_pages + 5      # request 1: page id out of range
    lens = inp.lens.copy()
    lens[2] = bt.shape[1] * cfg.page_size + 1  # request 2: longer than its mapped pages
    inp.block_table, inp.lens = bt, lens
    inp.max_len = int(lens.max())
    inp.score_stride = (inp.max_len + 63) // 64 * 64
    from sparse_paged_mla_amd.step import DecodeStep
    db = device_batch(inp)
    st = DecodeStep(db, num_splits=2)
    st.indexer()
    st.select()
    idx = st.idx.clone()
    idx[3, 5] = 800                  # request 3: index == L
    st.idx.copy_(idx)
    st.attend()
    st.merge()
    torch.cuda.synchronize()
    status = st.status.cpu().numpy()
    assert status[0] == 0
    assert status[1] & spm.BAD_PAGE
    assert status[2] & spm.BAD_LEN
    assert status[3] == spm.BAD_INDEX
    o = st.o.cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
    # Request 0 is untouched: compare with the oracle on its own selection.
    s_gpu = st.scores.cpu().numpy()
    parity.check_topk_exact(st.idx.cpu().numpy()[:1], s_gpu[:1], lens[:1], cfg.topk, "fault neighbour")
    o_ref, lse_ref, _ = oracle.mla_attention(inp.q[:1], inp.kv, inp.kv_scale, bt[:1], lens[:1],
                                             st.idx.cpu().numpy()[:1], cfg.n_heads, cfg.d_latent, cfg.d_rope,
                                             cfg.softmax_scale)
    parity.check_attention(o[:1], st.lse.cpu().numpy()[:1], o_ref, lse_ref, "fault neighbour")
    _, _, st_ref = oracle.indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, bt, lens)
    assert (st_ref[:3] == status[:3]).all()


# ----------------------------------------------------------- metamorphic checks

def test_page_permutation_and_determinism():
    _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=3)
    a = gen.make_inputs(cfg, lens=[3000, 5000, 4097])
    b = gen.make_inputs(cfg, lens=[3000, 5000, 4097], shuffle=False)
    _, s1 = _step(a, 2)
    _, s2 = _step(b, 2)
    _, s3 = _step(a, 2)
    for name in ("scores", "idx", "o", "lse"):
        x1, x2, x3 = (getattr(s, name).cpu().numpy() for s in (s1, s2, s3))
        if name == "scores":
            x1, x2, x3 = (np.concatenate([x[i, :L] for i, L in enumerate(a.lens)]) for x in (x1, x2, x3))
        assert np.array_equal(x1, x3), f"{name} not deterministic"
        assert np.array_equal(x1, x2), f"{name} changes under a page permutation"


def test_request_order_does_not_change_results():
    """Reordering the requests of a batch permutes the outputs and changes
    no bit of any request's scores, selection, o or lse (each request's work
    is independent of where it sits in the batch and of which waves share a
    workgroup with it)."""
    import dataclasses
    _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=5)
    lens = [3000, 70, 9000, 2049, 4100]
    a = gen.make_inputs(cfg, lens=lens)
    perm = np.array([3, 0, 4, 2, 1])
    b = dataclasses.replace(a, lens=a.lens[perm].copy(), block_table=a.block_table[perm].copy(),
                            q=a.q[perm].copy(), q_idx=a.q_idx[perm].copy(), w=a.w[perm].copy())
    for splits in (1, 2):
        _, s1 = _step(a, splits)
        _, s2 = _step(b, splits)
        for name in ("idx", "o", "lse", "status"):
            x1, x2 = getattr(s1, name).cpu().numpy(), getattr(s2, name).cpu().numpy()
            assert np.array_equal(x1[perm], x2), f"{name} changes when the requests are reordered"
        sc1, sc2 = s1.scores.cpu().numpy(), s2.scores.cpu().numpy()
        for j, i in enumerate(perm):
            assert np.array_equal(sc1[i, :lens[i]], sc2[j, :lens[i]]), "scores change when the requests are reordered"


def test_indexer_flags_bad_length_when_max_len_is_zero():
    """max_len 0 with a request of length 5: the indexer has nothing to
    score but still flags the request (a length above max_len is bad)."""
    spm = _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=2)
    inp = gen.make_inputs(cfg, lens=[0, 5])
    db = device_batch(inp)
    scores = torch.zeros(2, 64, dtype=torch.float32, device="cuda")
    st = torch.zeros(2, dtype=torch.int32, device="cuda")
    spm.dsa_indexer_scores(db.q_idx, db.w, db.k_idx, db.k_idx_scale, db.block_table, db.lens, 0, scores, st)
    torch.cuda.synchronize()
    assert list(st.cpu().numpy()) == [0, spm.BAD_LEN]
    _, _, st_ref = oracle.indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table, inp.lens,
                                         max_len=0, score_stride=64)
    assert list(st_ref) == [0, spm.BAD_LEN]


# Different split boundaries change the running max each probability is taken
# against before it is rounded to bf16 for the value contraction, so outputs
# agree to the bf16 rounding of the weights (relative 2^-9 each), not bit for
# bit: |do| <= 2^-8 * max|v| is the bound; 2e-3 is used.  lse is formed in
# fp32 from unrounded weights.
SPLIT_O_ATOL = 2e-3
SPLIT_LSE_ATOL = 2e-5


def test_splits_agree():
    _lib()
    cfg = gen.CONFIGS["c3f"].with_(batch=2)
    inp = gen.make_inputs(cfg, lens=[6000, 9000])
    outs = [_step(inp, s)[1] for s in (1, 2, 7, 32)]
    for st in outs[1:]:
        assert np.abs(st.o.cpu().numpy() - outs[0].o.cpu().numpy()).max() < SPLIT_O_ATOL
        assert np.abs(st.lse.cpu().numpy() - outs[0].lse.cpu().numpy()).max() < SPLIT_LSE_ATOL
        assert np.array_equal(st.idx.cpu().numpy(), outs[0].idx.cpu().numpy())


def test_k_ge_len_equals_dense():
    _lib()
    cfg = gen.CONFIGS["c3"].with_(batch=2, topk=4096)
    inp = gen.make_inputs(cfg, lens=[1000, 4096])
    _, sp = _step(inp, 2)
    dense = gen.make_inputs(cfg.with_(idx_heads=0, topk=0), lens=[1000, 4096])
    _, dn = _step(dense, 2)
    assert np.abs(sp.o.cpu().numpy() - dn.o.cpu().numpy()).max() < SPLIT_O_ATOL
    assert np.abs(sp.lse.cpu().numpy() - dn.lse.cpu().numpy()).max() < SPLIT_LSE_ATOL
    # With one split both paths attend the same tokens in the same order: bit-identical.
    _, sp1 = _step(inp, 1)
    _, dn1 = _step(dense, 1)
    assert np.array_equal(sp1.o.cpu().numpy(), dn1.o.cpu().numpy())
    assert np.array_equal(sp1.lse.cpu().numpy(), dn1.lse.cpu().numpy())


# --------------------------------------------------------------- lse merge only

@pytest.mark.parametrize("S", [2, 4, 5, 8])
def test_merge_matches_oracle_on_random_partials(S):
    """Split counts with a specialised kernel (2, 4, 8 at d = 512) and without
    (5); empty splits hold NaN partials, which must not be used."""
    spm = _lib()
    rng = np.random.default_rng(3)
    B, H, d = 3, 16, 512
    op = rng.standard_normal((B, S, H, d)).astype(np.float32)
    lp = (rng.standard_normal((B, S, H)) * 4).astype(np.float32)
    lp[0, 1:, :] = -np.inf                 # only split 0 non-empty
    op[0, 1:, :, :] = np.nan               # never written by an empty split
    lp[1, :, 3] = -np.inf                  # a fully empty row
    lp[2, S - 1, 5] = np.nan               # NaN propagates
    o = torch.empty(B, H, d, device="cuda")
    l = torch.empty(B, H, device="cuda")
    spm.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), o, l)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(op, lp)
    og, lg = o.cpu().numpy(), l.cpu().numpy()
    assert np.array_equal(np.isnan(lg), np.isnan(l_ref))
    ok = ~np.isnan(l_ref)
    assert np.array_equal(lg[ok] == -np.inf, l_ref[ok] == -np.inf)
    fin = np.isfinite(l_ref)
    assert np.abs(lg[fin] - l_ref[fin]).max() < 1e-5
    assert np.abs(og[ok] - o_ref[ok]).max() < 1e-5
