"""Pins of the fp64 oracle against things other than itself.

Each check uses a closed form, an invariant, a brute force written
independently with library routines (numpy einsum, scipy softmax/logsumexp,
Python's sort, torch's float8/bfloat16 casts), or a value printed on the
pages.  They are chosen so that a plausible slip in the oracle -- a dropped
term (the rope dims, the ReLU, the head weight), a wrong sign, a wrong index
or page mapping, a transposed operand, the wrong tie rule -- fails one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
import spmla_gen as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ decoders

def test_fp8_closed_form_all_codes():
    vals = np.array([oracle.fp8_e4m3_value(c) for c in range(256)])
    assert vals[0x7E] == 448.0
    assert vals[0x08] == 2.0 ** -6
    assert vals[0x01] == 2.0 ** -9
    assert vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x38] == 1.0
    assert vals[0x00] == 0.0 and math.copysign(1, vals[0x80]) == -1.0
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.sum(np.isnan(vals)) == 2
    np.testing.assert_array_equal(vals[0x80:0xFF], -vals[0x00:0x7F])
    assert np.all(np.diff(vals[0:0x7F]) > 0)  # strictly increasing magnitude over the positive codes


def test_fp8_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.fp8_e4m3_value(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, 4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_value(b) for b in bits])
    np.testing.assert_array_equal(ours, ref)


# ------------------------------------------------------- helpers for brute force

def _fp8_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _values(arr, scale=None):
    """Library-routine decode of a storage array to float64 (torch casts)."""
    if arr.dtype == np.float32:
        v = arr.astype(np.float64)
    elif arr.dtype == np.uint16:
        v = _bf16_to_f64(arr)
    else:
        v = _fp8_to_f64(arr) * scale.astype(np.float64)[..., None]
    return v


def _logical_rows(inp, pool, scale, b):
    """Rows of request b from an un-shuffled (contiguous) pool: a plain slice."""
    first = int(inp.block_table[b, 0])
    L = int(inp.lens[b])
    P = inp.cfg.page_size
    flat = _values(pool, scale).reshape(-1, pool.shape[-1])
    return flat[first * P: first * P + L]


@pytest.fixture(scope="module")
def c1_contig():
    return gen.make_inputs("c1", shuffle=False)


@pytest.fixture(scope="module")
def c1():
    return gen.make_inputs("c1")


def _fp8_small():
    cfg = gen.CONFIGS["c1"].with_(cache_dtype=gen.FP8, idx_dtype=gen.FP8, q_dtype=gen.BF16, name="c1f8")
    return cfg


# ------------------------------------------------------------------- indexer

def _brute_scores(inp, b):
    K = _logical_rows(inp, inp.k_idx, inp.k_idx_scale, b)           # [L, d]
    q = _values(inp.q_idx[b])                                         # [H, d]
    w = inp.w[b].astype(np.float64)                                   # [H]
    dots = np.einsum("hd,td->ht", q, K)
    return np.einsum("h,ht->t", w, np.maximum(dots, 0.0))


@pytest.mark.parametrize("cfg", ["c1", "c1f8"])
def test_indexer_matches_einsum_brute_force(cfg):
    c = gen.CONFIGS["c1"] if cfg == "c1" else _fp8_small()
    inp = gen.make_inputs(c, shuffle=False)
    s, a, st = oracle.indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table, inp.lens)
    assert not st.any()
    for b in range(inp.cfg.batch):
        L = inp.lens[b]
        ref = _brute_scores(inp, b)
        np.testing.assert_allclose(s[b, :L], ref, rtol=1e-12, atol=1e-12)
        assert np.all(a[b, :L] >= np.abs(s[b, :L]) - 1e-12)


def _brute_magnitudes(inp, b):
    """A_t = sum_h |w_h| sum_i |q_h,i k_t,i|: the term magnitudes of the score
    sum, the scale its tolerance is set against, summed the other way round
    (over heads first for every dim) so that no loop order is shared."""
    K = _logical_rows(inp, inp.k_idx, inp.k_idx_scale, b)           # [L, d]
    q = _values(inp.q_idx[b])                                         # [H, d]
    aw = np.abs(inp.w[b].astype(np.float64))                          # [H]
    per_dim = np.einsum("h,hd->d", aw, np.abs(q))                     # sum_h |w_h| |q_h,i|
    return np.abs(K) @ per_dim


def _abs_storage(arr):
    """The same storage with every sign bit cleared (fp32 values, bf16 or FP8 codes)."""
    if arr.dtype == np.float32:
        return np.abs(arr)
    return arr & (np.uint16(0x7FFF) if arr.dtype == np.uint16 else np.uint8(0x7F))


@pytest.mark.parametrize("cfg", ["c1", "c1f8"])
def test_indexer_magnitudes_match_brute_force(cfg):
    # The tiny case draws w ~ N(0,1), so negative weights are present and a
    # dropped |w_h| (or a stray factor, or a missing FP8 scale) changes A_t.
    c = gen.CONFIGS["c1"] if cfg == "c1" else _fp8_small()
    inp = gen.make_inputs(c, shuffle=False)
    assert (inp.w < 0).any() and (inp.w > 0).any()
    _, a, st = oracle.indexer_scores(inp.q_idx, inp.w, inp.k_idx, inp.k_idx_scale, inp.block_table, inp.lens)
    assert not st.any()
    for b in range(inp.cfg.batch):
        L = inp.lens[b]
        np.testing.assert_allclose(a[b, :L], _brute_magnitudes(inp, b), rtol=1e-12, atol=0)
    # A_t bounds |s_t| from above; with every weight and every operand taken
    # positive (no ReLU cut, no cancellation) the bound is reached exactly.
    q_abs, k_abs = _abs_storage(inp.q_idx), _abs_storage(inp.k_idx)
    s2, a2, _ = oracle.indexer_scores(q_abs, np.abs(inp.w), k_abs, inp.k_idx_scale, inp.block_table, inp.lens)
    for b in range(inp.cfg.batch):
        L = inp.lens[b]
        np.testing.assert_allclose(a2[b, :L], s2[b, :L], rtol=1e-12, atol=0)


def test_indexer_page_permutation_invariant(c1, c1_contig):
    s1, _, _ = oracle.indexer_scores(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, c1.block_table, c1.lens)
    s2, _, _ = oracle.indexer_scores(c1_contig.q_idx, c1_contig.w, c1_contig.k_idx, c1_contig.k_idx_scale,
                                     c1_contig.block_table, c1_contig.lens)
    for b in range(2):
        L = c1.lens[b]
        np.testing.assert_array_equal(s1[b, :L], s2[b, :L])


def test_indexer_special_cases(c1_contig):
    inp = c1_contig
    # w = 0 => every score is 0.
    s, _, _ = oracle.indexer_scores(inp.q_idx, np.zeros_like(inp.w), inp.k_idx, None, inp.block_table, inp.lens)
    for b in range(2):
        assert np.all(s[b, :inp.lens[b]] == 0.0)
    # One head, w = 1 => ReLU of the plain dot product.
    q1 = np.ascontiguousarray(inp.q_idx[:, :1, :])
    s, _, _ = oracle.indexer_scores(q1, np.ones((2, 1), np.float32), inp.k_idx, None, inp.block_table, inp.lens)
    for b in range(2):
        K = _logical_rows(inp, inp.k_idx, None, b)
        np.testing.assert_allclose(s[b, :inp.lens[b]], np.maximum(K @ q1[b, 0].astype(np.float64), 0), rtol=1e-13)
    # q_h = e_j for every head => sum_h w_h * ReLU(k_t[j]); negative w flips the sign of the sum.
    j = 5
    qe = np.zeros_like(inp.q_idx)
    qe[:, :, j] = 1.0
    w = np.array([[0.5, -2.0], [3.0, 1.0]], np.float32)
    s, _, _ = oracle.indexer_scores(qe, w, inp.k_idx, None, inp.block_table, inp.lens)
    for b in range(2):
        K = _logical_rows(inp, inp.k_idx, None, b)
        np.testing.assert_allclose(s[b, :inp.lens[b]], w[b].sum() * np.maximum(K[:, j], 0), rtol=1e-13)


def test_indexer_sampled_equals_full(c1):
    s, a, _ = oracle.indexer_scores(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, c1.block_table, c1.lens)
    sb = np.array([0, 0, 1, 1, 1], np.int32)
    stk = np.array([0, 36, 0, 50, 99], np.int64)
    s2, a2 = oracle.indexer_scores_at(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, c1.block_table, sb, stk)
    np.testing.assert_array_equal(s2, s[sb, stk])
    np.testing.assert_array_equal(a2, a[sb, stk])


def test_indexer_status_flags(c1):
    bt = c1.block_table.copy()
    bt[1, 3] = c1.num_pages  # out of range page used by request 1
    s, _, st = oracle.indexer_scores(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, bt, c1.lens)
    assert st[0] == 0 and st[1] == oracle.BAD_PAGE
    assert np.all(np.isnan(s[1, :100])) and not np.isnan(s[0, :37]).any()
    lens = c1.lens.copy()
    lens[0] = 200  # beyond its mapped pages (bt_stride * P = 112)
    _, _, st = oracle.indexer_scores(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, c1.block_table, lens)
    assert st[0] == oracle.BAD_LEN and st[1] == 0


# --------------------------------------------------------------------- top-k

def _brute_topk(s, L, k):
    def key(t):
        v = s[t]
        return (1, 0.0, t) if np.isnan(v) else (0, -float(v), t)
    order = sorted(range(L), key=key)
    sel = sorted(order[:min(k, L)])
    return sel + [-1] * (k - len(sel))


def test_topk_brute_force_with_ties_nan_negzero():
    rng = np.random.default_rng(1)
    for trial in range(200):
        L = int(rng.integers(1, 60))
        k = int(rng.integers(1, 70))
        s = rng.integers(-3, 4, L).astype(np.float64)  # many exact ties
        if trial % 3 == 0:
            s[rng.random(L) < 0.2] = np.nan
        if trial % 4 == 0:
            s[s == 0] = -0.0
        if trial % 5 == 0:
            s[rng.random(L) < 0.2] = -np.inf
        got = oracle.topk(s[None, :], np.array([L]), k)[0]
        assert list(got) == _brute_topk(s, L, k), (trial, s, k)


def test_topk_invariants_large():
    rng = np.random.default_rng(2)
    L, k = 50000, 2048
    s = np.round(rng.standard_normal(L) * 50) / 4  # coarse grid -> ties at the threshold
    idx = oracle.topk(s[None, :], np.array([L]), k)[0]
    assert np.all(np.diff(idx) > 0) and len(idx) == k
    sel = np.zeros(L, bool)
    sel[idx] = True
    assert s[sel].min() >= s[~sel].max()
    thr = s[sel].min()
    tied_sel = np.where(sel & (s == thr))[0]
    tied_un = np.where(~sel & (s == thr))[0]
    assert len(tied_un) == 0 or tied_un.min() > tied_sel.max()


def test_topk_degenerate():
    L, k = 300, 64
    idx = oracle.topk(np.full((1, L), 1.5), np.array([L]), k)[0]
    np.testing.assert_array_equal(idx, np.arange(k))
    s = np.random.default_rng(3).standard_normal((1, 40))
    idx = oracle.topk(s, np.array([40]), 64)[0]
    np.testing.assert_array_equal(idx, np.r_[np.arange(40), -np.ones(24)])
    idx = oracle.topk(s, np.array([0]), 8)[0]
    assert np.all(idx == -1)
    s = np.array([[-0.0, 0.0, -0.0, 1.0]])
    np.testing.assert_array_equal(oracle.topk(s, np.array([4]), 2)[0], [0, 3])


# ----------------------------------------------------------------- attention

def _brute_attention(inp, b, tokens=None):
    """Dense softmax without the max trick (fine for N(0,1) data at tiny sizes), library softmax."""
    cfg = inp.cfg
    C = _logical_rows(inp, inp.kv, inp.kv_scale, b)
    if tokens is not None:
        C = C[tokens]
    q = _values(inp.q[b])                                            # [H, D]
    z = cfg.softmax_scale * (q @ C.T)                                 # [H, n]
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    o = p @ C[:, :cfg.d_latent]
    lse = np.log(np.exp(z).sum(axis=1))
    # cross-check the hand softmax with the library's
    np.testing.assert_allclose(p, softmax(z, axis=1), rtol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-12)
    return o, lse


def _att(inp, idx=None, q=None, kv=None, kv_scale=None, bt=None, lens=None):
    c = inp.cfg
    return oracle.mla_attention(inp.q if q is None else q, inp.kv if kv is None else kv,
                                inp.kv_scale if kv_scale is None else kv_scale,
                                inp.block_table if bt is None else bt, inp.lens if lens is None else lens,
                                idx, c.n_heads, c.d_latent, c.d_rope, c.softmax_scale)


@pytest.mark.parametrize("cfg", ["c1", "c1f8"])
def test_attention_dense_matches_brute_force(cfg):
    c = gen.CONFIGS["c1"] if cfg == "c1" else _fp8_small()
    inp = gen.make_inputs(c, shuffle=False)
    o, lse, st = _att(inp)
    assert not st.any()
    for b in range(2):
        ro, rl = _brute_attention(inp, b)
        np.testing.assert_allclose(o[b], ro, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-12)


def test_attention_sparse_matches_brute_force(c1_contig):
    inp = c1_contig
    rng = np.random.default_rng(4)
    k = 20
    idx = np.full((2, k), -1, np.int32)
    sets = []
    for b in range(2):
        sel = np.sort(rng.choice(inp.lens[b], size=12 + 5 * b, replace=False))
        idx[b, :len(sel)] = sel
        rng.shuffle(idx[b])  # order and padding position must not matter
        sets.append(sel)
    o, lse, _ = _att(inp, idx)
    for b in range(2):
        ro, rl = _brute_attention(inp, b, sets[b])
        np.testing.assert_allclose(o[b], ro, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-12)


def test_attention_page_permutation_invariant(c1, c1_contig):
    o1, l1, _ = _att(c1)
    o2, l2, _ = _att(c1_contig)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_attention_closed_forms(c1_contig):
    inp = c1_contig
    c = inp.cfg
    # q = 0 => uniform weights: o = mean of the value rows, lse = ln |S|.
    o, lse, _ = _att(inp, q=np.zeros_like(inp.q))
    for b in range(2):
        C = _logical_rows(inp, inp.kv, None, b)
        np.testing.assert_allclose(o[b], np.broadcast_to(C[:, :c.d_latent].mean(0), o[b].shape), rtol=1e-12,
                                   atol=1e-14)
        np.testing.assert_allclose(lse[b], np.log(inp.lens[b]), rtol=1e-14)
    # Every row equal to one vector => o = its latent part, lse = z + ln |S|.
    row = gen.normals32(9, 0, 0, c.dim)
    kv = np.broadcast_to(row, inp.kv.shape).copy()
    o, lse, _ = _att(inp, kv=kv)
    for b in range(2):
        z = c.softmax_scale * (inp.q[b].astype(np.float64) @ row.astype(np.float64))
        np.testing.assert_allclose(o[b], np.broadcast_to(row[:c.d_latent], o[b].shape), rtol=1e-12)
        np.testing.assert_allclose(lse[b], z + np.log(inp.lens[b]), rtol=1e-12)


def test_topk_k_ge_len_equals_dense(c1):
    dense_o, dense_l, _ = _att(c1)
    s, _, _ = oracle.indexer_scores(c1.q_idx, c1.w, c1.k_idx, c1.k_idx_scale, c1.block_table, c1.lens)
    idx = oracle.topk(s, c1.lens, 128)
    o, l, _ = _att(c1, idx=idx)
    np.testing.assert_allclose(o, dense_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, dense_l, rtol=1e-12)


def test_attention_status(c1):
    idx = np.tile(np.arange(32, dtype=np.int32), (2, 1))
    idx[0, 5] = 37  # == L_0: out of range
    o, lse, st = _att(c1, idx=idx)
    assert st[0] == oracle.BAD_INDEX and st[1] == 0
    assert np.isnan(o[0]).all() and np.isnan(lse[0]).all() and not np.isnan(o[1]).any()
    bt = c1.block_table.copy()
    bt[0, 1] = -5
    _, _, st = _att(c1, bt=bt)
    assert st[0] == oracle.BAD_PAGE and st[1] == 0
    empty = np.full((2, 4), -1, np.int32)
    o, lse, st = _att(c1, idx=empty)
    assert not st.any() and np.all(o == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------- merge

def test_merge_partition_equals_unsplit(c1):
    rng = np.random.default_rng(5)
    full_o, full_l, _ = _att(c1)
    for S in (1, 2, 3, 7):
        parts_o, parts_l = [], []
        assign = [rng.integers(0, S, int(L)) for L in c1.lens]
        for j in range(S):
            k = int(max(c1.lens))
            idx = np.full((2, k), -1, np.int32)
            for b in range(2):
                sel = np.where(assign[b] == j)[0]
                idx[b, :len(sel)] = sel
            o, l, _ = _att(c1, idx=idx)
            parts_o.append(o)
            parts_l.append(l)
        o, l = oracle.lse_merge(np.stack(parts_o, 1), np.stack(parts_l, 1))
        np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, full_l, rtol=1e-13)


def test_merge_algebra():
    rng = np.random.default_rng(6)
    B, H, d = 3, 4, 8
    parts = [(rng.standard_normal((B, 1, H, d)), rng.standard_normal((B, 1, H)) * 3) for _ in range(3)]
    a, b, c = parts

    def m(*xs):
        o, l = oracle.lse_merge(np.concatenate([x[0] for x in xs], 1), np.concatenate([x[1] for x in xs], 1))
        return o[:, None], l[:, None]
    left = m(m(a, b), c)
    right = m(a, m(b, c))
    np.testing.assert_allclose(left[0], right[0], atol=1e-12)
    np.testing.assert_allclose(left[1], right[1], atol=1e-12)
    comm = m(c, a, b)
    np.testing.assert_allclose(comm[0], left[0], atol=1e-12)
    # Equal LSEs: plain average, lse + ln(m).
    lse_eq = np.broadcast_to(a[1], (B, 3, H)).copy()
    os_ = np.concatenate([a[0], b[0], c[0]], 1)
    o, l = oracle.lse_merge(os_, lse_eq)
    np.testing.assert_allclose(o, os_.mean(1), atol=1e-13)
    np.testing.assert_allclose(l, a[1][:, 0] + np.log(3), atol=1e-13)
    # An empty split (-inf) is the identity; all empty gives o = 0, lse = -inf.
    empty = (np.zeros((B, 1, H, d)), np.full((B, 1, H), -np.inf))
    o, l = m(a, empty)
    np.testing.assert_allclose(o[:, 0], a[0][:, 0], atol=1e-14)
    np.testing.assert_allclose(l[:, 0], a[1][:, 0], atol=1e-14)
    o, l = m(empty, empty)
    assert np.all(o == 0) and np.all(l == -np.inf)
    # Weights use lse differences: a shift of every lse by c leaves o unchanged and shifts lse by c.
    o1, l1 = m(a, b)
    o2, l2 = m((a[0], a[1] + 7.5), (b[0], b[1] + 7.5))
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + 7.5, atol=1e-12)


# --------------------------------------------------------- cache accounting

def test_kv_size_closed_form_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_size.json")))
    e = g["mha_fp16_example"]
    per_tok = oracle.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["bytes_per_elem"])
    assert per_tok == 1474560.0
    assert round(per_tok / 1e6, 2) == e["bytes_per_token_MB"]
    assert round(per_tok * 8192 / 1e9) == e["seq_8k_GB"]
    assert round(per_tok * 16384 / 1e9) == e["seq_16k_GB"]
    # FP8 halves the per-element bytes, which doubles the tokens a fixed budget holds.
    f = g["fp8_capacity"]
    ratio = oracle.kv_bytes_per_token(1, 1, 1, 2) / oracle.kv_bytes_per_token(1, 1, 1, 1)
    assert abs(f["fp8_tokens"] / f["bf16_tokens"] - ratio) < 0.01


def test_mla_pool_accounting_matches_generator_layout():
    assert oracle.mla_bytes_per_token(512, 64, 2) == 1152.0
    assert oracle.mla_bytes_per_token(512, 64, 1, 4) == 580.0
    for name in ("c1", "c1f8"):
        c = gen.CONFIGS["c1"] if name == "c1" else _fp8_small()
        inp = gen.make_inputs(c)
        slots = inp.num_pages * c.page_size
        nbytes = inp.kv.nbytes + (inp.kv_scale.nbytes if inp.kv_scale is not None else 0)
        elem = inp.kv.itemsize
        assert nbytes / slots == oracle.mla_bytes_per_token(c.d_latent, c.d_rope, elem, 4 if elem == 1 else 0)


# --------------------------------------------------------------- cache append

def _fp8_values():
    return np.array([oracle.fp8_e4m3_value(c) for c in range(256)])


def test_fp8_encode_round_trips_every_code():
    vals = _fp8_values()
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    codes = oracle.fp8_e4m3_encode(np.array([vals[c] for c in finite], np.float32))
    np.testing.assert_array_equal(codes, np.array(finite, np.uint8))
    assert oracle.fp8_e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_fp8_encode_ties_go_to_even_and_saturate():
    vals = _fp8_values()
    lo = np.arange(0x00, 0x7E)
    mids = ((vals[lo] + vals[lo + 1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[lo] + vals[lo + 1]) / 2)  # exact in fp32
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(mids), want)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(-mids), want | 0x80)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(up), (lo + 1).astype(np.uint8))
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(dn), lo.astype(np.uint8))
    big = np.array([448.0, 448.01, 463.9, 464.0, 1e6, np.inf, -500.0], np.float32)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(big), [0x7E] * 6 + [0xFE])
    tiny = np.array([2.0 ** -10, 2.0 ** -10 * 1.0001, -2.0 ** -11, -0.0], np.float32)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(tiny), [0x00, 0x01, 0x80, 0x80])


def test_fp8_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 200_000))
    q = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(q), ref)


def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(100_000).astype(np.float32) * np.exp2(rng.integers(-20, 20, 100_000))
    x = x.astype(np.float32)
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact halfway cases
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_encode(x), ref)


def _append_case(pool_dtype, dim=40, P=4, num_pages=6):
    rng = np.random.default_rng(7)
    bt = np.array([[3, 1], [0, 5], [2, 4]], np.int32)
    if pool_dtype == "fp8":
        pool = np.full((num_pages, P, dim), 0x55, np.uint8)
        sc = np.full((num_pages, P), 9.0, np.float32)
    elif pool_dtype == "bf16":
        pool, sc = np.full((num_pages, P, dim), 0x1234, np.uint16), None
    else:
        pool, sc = np.full((num_pages, P, dim), 9.0, np.float32), None
    return rng, bt, pool, sc


def test_cache_append_fp8_closed_forms():
    rng, bt, pool, sc = _append_case("fp8")
    dim, P = pool.shape[2], pool.shape[1]
    rows = np.zeros((3, dim), np.float32)
    rows[0, 7] = -3.25                            # one non-zero element
    x2 = rng.standard_normal(dim).astype(np.float32) * 5
    rows[2] = x2
    pos = np.array([5, 2, 6], np.int32)          # pages bt[0][1]=1 slot 1, bt[1][0]=0 slot 2, bt[2][1]=4 slot 2
    before = pool.copy(), sc.copy()
    st = oracle.cache_append(rows, pool, sc, bt, pos)
    assert not st.any()
    # request 0: scale = 3.25/448 in fp32, the element itself -> -448
    assert sc[1, 1] == np.float32(np.float32(3.25) / np.float32(448.0))
    want0 = np.zeros(dim, np.uint8)
    want0[7] = 0xFE
    np.testing.assert_array_equal(pool[1, 1], want0)
    # request 1: an all-zero row has scale 1 and zero codes
    assert sc[0, 2] == 1.0 and not pool[0, 2].any()
    # request 2: the amax element hits 448 exactly; all others are within half
    # an e4m3 step of x / scale (relative 2^-4 for normals, 2^-10 absolute below)
    s2 = sc[4, 2]
    assert s2 == np.float32(np.float32(np.abs(x2).max()) / np.float32(448.0))
    vals = _fp8_values()
    deq = vals[pool[4, 2]]
    q = x2.astype(np.float64) / np.float64(s2)
    j = int(np.argmax(np.abs(x2)))
    assert abs(deq[j]) == 448.0
    err = np.abs(deq - q)
    assert np.all(err <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))
    # every other slot is untouched
    changed = np.zeros(pool.shape[:2], bool)
    changed[1, 1] = changed[0, 2] = changed[4, 2] = True
    assert np.array_equal(pool[~changed], before[0][~changed]) and np.array_equal(sc[~changed], before[1][~changed])


@pytest.mark.parametrize("pool_dtype", ["bf16", "fp32"])
def test_cache_append_wide_pools(pool_dtype):
    rng, bt, pool, _ = _append_case(pool_dtype)
    dim = pool.shape[2]
    rows = rng.standard_normal((3, dim)).astype(np.float32)
    pos = np.array([0, 7, 3], np.int32)          # page 3 slot 0, page 5 slot 3, page 2 slot 3
    st = oracle.cache_append(rows, pool, None, bt, pos)
    assert not st.any()
    for b, (pg, sl) in enumerate([(3, 0), (5, 3), (2, 3)]):
        if pool_dtype == "bf16":
            ref = torch.from_numpy(rows[b]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            ref = rows[b]
        np.testing.assert_array_equal(pool[pg, sl], ref)
    # bf16 input rows into an FP8 pool decode exactly before quantising
    _, bt, p8, sc = _append_case("fp8")
    bits = gen.to_bf16_bits(rows)
    oracle.cache_append(bits, p8, sc, bt, pos)
    p8b, scb = _append_case("fp8")[2:]
    oracle.cache_append(gen.bf16_bits_to_f32(bits), p8b, scb, bt, pos)
    assert np.array_equal(p8, p8b) and np.array_equal(sc, scb)


def test_cache_append_status_and_skips():
    _, bt, pool, sc = _append_case("fp8")
    bt = bt.copy()
    bt[1, 1] = 99                                 # request 1's second page is not a pool page
    rows = np.ones((3, pool.shape[2]), np.float32)
    pos = np.array([-1, 6, 8], np.int32)          # skip; page 99; past the 2 mapped pages
    before = pool.copy(), sc.copy()
    st = oracle.cache_append(rows, pool, sc, bt, pos)
    assert list(st) == [0, oracle.BAD_PAGE, oracle.BAD_LEN]
    assert np.array_equal(pool, before[0]) and np.array_equal(sc, before[1])


# ------------------------------------------------------- page integrity check

def _tag_case(seed=3, B=6, P=16, stride=5):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, stride * P + 1, B).astype(np.int32)
    num_pages = B * stride + 4
    bt = rng.permutation(num_pages)[: B * stride].reshape(B, stride).astype(np.int32)
    page_tags = rng.integers(0, 2 ** 63, num_pages, dtype=np.uint64)
    bt_tags = page_tags[bt]
    return rng, lens, bt, bt_tags, page_tags, P


def test_page_check_closed_forms():
    rng, lens, bt, bt_tags, page_tags, P = _tag_case()
    assert not oracle.page_check(bt, bt_tags, lens, page_tags, P).any()
    # A reallocated page (new tag) flags exactly the requests whose length covers it.
    b, j = 2, (int(lens[2]) - 1) // P
    page_tags2 = page_tags.copy()
    page_tags2[bt[b, j]] ^= np.uint64(1)
    st = oracle.page_check(bt, bt_tags, lens, page_tags2, P)
    assert list(np.nonzero(st)[0]) == [b] and st[b] == oracle.BAD_TAG
    # Entries past a request's pages are never looked at.
    lens3 = lens.copy()
    lens3[0] = P                                  # one page
    bt3, tags3 = bt.copy(), bt_tags.copy()
    bt3[0, 1:] = -7
    tags3[0, 1:] = 12345
    assert not oracle.page_check(bt3, tags3, lens3, page_tags, P).any()
    # Bad page id, bad length, empty request.
    bt4 = bt.copy()
    bt4[1, 0] = 10 ** 6
    lens4 = lens.copy()
    lens4[3] = bt.shape[1] * P + 1
    lens4[4] = 0
    st = oracle.page_check(bt4, bt_tags, lens4, page_tags, P, max_len=bt.shape[1] * P + 1)
    assert st[1] == oracle.BAD_PAGE and st[3] == oracle.BAD_LEN and st[4] == 0
    assert st[0] == st[2] == st[5] == 0


def test_page_check_matches_numpy_brute_force():
    for seed in range(20):
        rng, lens, bt, bt_tags, page_tags, P = _tag_case(seed, B=12, stride=7)
        page_tags = page_tags.copy()
        flip = rng.choice(page_tags.size, 5, replace=False)
        page_tags[flip] += np.uint64(1)
        bt = bt.copy()
        bt[rng.integers(0, bt.shape[0]), rng.integers(0, bt.shape[1])] = -1
        pages = (lens + P - 1) // P
        used = np.arange(bt.shape[1])[None, :] < pages[:, None]
        bad_page = used & ((bt < 0) | (bt >= page_tags.size))
        safe = np.clip(bt, 0, page_tags.size - 1)
        bad_tag = used & ~bad_page & (page_tags[safe] != bt_tags)
        want = np.where(bad_page.any(1), oracle.BAD_PAGE, 0) | np.where(bad_tag.any(1), oracle.BAD_TAG, 0)
        np.testing.assert_array_equal(oracle.page_check(bt, bt_tags, lens, page_tags, P), want)


# ---------------------------------------------------------- multi-query step

def test_multi_query_step_matches_causal_brute_force():
    """Q new tokens per request with k >= L (every visible token selected):
    each query's attention equals a numpy softmax over the tokens a causal
    mask (numpy tril) leaves it, and its scores equal an einsum brute force on
    exactly those tokens; a request shorter than Q is flagged."""
    Q = 3
    cfg = gen.CONFIGS["c1"].with_(batch=3)
    inp = gen.make_inputs(cfg, lens=[37, 5, 2], shuffle=True)
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, Q, cfg.n_heads, cfg.dim)).astype(np.float32)
    q_idx = rng.standard_normal((3, Q, cfg.idx_heads, cfg.idx_dim)).astype(np.float32)
    w = rng.standard_normal((3, Q, cfg.idx_heads)).astype(np.float32)
    r = oracle.multi_query_step(q, q_idx, w, inp.kv, inp.kv_scale, inp.k_idx, inp.k_idx_scale, inp.block_table,
                                inp.lens, 64, cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    assert list(r["status"]) == [0, 0, oracle.BAD_LEN]
    P = cfg.page_size
    for b in range(2):
        L = int(inp.lens[b])
        rows = np.array([int(inp.block_table[b, t // P]) * P + t % P for t in range(L)])
        c = inp.kv.reshape(-1, cfg.dim)[rows].astype(np.float64)
        kk = inp.k_idx.reshape(-1, cfg.idx_dim)[rows].astype(np.float64)
        mask = np.tril(np.ones((L, L), bool))[L - Q:]         # row i: what position L-Q+i may see
        for i in range(Q):
            vis = mask[i]
            assert vis.sum() == L - Q + 1 + i
            dots = np.einsum("hd,td->ht", q_idx[b, i].astype(np.float64), kk)
            s_ref = np.einsum("h,ht->t", w[b, i].astype(np.float64), np.maximum(dots, 0.0))
            np.testing.assert_allclose(r["scores"][b, i, :vis.sum()], s_ref[vis], rtol=1e-12, atol=1e-12)
            z = cfg.softmax_scale * np.einsum("hd,td->ht", q[b, i].astype(np.float64), c)[:, vis]
            np.testing.assert_allclose(r["o"][b, i], softmax(z, axis=1) @ c[vis, :cfg.d_latent], rtol=1e-10,
                                       atol=1e-12)
            np.testing.assert_allclose(r["lse"][b, i], logsumexp(z, axis=1), rtol=1e-12)
            assert list(r["idx"][b, i, :vis.sum()]) == list(np.nonzero(vis)[0])
    assert np.isnan(r["o"][2]).all()


# ------------------------------------------------------------ prefill chunk

def test_prefill_chunk_matches_causal_brute_force_and_blocks_merge():
    """Dense causal attention of a chunk of new tokens: each query equals a
    numpy softmax over the tokens a tril mask leaves it; computing the context
    in 3 blocks and merging the block partials gives the same result."""
    Q = 4
    cfg = gen.CONFIGS["c1"].with_(batch=2)
    inp = gen.make_inputs(cfg, lens=[37, 100], shuffle=True)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, Q, cfg.n_heads, cfg.dim)).astype(np.float32)
    o1, l1, st = oracle.prefill_chunk_attention(q, inp.kv, inp.kv_scale, inp.block_table, inp.lens, cfg.n_heads,
                                                cfg.d_latent, cfg.d_rope, cfg.softmax_scale)
    o3, l3, _ = oracle.prefill_chunk_attention(q, inp.kv, inp.kv_scale, inp.block_table, inp.lens, cfg.n_heads,
                                               cfg.d_latent, cfg.d_rope, cfg.softmax_scale, blocks=3)
    assert not st.any()
    np.testing.assert_allclose(o3, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l3, l1, rtol=1e-13)
    P = cfg.page_size
    for b in range(2):
        L = int(inp.lens[b])
        rows = np.array([int(inp.block_table[b, t // P]) * P + t % P for t in range(L)])
        c = inp.kv.reshape(-1, cfg.dim)[rows].astype(np.float64)
        mask = np.tril(np.ones((L, L), bool))[L - Q:]
        for i in range(Q):
            z = cfg.softmax_scale * np.einsum("hd,td->ht", q[b, i].astype(np.float64), c)[:, mask[i]]
            np.testing.assert_allclose(o1[b, i], softmax(z, axis=1) @ c[mask[i], :cfg.d_latent], rtol=1e-10,
                                       atol=1e-12)
            np.testing.assert_allclose(l1[b, i], logsumexp(z, axis=1), rtol=1e-12)
