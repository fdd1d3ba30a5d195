"""GPU parity of kv_cache_append (quantise-on-write) against the oracle.

Codes, scales and bf16 bits are compared bit for bit over the whole pool, so
a write to a wrong slot, or any write beyond the target slots, fails too.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _lib():
    import sparse_paged_mla_amd as spm
    spm.load_library()
    return spm


def _layout(B, pages_per_req, P, seed, spare=7):
    """Block table over a shuffled pool with a few unused pages."""
    rng = np.random.default_rng(seed)
    num_pages = B * pages_per_req + spare
    perm = rng.permutation(num_pages)[: B * pages_per_req].astype(np.int32)
    return rng, perm.reshape(B, pages_per_req), num_pages


def _rows(rng, B, dim):
    """Rows with per-row magnitudes from 1e-3 to 1e3, plus special rows."""
    x = rng.standard_normal((B, dim)).astype(np.float32) * np.exp(rng.uniform(-7, 7, (B, 1))).astype(np.float32)
    x[0] = 0.0                                  # all-zero row: scale 1
    x[1] = 0.0
    x[1, 5] = -2.5                              # one non-zero element
    x[2, ::3] = -0.0                            # negative zeros among ordinary values
    return x


def _run(spm, rows_np, row_kind, pool_kind, bt, num_pages, P, pos, seed):
    B, dim = rows_np.shape
    rng = np.random.default_rng(seed + 1)
    if pool_kind == "fp8":
        pool = rng.integers(0, 256, (num_pages, P, dim), dtype=np.uint8)
        sc = rng.standard_normal((num_pages, P)).astype(np.float32)
    elif pool_kind == "bf16":
        pool = rng.integers(0, 1 << 16, (num_pages, P, dim), dtype=np.uint16)
        sc = None
    else:
        pool = rng.standard_normal((num_pages, P, dim)).astype(np.float32)
        sc = None
    if row_kind == "bf16":
        bits = (rows_np.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 values do
        rows_in = bits
        rows_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        rows_in = rows_np
        rows_t = torch.from_numpy(rows_np).cuda()
    ref_pool, ref_sc = pool.copy(), None if sc is None else sc.copy()
    ref_st = oracle.cache_append(rows_in, ref_pool, ref_sc, bt, pos)
    pool_t = torch.from_numpy(pool.view(np.int16) if pool_kind == "bf16" else pool).cuda()
    if pool_kind == "bf16":
        pool_t = pool_t.view(torch.bfloat16)
    sc_t = None if sc is None else torch.from_numpy(sc).cuda()
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    spm.kv_cache_append(rows_t, pool_t, sc_t, torch.from_numpy(bt).cuda(), torch.from_numpy(pos).cuda(), status)
    torch.cuda.synchronize()
    got = pool_t.view(torch.int16).cpu().numpy().view(np.uint16) if pool_kind == "bf16" else pool_t.cpu().numpy()
    assert np.array_equal(status.cpu().numpy(), ref_st)
    diff = np.argwhere(got != ref_pool)
    assert diff.size == 0, f"{len(diff)} pool elements differ, first at {diff[:4].tolist()}"
    if sc is not None:
        assert np.array_equal(sc_t.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
    return ref_st


@pytest.mark.parametrize("dim", [576, 128, 4096])
@pytest.mark.parametrize("row_kind", ["bf16", "fp32"])
def test_append_fp8_bit_exact(dim, row_kind):
    """The c3f shapes (64 requests; latent rows of 576, indexer keys of 128;
    page 64) and the largest row."""
    spm = _lib()
    B, P = 64, 64
    rng, bt, num_pages = _layout(B, 3, P, seed=dim)
    print(f"[append] fp8 dim={dim} rows={row_kind}", flush=True)
    rows = _rows(rng, B, dim)
    pos = rng.integers(0, 3 * P, B).astype(np.int32)
    pos[3] = -1                                # skipped request
    _run(spm, rows, row_kind, "fp8", bt, num_pages, P, pos, seed=dim)


def test_append_fp8_ties_and_extremes():
    """Rows whose absmax is 448 have scale exactly 1, so x / s = x: the
    quotients then sit exactly on midpoints between e4m3 codes (ties to the
    even code), one fp32 step either side of them, in the subnormal range, and
    at the top of the range."""
    spm = _lib()
    vals = np.array([oracle.fp8_e4m3_value(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    cand = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           vals.astype(np.float32), [0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 447.9, 440.0]]).astype(np.float32)
    dim = 128
    n_rows = (len(cand) + dim - 2) // (dim - 1)
    rows = np.zeros((n_rows, dim), np.float32)
    flat = np.resize(cand, n_rows * (dim - 1)).reshape(n_rows, dim - 1)
    sign = np.where(np.arange(flat.size).reshape(flat.shape) % 2 == 0, 1.0, -1.0).astype(np.float32)
    rows[:, :-1] = flat * sign
    rows[:, -1] = 448.0                         # scale exactly 1
    P = 16
    rng, bt, num_pages = _layout(n_rows, 1, P, seed=11)
    pos = rng.integers(0, P, n_rows).astype(np.int32)
    print(f"[append] ties rows={n_rows}", flush=True)
    _run(spm, rows, "fp32", "fp8", bt, num_pages, P, pos, seed=11)


@pytest.mark.parametrize("pool_kind", ["bf16", "fp32"])
@pytest.mark.parametrize("row_kind", ["bf16", "fp32"])
def test_append_wide_pools(pool_kind, row_kind):
    spm = _lib()
    B, P, dim = 8, 16, 80
    rng, bt, num_pages = _layout(B, 2, P, seed=5)
    rows = _rows(rng, B, dim)
    rows[4, :8] = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0e38, 1e-40, -1e-42,
                            0.1, 0.2], np.float32)  # bf16 ties, a huge value, subnormals
    pos = rng.integers(0, 2 * P, B).astype(np.int32)
    print(f"[append] {pool_kind} pool rows={row_kind}", flush=True)
    _run(spm, rows, row_kind, pool_kind, bt, num_pages, P, pos, seed=5)


def test_append_flags_bad_requests_and_writes_nothing_for_them():
    spm = _lib()
    B, P, dim = 6, 16, 64
    rng, bt, num_pages = _layout(B, 2, P, seed=9)
    bt = bt.copy()
    bt[1, 1] = num_pages + 3                    # not a pool page
    bt[2, 0] = -5
    rows = _rows(rng, B, dim)
    pos = np.array([3, 20, 0, 32, -1, 31], np.int32)  # request 3: past its two mapped pages
    print("[append] bad requests", flush=True)
    st = _run(spm, rows, "fp32", "fp8", bt, num_pages, P, pos, seed=9)
    assert list(st) == [0, oracle.BAD_PAGE, oracle.BAD_PAGE, oracle.BAD_LEN, 0, 0]


def test_append_pair_one_launch_bit_exact():
    """Latent rows and indexer keys of the same tokens in one launch (the c3f
    shapes), each pool bit for bit against the oracle; a bad page and a
    skipped request."""
    spm = _lib()
    B, P = 64, 64
    rng, bt, num_pages = _layout(B, 3, P, seed=31)
    bt = bt.copy()
    bt[5, 1] = num_pages + 2
    rows_kv, rows_ix = _rows(rng, B, 576), _rows(rng, B, 128)
    pos = rng.integers(0, 3 * P, B).astype(np.int32)
    pos[5] = 70                               # page 1 of request 5: not a pool page
    pos[6] = -1
    bits_kv, bits_ix = gen_bits(rows_kv), gen_bits(rows_ix)
    pools, scales, refs = [], [], []
    for dim, bits in ((576, bits_kv), (128, bits_ix)):
        pool = rng.integers(0, 256, (num_pages, P, dim), dtype=np.uint8)
        sc = rng.standard_normal((num_pages, P)).astype(np.float32)
        rp, rs = pool.copy(), sc.copy()
        st_ref = oracle.cache_append(bits, rp, rs, bt, pos)
        pools.append(torch.from_numpy(pool).cuda())
        scales.append(torch.from_numpy(sc).cuda())
        refs.append((rp, rs, st_ref))
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    print("[append] pair", flush=True)
    spm.kv_cache_append_pair(bf16_tensor(bits_kv), pools[0], scales[0], bf16_tensor(bits_ix), pools[1], scales[1],
                             torch.from_numpy(bt).cuda(), torch.from_numpy(pos).cuda(), status)
    torch.cuda.synchronize()
    for k in range(2):
        rp, rs, st_ref = refs[k]
        assert np.array_equal(pools[k].cpu().numpy(), rp)
        assert np.array_equal(scales[k].cpu().numpy().view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(status.cpu().numpy(), st_ref)
    assert status.cpu().numpy()[5] == oracle.BAD_PAGE


def gen_bits(rows):
    return (rows.view(np.uint32) >> 16).astype(np.uint16)


def bf16_tensor(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
