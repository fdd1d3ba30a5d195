"""GPU parity of kv_page_check against the oracle (status bits, bit for bit)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _lib():
    import sparse_paged_mla_amd as spm
    spm.load_library()
    return spm


def _case(B, lo, hi, P, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, B).astype(np.int32)
    stride = int((hi + P - 1) // P) + 3
    num_pages = int(((lens + P - 1) // P).sum()) + 11
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, stride), -1, np.int32)
    at = 0
    for b in range(B):
        n = (int(lens[b]) + P - 1) // P
        bt[b, :n] = perm[at:at + n]
        at += n
    page_tags = (np.arange(num_pages, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)) ^ np.uint64(seed)
    bt_tags = np.where(bt >= 0, page_tags[np.clip(bt, 0, None)], np.uint64(0)).astype(np.uint64)
    return rng, lens, bt, bt_tags, page_tags


def _run(spm, lens, bt, bt_tags, page_tags, P, max_len, pre=None):
    B = lens.shape[0]
    status = torch.zeros(B, dtype=torch.int32, device="cuda") if pre is None else torch.from_numpy(pre).cuda()
    spm.kv_page_check(torch.from_numpy(bt).cuda(), torch.from_numpy(bt_tags.view(np.int64)).cuda(),
                      torch.from_numpy(lens).cuda(), max_len, torch.from_numpy(page_tags.view(np.int64)).cuda(), P,
                      status)
    torch.cuda.synchronize()
    return status.cpu().numpy()


@pytest.mark.parametrize("P", [16, 64])
def test_page_check_c3f_shapes(P):
    """64 requests of 32K-128K tokens: clean, then with stale tags at the first,
    a middle and the last covered page, a bad page id, a bad length, and
    garbage past a request's pages (never read)."""
    spm = _lib()
    rng, lens, bt, bt_tags, page_tags = _case(64, 32768, 131072, P, seed=P)
    max_len = int(lens.max())
    print(f"[page_check] P={P} clean", flush=True)
    got = _run(spm, lens, bt, bt_tags, page_tags, P, max_len)
    assert not got.any()
    pt = page_tags.copy()
    bt2, tags2, lens2 = bt.copy(), bt_tags.copy(), lens.copy()
    last = (lens + P - 1) // P - 1
    pt[bt[3, 0]] += np.uint64(1)                    # reallocated page: first page of request 3
    pt[bt[10, last[10] // 2]] ^= np.uint64(1 << 40)  # a middle page of request 10
    tags2[20, last[20]] += np.uint64(7)             # stale recorded tag: last page of request 20
    bt2[30, 5] = 10 ** 8                             # page id out of range
    bt2[31, 7] = -1
    lens2[40] = bt.shape[1] * P + 5                  # longer than its table
    bt2[50, last[50] + 1:] = 10 ** 8                 # garbage past the last page: not read
    tags2[50, last[50] + 1:] = 99
    ml = int(lens2.max())
    print(f"[page_check] P={P} faults", flush=True)
    got = _run(spm, lens2, bt2, tags2, pt, P, ml)
    want = oracle.page_check(bt2, tags2, lens2, pt, P, max_len=ml)
    np.testing.assert_array_equal(got, want)
    assert set(np.nonzero(got)[0]) == {3, 10, 20, 30, 31, 40}
    assert got[3] == spm.BAD_TAG and got[30] == spm.BAD_PAGE and got[40] == spm.BAD_LEN


def test_page_check_random_against_oracle_and_keeps_earlier_bits():
    spm = _lib()
    P = 16
    rng, lens, bt, bt_tags, page_tags = _case(200, 0, 3000, P, seed=4)
    for trial in range(5):
        pt = page_tags.copy()
        flip = rng.choice(pt.size, 25, replace=False)
        pt[flip] ^= np.uint64(1) << np.uint64(trial)
        bt2 = bt.copy()
        bt2[rng.integers(0, 200, 5), rng.integers(0, 10, 5)] = -3
        pre = (rng.integers(0, 2, 200) * spm.BAD_INDEX).astype(np.int32)
        max_len = int(lens.max()) if trial else int(lens.max()) - 1   # trial 0: the longest requests are too long
        print(f"[page_check] random trial {trial}", flush=True)
        got = _run(spm, lens, bt2, bt_tags, pt, P, max_len, pre=pre)
        want = oracle.page_check(bt2, bt_tags, lens, pt, P, max_len=max_len) | pre
        np.testing.assert_array_equal(got, want)
