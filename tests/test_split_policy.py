"""The host-side split policy against the decode kernels' own workgroup
order.  `wg_coord` (csrc/decode_ws.h) is compiled for the host and its
map from workgroup id to (request, split, head group) is checked: it is a
bijection for equal and fixed-length splits, a pair's head-group workgroups
share an XCD in every full round, and the per-XCD count of workgroups with
work that `balanced_splits` relies on (`_busy_per_xcd`) is the count this
order produces (the hardware deals workgroup ids round-robin over the 8
XCDs, so id i runs on XCD i mod 8)."""
import os
import subprocess

import numpy as np
import pytest

import spmla_gen as gen
from sparse_paged_mla_amd.step import _busy_per_xcd, balanced_splits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def order(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = tmp_path_factory.mktemp("wg") / "wg_coord_dump"
    src = os.path.join(ROOT, "tests", "host_mapping", "wg_coord_dump.cpp")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-x", "hip", src,
                    "-I", os.path.join(ROOT, "sparse_paged_mla_amd", "csrc"), "-o", str(exe)],
                   check=True, capture_output=True)

    def run(batch, num_splits, n_hg, spread):
        out = subprocess.run([str(exe), str(batch), str(num_splits), str(n_hg), str(int(spread))],
                             check=True, capture_output=True, text=True).stdout
        return np.array([[int(x) for x in line.split()] for line in out.splitlines()], dtype=np.int64).reshape(-1, 3)
    return run


GRIDS = [(1, 1, 1), (3, 2, 2), (32, 6, 2), (64, 2, 2), (5, 7, 4), (128, 1, 2), (4, 8, 4), (33, 3, 1), (7, 1, 4)]


@pytest.mark.parametrize("spread", [False, True])
@pytest.mark.parametrize("batch,num_splits,n_hg", GRIDS)
def test_workgroup_order_is_a_bijection(order, batch, num_splits, n_hg, spread):
    m = order(batch, num_splits, n_hg, spread)
    n = batch * num_splits * n_hg
    assert m.shape == (n, 3)
    assert ((m[:, 0] >= 0) & (m[:, 0] < batch)).all()
    assert ((m[:, 1] >= 0) & (m[:, 1] < num_splits)).all()
    assert ((m[:, 2] >= 0) & (m[:, 2] < n_hg)).all()
    keys = (m[:, 0] * num_splits + m[:, 1]) * n_hg + m[:, 2]
    assert np.array_equal(np.sort(keys), np.arange(n))


@pytest.mark.parametrize("batch,num_splits,n_hg", GRIDS)
def test_head_groups_of_a_pair_share_an_xcd(order, batch, num_splits, n_hg):
    """Fixed-length order: in every full round of 8 pairs the n_hg
    workgroups of a (request, split) pair run on one XCD (they read the same
    rows, so they share its L2)."""
    m = order(batch, num_splits, n_hg, True)
    full_ids = (batch * num_splits // 8) * 8 * n_hg
    xcd_of = {}
    for bid in range(full_ids):
        b, s, _ = m[bid]
        xcd_of.setdefault((b, s), set()).add(bid % 8)
    assert all(len(x) == 1 for x in xcd_of.values())


def _lens_cases():
    c2 = gen.CONFIGS["c2"]
    cases = [("c2", [int(x) for x in gen.draw_lengths(c2)])]
    for seed in range(4):
        rng = np.random.default_rng(seed)
        B = int(rng.integers(3, 96))
        cases.append((f"ragged{seed}", [int(x) for x in rng.integers(0, 9000, size=B)]))
    cases.append(("with_empty", [0, 5, 8192, 0, 1024, 3000, 7777, 64]))
    return cases


@pytest.mark.parametrize("name,lens", _lens_cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_busy_per_xcd_is_what_the_order_gives(order, name, lens):
    num_splits, c = balanced_splits(lens, 128)
    n_hg = 2
    m = order(len(lens), num_splits, n_hg, True)
    busy = [0] * 8
    for bid, (b, s, _) in enumerate(m):
        if s * c < lens[b]:  # the kernels' non-empty split at a fixed split length c
            busy[bid % 8] += 1
    assert busy == _busy_per_xcd(lens, c, num_splits, n_hg)
    if c < max(lens):
        assert max(busy) <= 256 // 8
