"""topk_select_noalloc (the top-k call with the library's static device
workspace) against topk_select with a caller workspace, through the C ABI:
bit-identical indices on two calls in a row, the second with a smaller input,
both taking the multi-launch path that uses the workspace; and sizes beyond
the static workspace rejected with nothing enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from tests import parity

pytestmark = pytest.mark.gpu


def _lib():
    import sparse_paged_mla_amd as spm
    spm.load_library()
    return spm


def _scores(rng, lens, stride):
    S = rng.standard_normal((len(lens), stride)).astype(np.float32) * 3 + 10
    S[0, ::11] = np.round(S[0, ::11])  # ties
    return S


def _both(spm, S, lens, k, max_len):
    s = torch.from_numpy(S).cuda()
    l = torch.tensor(lens, dtype=torch.int32, device="cuda")
    B = len(lens)
    ref = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(spm.topk_workspace_bytes(B, max_len, k), 256), dtype=torch.uint8, device="cuda")
    st_ref = torch.zeros(B, dtype=torch.int32, device="cuda")
    spm.topk_select(s, l, max_len, k, ref, ws, st_ref)
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    spm.topk_select_noalloc(s, l, max_len, k, out, st)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy(), st_ref.cpu().numpy(), st.cpu().numpy()


def test_noalloc_matches_topk_select_twice():
    spm = _lib()
    rng = np.random.default_rng(77)
    # Call 1: rows past the one-launch limit (max_len > 65536), a short one
    # and one of at most one chunk among them.
    lens1 = [131000, 90000, 40000, 7000, 2049, 1500]
    S1 = _scores(rng, lens1, 131072)
    need1 = spm.topk_workspace_bytes(len(lens1), max(lens1), 2048)
    assert 0 < need1 <= 32 << 20
    print(f"[no-alloc] call 1: B={len(lens1)} max_len={max(lens1)} k=2048 workspace {need1} bytes", flush=True)
    ref, out, st_ref, st = _both(spm, S1, lens1, 2048, max(lens1))
    assert not st_ref.any() and not st.any()
    np.testing.assert_array_equal(out, ref)
    parity.check_topk_exact(out, S1, np.array(lens1), 2048, "no-alloc call 1")
    # Call 2, smaller: fewer requests, shorter rows, a smaller k and a row
    # stride that is not a multiple of 4 floats (the multi-launch path again).
    lens2 = [20000, 9000, 300]
    S2 = _scores(rng, lens2, 20001)
    print(f"[no-alloc] call 2: B={len(lens2)} max_len={max(lens2)} k=512", flush=True)
    ref, out, st_ref, st = _both(spm, S2, lens2, 512, max(lens2))
    assert not st_ref.any() and not st.any()
    np.testing.assert_array_equal(out, ref)
    parity.check_topk_exact(out, S2, np.array(lens2), 512, "no-alloc call 2")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    spm = _lib()
    lib = spm.load_library()
    B, max_len, k = 1024, 1 << 20, 2048
    assert spm.topk_workspace_bytes(B, max_len, k) > 32 << 20
    out = torch.full((4, k), -7, dtype=torch.int32, device="cuda")
    s = torch.zeros(4, 16, device="cuda")
    l = torch.zeros(4, dtype=torch.int32, device="cuda")
    # Pointers to small buffers: the call must reject the sizes before it
    # reads or writes anything.
    rc = lib.topk_select_noalloc(ctypes.c_void_p(s.data_ptr()), max_len, ctypes.c_void_p(l.data_ptr()), B, max_len, k,
                                 ctypes.c_void_p(out.data_ptr()), None, None)
    assert rc == -4, rc  # SPMLA_EWORKSPACE
    assert b"static scratch" in lib.spmla_last_error()
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -7).all()
