"""Shared parity checks between the HIP path and the oracle (used by the GPU tests).

Tolerances (stated once, here):
 - indexer scores: |s_gpu - s_ref| <= 1e-4 * max(|s_ref|, A_t), where
   A_t = sum_h |w_h| sum_i |q_h,i k_t,i| is the size of the terms an fp32
   accumulation adds (it stands in for |s_ref| when the terms cancel to near
   zero); and, for scores not dominated by cancellation
   (|s_ref| >= 1e-2 A_t), the plain relative error |ds| / |s_ref| <= 1e-4.
 - top-k: bit-exact against the oracle's top-k applied to the GPU's own fp32
   score array (so a score rounding difference cannot masquerade as a
   selection error).
 - attention: max |o_gpu - o_ref| <= 1e-2 and |lse_gpu - lse_ref| <= 1e-3 |lse_ref|,
   the oracle attending exactly the GPU-selected token set.  |lse_ref| is
   floored at 1 so that a one-token set whose logit happens to be near 0
   is not held to an absolute 1e-6 (every workload lse is >= 3 anyway).
"""
import numpy as np

import oracle

SCORE_RTOL = 1e-4
O_ATOL = 1e-2
LSE_RTOL = 1e-3


def check_scores(s_gpu, s_ref, mags, what=""):
    s_gpu = np.asarray(s_gpu, np.float64)
    err = np.abs(s_gpu - s_ref)
    bound = SCORE_RTOL * np.maximum(np.abs(s_ref), mags)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} scores outside tolerance; worst err {err[bad].max()}"
    plain = np.abs(s_ref) >= 1e-2 * mags
    if plain.any():
        rel = err[plain] / np.abs(s_ref[plain])
        assert rel.max() <= SCORE_RTOL, f"{what}: plain relative error {rel.max()}"
    return float(err.max()) if err.size else 0.0


def check_topk_exact(idx_gpu, scores_gpu, lens, k, what=""):
    ref = oracle.topk(np.asarray(scores_gpu, np.float64), lens, k)
    mism = np.nonzero((np.asarray(idx_gpu) != ref).any(axis=1))[0]
    assert len(mism) == 0, f"{what}: top-k differs for requests {mism[:8]}"


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: finiteness of lse differs"
    assert np.array_equal(lse_gpu[~fin], lse_ref[~fin]), f"{what}: -inf/nan lse differs"
    d_o = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    assert d_o <= O_ATOL, f"{what}: max |do| = {d_o}"
    if fin.any():
        rel = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(np.abs(lse_ref[fin]), 1.0)
        assert rel.max() <= LSE_RTOL, f"{what}: max lse rel err {rel.max()}"
    return float(d_o)
