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
 - attention, relative RMS (the workload's 1e-2 max-abs allows tens of per
   cent on outputs of size 0.03, so a second, relative check is kept): the
   kernels carry each softmax weight to the value contraction with 8
   significant bits (relative rounding error <= 2^-9 per weight, the only
   rounding on the path that is not far smaller), and o = sum_t p_t v_t /
   sum_t p_t.  With independent roundings delta_t the error of o is
   sum_t p_t delta_t (v_t - o) / sum_t p_t, whose RMS is at most 2^-9 times
   the RMS of o's own spread; rms(o_gpu - o_ref) <= 2^-8 rms(o_ref) (twice
   that) is asserted.  A missing token, a lost scale or a transposed
   operand moves o by far more than that.
"""
import numpy as np

import oracle

SCORE_RTOL = 1e-4
O_ATOL = 1e-2
LSE_RTOL = 1e-3
O_REL_RMS = 2.0 ** -8


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
        r = rel_rms(o_gpu[fin], o_ref[fin])
        assert r <= O_REL_RMS, f"{what}: relative RMS error of o {r:.3e} > 2^-8"
    return float(d_o)


def rel_rms(o_gpu, o_ref):
    """rms(o_gpu - o_ref) / rms(o_ref) over the given rows (0 when o_ref is 0)."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    den = np.sqrt(np.mean(o_ref ** 2)) if o_ref.size else 0.0
    num = np.sqrt(np.mean((o_gpu - o_ref) ** 2)) if o_ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def end_to_end(idx_gpu, o_gpu, s_ref, lens, k, oracle_attention):
    """Diagnostic only (nothing asserted): the oracle's own path -- top-k of
    its fp64 scores, then attention over that selection -- against the GPU.
    Returns the number of selected tokens that differ (tokens the GPU picked
    that the fp64 ranking would not, summed over requests: swaps at the
    selection boundary caused by fp32 score rounding), the max |do| and the
    relative RMS of o against the oracle's end-to-end o.
    oracle_attention(idx) must return the oracle's (o, lse) over idx."""
    idx_ref = oracle.topk(np.asarray(s_ref, np.float64), lens, k)
    swaps = 0
    for b in range(len(lens)):
        a = set(int(x) for x in np.asarray(idx_gpu)[b] if x >= 0)
        r = set(int(x) for x in idx_ref[b] if x >= 0)
        swaps += len(a - r)
    o_ref, _ = oracle_attention(idx_ref)
    o_gpu = np.asarray(o_gpu, np.float64)
    ok = np.isfinite(o_ref).all(axis=-1)
    d_o = float(np.abs(o_gpu[ok] - o_ref[ok]).max()) if ok.any() else 0.0
    return {"swaps": swaps, "selected": int(sum(min(k, int(L)) for L in lens)), "max_abs_do": d_o,
            "rel_rms_o": rel_rms(o_gpu[ok], o_ref[ok])}
