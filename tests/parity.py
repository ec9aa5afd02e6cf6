"""Acceptance rules for comparing the HIP path with the fp64 oracle.

* Summaries: bit-exact (both sides compute RNE(fl64(fl64 sum / n))).
* Block selection: the GPU's set may differ from the oracle's only at blocks
  whose fp64 relevance lies within 1e-5 * max|relevance| of the row's k-th
  largest value (a "near tie"); such swaps are counted and reported.
* Attention outputs: compared with the oracle's attention over the GPU's own
  selection, max |out - ref| <= 2e-3 and max |lse - ref| <= 1e-3.
* Votes: may differ from the oracle's only at tokens inside some head's near-
  tie band around its per-head threshold, by at most the number of such heads;
  the token set must be exactly the integer rule applied to the GPU's votes.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TIE = 1e-5
OUT_TOL = 2e-3
LSE_TOL = 1e-3


def check_block_selection(gpu_idx: np.ndarray, raw: np.ndarray, k: int):
    """gpu_idx [rows, keff] int32, raw fp64 relevance [rows, NB].  Returns the
    number of near-tie swaps; raises AssertionError on any other mismatch."""
    rows, nb = raw.shape
    keff = min(k, nb)
    gpu_idx = gpu_idx.reshape(rows, keff)
    assert np.all(np.diff(gpu_idx, axis=1) > 0), "block_idx rows must be strictly ascending"
    assert gpu_idx.min() >= 0 and gpu_idx.max() < nb
    ref = oracle.topk(raw, k)
    swaps = 0
    for r in range(rows):
        gs, os_ = set(gpu_idx[r].tolist()), set(ref[r].tolist())
        if gs == os_:
            continue
        thr = np.sort(raw[r])[::-1][keff - 1]
        tol = REL_TIE * np.abs(raw[r]).max()
        for j in gs ^ os_:
            assert abs(raw[r, j] - thr) <= tol, (
                "row %d: block %d (score %.9g) swapped with a gap %.3g > %.3g to the threshold %.9g"
                % (r, j, raw[r, j], abs(raw[r, j] - thr), tol, thr))
        swaps += len(gs - os_)
    return swaps


def check_attention(out, lse, ref_out, ref_lse, tol=OUT_TOL, lse_tol=LSE_TOL):
    err = float(np.abs(out.astype(np.float64) - ref_out).max())
    assert err <= tol, "max |out - oracle| = %.3g > %.3g" % (err, tol)
    lerr = 0.0
    if lse is not None:
        lerr = float(np.abs(lse.astype(np.float64) - ref_lse).max())
        assert lerr <= lse_tol, "max |lse - oracle| = %.3g > %.3g" % (lerr, lse_tol)
    return err, lerr


def check_votes(gpu_votes: np.ndarray, gpu_idx: np.ndarray, logits: np.ndarray, N: int, W: int,
                exact: bool = False):
    """gpu_votes [B,T] (uint8), gpu_idx [B,min(N,T)], oracle logits [B,Hq,T]."""
    B, Hq, T = logits.shape
    ref_votes = oracle.votes(logits, N, W)
    gv = gpu_votes.astype(np.int32)
    # the set is the exact integer rule applied to the GPU's own votes
    expect = oracle.set_from_votes(gv, N, W)
    np.testing.assert_array_equal(gpu_idx, expect)
    if exact:
        np.testing.assert_array_equal(gv, ref_votes)
        return 0
    if T <= N:
        assert gv.sum() == 0
        return 0
    C, Kv = T - W, N - W
    diff = np.abs(gv - ref_votes)
    if not diff.any():
        return 0
    allowed = np.zeros((B, T), np.int32)
    for b in range(B):
        for h in range(Hq):
            lg = logits[b, h, :C]
            thr = np.sort(lg)[::-1][Kv - 1]
            tol = REL_TIE * np.abs(lg).max()
            allowed[b, :C] += (np.abs(lg - thr) <= tol).astype(np.int32)
    bad = diff > allowed
    assert not bad.any(), "votes differ beyond the near-tie bands at %s" % (np.argwhere(bad)[:8],)
    return int(diff.sum())
