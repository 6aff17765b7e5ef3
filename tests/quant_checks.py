"""Checks of RVQ encodings and codebook fits where more than one answer is correct.

The residual encoder's decision (the nearest of 256 entries) is unique only when the best and
second-best squared distances are further apart than the rounding of the precision the decision is
taken in.  The GPU takes it in fp32 (differences, squares and the 8-term sum rounded, and, after
stage 0, a residual rounded at each subtraction); the oracle in fp64.  With u = 2^-24 the fp32
error of a distance difference d2 - d1 is below 12 u (d1 + d2) + 4 u N, where N is the largest
squared norm of the stage inputs so far (the arithmetic adds at most 10 u per distance, the
rounded residual moves a difference by at most 2 |eps| (sqrt d1 + sqrt d2) with |eps| <= 2 u sqrt N).
So a decision is a near-tie, where either entry is a correct answer, when

    d2 - d1 <= TIE * (d1 + d2 + N),   TIE = 2^-16   (16x the bound above).

Everything here is numpy in fp64 on the caller's arrays; nothing calls the oracle or the GPU.
"""
import math

import numpy as np

TIE = 2.0 ** -16


def stage_distances(V, C):
    """Squared distances [n, 256] of rows V [n, 8] to the entries C [256, 8], fp64."""
    V = np.asarray(V, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    return (V * V).sum(1)[:, None] - 2.0 * V @ C.T + (C * C).sum(1)[None, :]


def exact_stage_distances(V, C):
    V = np.asarray(V, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    return ((V[:, None, :] - C[None, :, :]) ** 2).sum(axis=2)


def check_path(W, cb, codes, groups=None):
    """Along each group's own codes: every stage's pick is the nearest entry to that group's exact
    residual, or within TIE of it.  Returns the number of decisions that were not the unique nearest
    (near-ties the codes resolved either way).  Raises AssertionError on a pick outside the bound."""
    V = np.asarray(W, dtype=np.float32).reshape(-1, 8).astype(np.float64)
    C = np.asarray(codes).reshape(-1, 3)
    if groups is not None:
        V, C = V[groups], C[groups]
    nmax = (V * V).sum(1)
    ties = 0
    for s in range(3):
        c = C[:, s].astype(np.int64)
        nmax = np.maximum(nmax, (V * V).sum(1))
        for i in range(0, len(V), 4096):
            D = exact_stage_distances(V[i:i + 4096], cb[s])
            sl = slice(i, i + 4096)
            pick = D[np.arange(len(D)), c[sl]]
            d1 = D.min(axis=1)
            bad = pick - d1 > TIE * (pick + d1 + nmax[sl])
            assert not bad.any(), (s, i + np.flatnonzero(bad)[:5])
            ties += int((c[sl] != D.argmin(axis=1)).sum())
        V = V - np.asarray(cb[s], dtype=np.float64)[c]
    return ties


def compare_with_oracle_codes(W, cb, got, want, margins):
    """GPU codes `got` against the oracle's `want` (with its margins): every group equal, except groups
    whose first differing stage is an oracle near-tie; those groups are then checked along the GPU's
    own path.  Returns the number of such groups."""
    G = np.asarray(got).reshape(-1, 3)
    O = np.asarray(want).reshape(-1, 3)
    M = np.asarray(margins).reshape(-1, 3, 3)
    diff = np.flatnonzero(np.any(G != O, axis=1))
    if diff.size == 0:
        return 0
    s0 = np.argmax(G[diff] != O[diff], axis=1)
    d1, d2 = M[diff, s0, 0], M[diff, s0, 1]
    nmax = np.array([M[i, :s + 1, 2].max() for i, s in zip(diff, s0)])
    far = d2 - d1 > TIE * (d1 + d2 + nmax)
    assert not far.any(), ("code differs at a decision the oracle finds unique", diff[far][:5], s0[far][:5])
    check_path(W, cb, got, groups=diff)
    return int(diff.size)


def fsum_means(X, assign, n_centroids=256):
    """Correctly rounded means (math.fsum, then one rounding to fp32) of the rows of X [n, 8] per
    centroid; None where a centroid has no members."""
    X = np.asarray(X, dtype=np.float64)
    out = [None] * n_centroids
    order = np.argsort(assign, kind="stable")
    a = np.asarray(assign)[order]
    bounds = np.searchsorted(a, np.arange(n_centroids + 1))
    for c in range(n_centroids):
        m = order[bounds[c]:bounds[c + 1]]
        if m.size:
            out[c] = np.array([math.fsum(X[m, j]) / m.size for j in range(X.shape[1])], dtype=np.float32)
    return out


def ulps_apart(a, b):
    """|a - b| in units of the fp32 spacing at the larger magnitude (elementwise)."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)))
    return np.abs(a.astype(np.float64) - b.astype(np.float64)) / sp.astype(np.float64)
