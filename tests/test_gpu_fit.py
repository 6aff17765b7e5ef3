"""Codebook fitting on the GPU (rvq_fit, residual k-means).

The oracle fits with the plain definition (fp64 distances and residuals, one fp64 sum per mean in
index order); the GPU takes the nearest-entry decisions in fp32 and sums each mean in runs.  The two
agree bit for bit where every value is exact (the lattices below).  On Gaussian weights, where
near-ties make more than one assignment correct and a flipped one changes a later mean, the GPU fit is
checked by what defines it, one Lloyd step at a time:
  * its codes are the nearest-entry decisions with its own codebooks, along its own residual path
    (each pick the nearest, or within the fp32 rounding bound of it: tests/quant_checks.py);
  * stage 0's centroids after K iterations are the correctly rounded means (within one fp32 ulp) of
    the members that a (K - 1)-iteration run's last assignment gave them; empty ones keep their value;
  * with no iteration each stage starts at the named residual sub-vectors; with one iteration each
    stage's centroids are the means of the members of its first assignment (decided here in fp64
    from those starts; centroids that a near-tie could have given another member are skipped);
  * the fit's squared error is within 1 % of the oracle's;
  * a repeated run, and a run on a reused workspace, give the same bits (determinism, not parity).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
from quant_checks import TIE, check_path, fsum_means, stage_distances, ulps_apart
from test_oracle_pins import _lattice_data

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _input(rows, cols, seed, dup=32):
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    n = rows * cols // 8
    init = np.stack([rng.choice(n, 256, replace=n < 256) for _ in range(3)]).astype(np.int32)
    init[1, 256 - dup:] = init[1, :dup]   # repeated starts (centroids that begin without members)
    return W, init


def _same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def _gpu_fit(W, iters, init, workspace=None):
    cb, codes = rvq.rvq_fit(torch.from_numpy(W).cuda(), iters, init, workspace=workspace)
    return cb.cpu().numpy(), codes.cpu().numpy()


def _residuals_fp32(W, cb, codes):
    """The stage inputs as the GPU forms them (fp32, one rounding per subtraction): R[0] = W, R[s+1] =
    R[s] - C_s[code_s].  numpy's float32 subtraction is the IEEE operation, so these are its bits."""
    R = [W.reshape(-1, 8).astype(np.float32)]
    c = codes.reshape(-1, 3).astype(np.int64)
    for s in range(2):
        R.append(R[-1] - cb[s][c[:, s]])
    return R


def _sq_error(W, cb, codes):
    X = W.reshape(-1, 8).astype(np.float64)
    c = codes.reshape(-1, 3).astype(np.int64)
    rec = sum(cb[s].astype(np.float64)[c[:, s]] for s in range(3))
    return float(np.sum((X - rec) ** 2) / np.sum(X ** 2))


def _first_assignment_means_match(R, start, got, chunk=32768):
    """One Lloyd step of one stage from `start` [256, 8]: the members of each centroid are decided in
    fp64 here (a later copy of an identical start never wins: ties go to the lower index in any
    precision).  Where no near-tie touches a centroid, its GPU value must be the correctly rounded mean
    of its members within one ulp (a centroid without members keeps its start).  Where k near-tie rows
    could have gone to or from it, the GPU's member set A' differs from this one, A, by at most those
    rows, so its mean moves by at most sum_U |x - m| / (|A| - k) (plus one ulp).  Returns (centroids
    checked exactly, centroids checked within that bound)."""
    X = R.astype(np.float64)
    nmax = (X * X).sum(1)
    _, first = np.unique(start, axis=0, return_index=True)
    later_copy = np.ones(256, bool)
    later_copy[first] = False
    assign = np.empty(len(X), np.int64)
    touch = [[] for _ in range(256)]
    for i in range(0, len(X), chunk):
        D = stage_distances(X[i:i + chunk], start)
        D[:, later_copy] = np.inf
        part = np.partition(D, 1, axis=1)
        assign[i:i + chunk] = D.argmin(axis=1)
        near = part[:, 1] - part[:, 0] <= 2 * TIE * (part[:, 0] + part[:, 1] + nmax[i:i + chunk])
        for r in np.flatnonzero(near):
            dmin = part[r, 0]
            lim = dmin + 2 * TIE * (3 * dmin + nmax[i + r])
            for c in np.flatnonzero(D[r] <= lim):
                touch[c].append(i + r)
    means = fsum_means(R, assign)
    count = np.bincount(assign, minlength=256)
    exact = bounded = 0
    for c in range(256):
        k = len(touch[c])
        want = start[c] if means[c] is None else means[c]
        if k == 0:
            assert ulps_apart(got[c], want).max() <= 1.0, c
            exact += 1
        elif count[c] > k:
            dev = np.abs(X[touch[c]] - want.astype(np.float64)).sum(axis=0) / (count[c] - k)
            slack = dev + np.spacing(np.abs(want)).astype(np.float64)
            assert np.all(np.abs(got[c].astype(np.float64) - want) <= slack), (c, k)
            bounded += 1
    return exact, bounded


# ---------------------------------------------------------------- exact arithmetic: oracle parity

def test_fit_recovers_a_separated_balanced_lattice_on_gpu():
    """The oracle's exact-recovery case, through the GPU: the pinned lattice values themselves."""
    W, digits, (S0, S1, S2) = _lattice_data(21)

    def first(**want):
        m = np.ones(len(digits), bool)
        for k, v in want.items():
            m &= digits[:, int(k[1])] == v
        return int(np.flatnonzero(m)[0])
    init = np.zeros((3, 256), np.int32)
    for c in range(256):
        init[0, c] = first(s0=c, s1=0, s2=1)
        init[1, c] = first(s1=c % 8, s2=0)
        init[2, c] = first(s2=c % 5)
    cb, codes = _gpu_fit(W, 2, init)
    assert np.array_equal(cb[0], S0.astype(np.float32))
    assert np.array_equal(cb[1], S1[np.arange(256) % 8].astype(np.float32))
    assert np.array_equal(cb[2], S2[np.arange(256) % 5].astype(np.float32))
    assert np.array_equal(codes.reshape(-1, 3), digits)


@pytest.mark.parametrize("iters", [1, 3])
def test_fit_matches_oracle_on_a_spread_lattice(iters):
    """Every lattice point twice, at +n and -n for a noise vector n on a 2^-10 grid: clusters of
    non-zero spread whose sums cancel exactly, so every distance decision is clear and every mean and
    residual exact in fp32 and fp64.  Codebooks and codes equal the oracle's bit for bit."""
    W0, digits, _ = _lattice_data(22)
    rng = np.random.default_rng(23)
    n = (rng.integers(-20, 21, W0.reshape(-1, 8).shape) * 2.0 ** -10).astype(np.float32)
    X = np.concatenate([W0.reshape(-1, 8) + n, W0.reshape(-1, 8) - n]).astype(np.float32)
    W = X.reshape(-1, 512)
    d2 = np.concatenate([digits, digits])
    init = np.zeros((3, 256), np.int32)
    for c in range(256):
        init[0, c] = int(np.flatnonzero((d2[:, 0] == c) & (d2[:, 1] == 0) & (d2[:, 2] == 1))[0])
        init[1, c] = int(np.flatnonzero((d2[:, 1] == c % 8) & (d2[:, 2] == 0))[0])
        init[2, c] = int(np.flatnonzero(d2[:, 2] == c % 5)[0])
    say(f"rvq_fit spread lattice iters={iters}")
    cb_o, codes_o = oracle.rvq_fit(W, iters, init)
    cb, codes = _gpu_fit(W, iters, init)
    assert np.array_equal(codes, codes_o)
    assert _same(cb, cb_o)


# ---------------------------------------------------------------- Gaussian weights: the definition, step by step

@pytest.mark.parametrize("rows,cols,seed", [
    (64, 512, 1),      # 4096 sub-vectors: two runs of the GPU's first summation level
    (100, 264, 2),     # ragged: 3300 sub-vectors, the last run partial
    (512, 1024, 4),    # 65,536 sub-vectors, 32 runs
])
def test_fit_codes_are_nearest_entries_of_its_codebooks(rows, cols, seed):
    say(f"rvq_fit {rows}x{cols}: codes vs own codebooks, error vs oracle")
    W, init = _input(rows, cols, seed)
    cb, codes = _gpu_fit(W, 4, init)
    ties = check_path(W, cb, codes)
    assert ties <= max(2, 1e-3 * codes.size)
    cb_o, codes_o = oracle.rvq_fit(W, 4, init)
    e, e_o = _sq_error(W, cb, codes), _sq_error(W, cb_o, codes_o)
    assert e <= 1.01 * e_o, (e, e_o)


@pytest.mark.parametrize("K", [1, 3])
def test_fit_stage0_update_is_the_mean_of_the_previous_assignment(K):
    say(f"rvq_fit 128x512 stage-0 Lloyd step K={K}")
    W, init = _input(128, 512, 9)
    cbp, codesp = _gpu_fit(W, K - 1, init)
    cb, _ = _gpu_fit(W, K, init)
    X = W.reshape(-1, 8)
    means = fsum_means(X, codesp.reshape(-1, 3)[:, 0])
    for c in range(256):
        want = cbp[0, c] if means[c] is None else means[c]
        assert ulps_apart(cb[0, c], want).max() <= 1.0, c


def test_fit_starts_and_first_step_of_every_stage():
    """No iteration: stage s's centroids are the named sub-vectors of the GPU's own stage input.  One
    iteration: each stage's centroids are the means of its first assignment from those starts."""
    say("rvq_fit 100x264 starts and first Lloyd step per stage")
    W, init = _input(100, 264, 10)
    cb0, codes0 = _gpu_fit(W, 0, init)
    R = _residuals_fp32(W, cb0, codes0)
    for s in range(3):
        assert np.array_equal(cb0[s], R[s][init[s]]), s
    assert check_path(W, cb0, codes0) <= 2
    cb1, codes1 = _gpu_fit(W, 1, init)
    R = _residuals_fp32(W, cb1, codes1)
    for s in range(3):
        exact, bounded = _first_assignment_means_match(R[s], R[s][init[s]], cb1[s])
        say(f"  stage {s}: {exact} centroids exact, {bounded} within the near-tie bound")
        assert exact + bounded >= 250 and exact >= 200
    assert check_path(W, cb1, codes1) <= 2


def test_fit_full_size():
    """One 2048 x 7168 matrix (1,835,008 sub-vectors, 896 runs), one Lloyd iteration per stage: codes
    are the GPU encoder's with the fitted codebooks and the nearest entries along their own path; each
    stage's centroids are the means of its first assignment; the error falls stage by stage and is
    within 1 % of the oracle's fit."""
    say("rvq_fit 2048x7168 iters=1 (checks ~30 s)")
    W, init = _input(2048, 7168, 6)
    Wd = torch.from_numpy(W).cuda()
    cbt, codest = rvq.rvq_fit(Wd, 1, init)
    assert torch.equal(codest, rvq.rvq_encode(Wd, cbt))
    cb, codes = cbt.cpu().numpy(), codest.cpu().numpy()
    rng = np.random.default_rng(1)
    sample = rng.choice(codes.size // 3, 20000, replace=False)
    check_path(W, cb, codes, groups=sample)
    R = _residuals_fp32(W, cb, codes)
    exact, bounded = _first_assignment_means_match(R[0], R[0][init[0]], cb[0])
    say(f"  stage 0: {exact} centroids exact, {bounded} within the near-tie bound")
    assert exact + bounded == 256
    X = W.reshape(-1, 8).astype(np.float64)
    c = codes.reshape(-1, 3).astype(np.int64)
    err = [float(np.sum((X - sum(cb[s][c[:, s]] for s in range(k + 1))) ** 2)) for k in range(3)]
    assert err[0] > err[1] > err[2]
    cb_o, codes_o = oracle.rvq_fit(W, 1, init)
    assert _sq_error(W, cb, codes) <= 1.01 * _sq_error(W, cb_o, codes_o)


def test_fit_is_deterministic_and_reuses_its_workspace():
    """The same call twice gives the same bits; two calls on one workspace (the second on a smaller
    matrix) give what fresh calls give."""
    ws = torch.empty(rvq.lib().rvq_fit_workspace_bytes(256, 512), dtype=torch.uint8, device="cuda")
    for rows, cols, seed in ((256, 512, 7), (33, 136, 8)):
        say(f"rvq_fit {rows}x{cols} determinism")
        W, init = _input(rows, cols, seed)
        a_cb, a_codes = _gpu_fit(W, 3, init, workspace=ws)
        b_cb, b_codes = _gpu_fit(W, 3, init)
        assert _same(a_cb, b_cb) and np.array_equal(a_codes, b_codes)
        assert check_path(W, a_cb, a_codes) <= 2
