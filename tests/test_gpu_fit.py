"""Codebook fitting on the GPU (rvq_fit, residual k-means) against the oracle's, bit for bit: the
same fp32 decisions and the same fixed-order fp64 means give identical codebooks and codes."""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
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


@pytest.mark.parametrize("rows,cols,iters,seed", [
    (64, 512, 6, 1),      # 4096 sub-vectors: two runs of the mean's first level
    (100, 264, 3, 2),     # ragged: 3300 sub-vectors, the last run partial
    (1, 8, 2, 3),         # one sub-vector: every centroid starts at it
    (512, 1024, 2, 4),    # 65,536 sub-vectors, 32 runs
    (37, 2056, 0, 5),     # no iteration: starts, then one assignment per stage
])
def test_fit_matches_oracle(rows, cols, iters, seed):
    say(f"rvq_fit {rows}x{cols} iters={iters}")
    W, init = _input(rows, cols, seed)
    cb_o, codes_o = oracle.rvq_fit(W, iters, init)
    cb, codes = rvq.rvq_fit(torch.from_numpy(W).cuda(), iters, init)
    assert _same(cb.cpu().numpy(), cb_o)
    assert np.array_equal(codes.cpu().numpy(), codes_o)


def test_fit_recovers_a_separated_balanced_lattice_on_gpu():
    """The oracle's exact-recovery case, through the GPU."""
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
    cb, codes = rvq.rvq_fit(torch.from_numpy(W).cuda(), 2, init)
    cb = cb.cpu().numpy()
    assert np.array_equal(cb[0], S0.astype(np.float32))
    assert np.array_equal(cb[1], S1[np.arange(256) % 8].astype(np.float32))
    assert np.array_equal(cb[2], S2[np.arange(256) % 5].astype(np.float32))
    assert np.array_equal(codes.cpu().numpy().reshape(-1, 3), digits)


def test_fit_full_size_matches_oracle():
    """One 2048 x 7168 matrix (1,835,008 sub-vectors, 896 runs), one Lloyd iteration per stage, against
    the oracle bit for bit; the codes equal the GPU encoder's with the fitted codebooks, and the
    squared error falls stage by stage."""
    say("rvq_fit 2048x7168 iters=1 (oracle ~10 s)")
    W, init = _input(2048, 7168, 6)
    Wd = torch.from_numpy(W).cuda()
    cb, codes = rvq.rvq_fit(Wd, 1, init)
    assert torch.equal(codes, rvq.rvq_encode(Wd, cb))
    cb_o, codes_o = oracle.rvq_fit(W, 1, init)
    assert _same(cb.cpu().numpy(), cb_o)
    assert np.array_equal(codes.cpu().numpy(), codes_o)
    X = W.reshape(-1, 8).astype(np.float64)
    c = codes_o.reshape(-1, 3)
    err = [float(np.sum((X - sum(cb_o[s][c[:, s]] for s in range(k + 1))) ** 2)) for k in range(3)]
    assert err[0] > err[1] > err[2]


def test_fit_workspace_reuse_and_repeat():
    """Two calls on the same workspace (the second on a smaller matrix) give the oracle's results."""
    ws = torch.empty(rvq.lib().rvq_fit_workspace_bytes(256, 512), dtype=torch.uint8, device="cuda")
    for rows, cols, seed in ((256, 512, 7), (33, 136, 8)):
        W, init = _input(rows, cols, seed)
        cb, codes = rvq.rvq_fit(torch.from_numpy(W).cuda(), 3, init, workspace=ws)
        cb_o, codes_o = oracle.rvq_fit(W, 3, init)
        assert _same(cb.cpu().numpy(), cb_o) and np.array_equal(codes.cpu().numpy(), codes_o)
