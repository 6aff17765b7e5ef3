"""The near-tie rule of tests/quant_checks.py on the CPU: an emulation of an encoder that takes its
decisions in fp32 (numpy float32 operations, each rounded as IEEE prescribes, no fused operations:
difference, square, sum over the 8 dims in order, residual rounded at each subtraction) differs from
the oracle's fp64 decisions only at decisions the rule calls near-ties, and a pick that is not the
nearest at a clear decision is refused."""
import numpy as np
import pytest

import oracle
import synth
from quant_checks import TIE, check_path, compare_with_oracle_codes


def encode_fp32(W, cb):
    V = np.asarray(W, dtype=np.float32).reshape(-1, 8).copy()
    codes = np.empty((len(V), 3), np.uint8)
    for s in range(3):
        C = cb[s].astype(np.float32)
        d = np.zeros((len(V), 256), np.float32)
        for j in range(8):
            t = V[:, j:j + 1] - C[None, :, j]
            d = d + t * t
        best = d.argmin(axis=1)
        codes[:, s] = best
        V = V - C[best]
    return codes.reshape(W.shape[0], W.shape[1] // 8, 3)


def test_fp32_decisions_differ_from_fp64_only_at_near_ties():
    cb = synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)
    rng = np.random.default_rng(3)
    # values near the tie bound are common when two entries are (almost) mirror images around a
    # sub-vector: build a third of the groups as midpoints of two entries, plus tiny noise
    W = rng.standard_normal((384, 256)).astype(np.float32).reshape(-1, 8)
    a, b = rng.integers(0, 256, (2, len(W) // 3))
    W[:len(W) // 3] = 0.5 * (cb[0][a] + cb[0][b]) + 1e-7 * rng.standard_normal((len(W) // 3, 8))
    W = W.reshape(384, 256).astype(np.float32)
    got = encode_fp32(W, cb)
    want, margins = oracle.rvq_encode(W, cb, margins=True)
    flipped = compare_with_oracle_codes(W, cb, got, want, margins)
    assert 0 < flipped < 0.02 * got.size / 3      # the midpoints do produce some flips
    # the flips sit well inside the rule (its bound carries a 16x margin over the fp32 error)
    G, O, M = got.reshape(-1, 3), want.reshape(-1, 3), margins.reshape(-1, 3, 3)
    rows = np.flatnonzero(np.any(G != O, axis=1))
    s0 = np.argmax(G[rows] != O[rows], axis=1)
    rel = (M[rows, s0, 1] - M[rows, s0, 0]) / (M[rows, s0, 0] + M[rows, s0, 1] + M[rows, :, 2].max(axis=1))
    assert rel.max() <= TIE / 4


def test_a_wrong_pick_is_refused():
    cb = synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)
    W = np.random.default_rng(4).standard_normal((16, 64)).astype(np.float32)
    want, margins = oracle.rvq_encode(W, cb, margins=True)
    assert check_path(W, cb, want) == 0
    bad = want.copy()
    bad[3, 2, 1] = np.uint8((int(bad[3, 2, 1]) + 7) % 256)
    with pytest.raises(AssertionError):
        compare_with_oracle_codes(W, cb, bad, want, margins)
