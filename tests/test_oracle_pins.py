"""Pins for the fp64 oracle: each test ties an oracle function to something
other than itself (page-printed constants, closed forms, an independent
encoding, a library routine, brute force, or an invariant), chosen so that a
plausible slip (dropped stage, swapped stage order, transposed group layout,
wrong sign, wrong tie order) fails at least one of them.

Pinned functions and what pins them:
  dequant / gemv   : page constants (3 B per 8 weights), binary-digit encoding
                     (exact integers), stage-0-only dense reduction to numpy
                     matmul, linearity, power-of-two scaling, relabelling
  lut / via_lut    : closed form on digit codebooks (T_s[c] = 16c, 4c, c),
                     brute force over all 256^3 triples, exact equality with
                     gemv on small integers
  expert           : torch fp64 dense SwiGLU on independently built weights,
                     zero input, k=1 mixing
  router / topk    : numpy matmul on widened bf16, lexsort order, scipy softmax
                     (k = E), gate = 1 at k = 1, exact ties -> lower id
  moe_layer /      : k = 1 is the one expert, identical experts give that expert (gates sum to 1),
  moe_mix            the residual added once, and each expert weighed by its own gate (experts
                     with disjoint output coordinates against scipy's softmax of the kept logits)
  rmsnorm          : torch rms_norm, closed-form RMS of the output
  gemv_batch /     : T tokens at once equal T one-token calls bit for bit (each token's
  expert_batch       sums are independent of the others)
  moe_chunk        : token by token equal to moe_layer (routing, gates, residual), with
                     several tokens on one expert, a token subset, and k = 1
  rvq_encode       : the binary-digit encoding built by bit extraction (greedy residual
                     search must recover it exactly), exact codebook entries with a zero
                     entry in the later stages, re-encoding of a decode, numpy brute force
                     of every decision along the path, exact ties -> lower index, and the
                     reported margins (best, second-best distance, input norm)
  rvq_fit          : exact recovery of a separated balanced lattice, Lloyd's update against
                     math.fsum means of the previous assignment, starts taken from the
                     residual, codes = rvq_encode with the fitted codebooks, monotone
                     stage-0 distortion
  crc32            : the standard check value of CRC-32 ("123456789" -> 0xCBF43926),
                     zlib.crc32 on random buffers of ragged lengths, single-bit flips
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _digit_codebooks():
    """Stage s codebook entry c = weight_s * (bit j of c) for j = 0..7, weights (16, 4, 1)."""
    bits = ((np.arange(256)[:, None] >> np.arange(8)[None, :]) & 1).astype(np.float32)
    return np.stack([16.0 * bits, 4.0 * bits, 1.0 * bits]).astype(np.float32)


def _digit_encode(W):
    """Encode W (entries 16a+4b+c, a,b,c in {0,1}) into codes [rows, cols/8, 3]: stage s's
    code for a group is the 8-bit pattern of that digit across the group's 8 columns."""
    rows, cols = W.shape
    Wi = W.astype(np.int64)
    digits = [(Wi >> 4) & 1, (Wi >> 2) & 1, Wi & 1]
    assert np.array_equal(16 * digits[0] + 4 * digits[1] + digits[2], Wi)
    codes = np.zeros((rows, cols // 8, 3), dtype=np.uint8)
    for s in range(3):
        d = digits[s].reshape(rows, cols // 8, 8)
        codes[:, :, s] = (d << np.arange(8)[None, None, :]).sum(axis=2).astype(np.uint8)
    return codes


def _digit_matrix(rng, rows, cols):
    vals = np.array([16 * a + 4 * b + c for a in (0, 1) for b in (0, 1) for c in (0, 1)])
    return vals[rng.integers(0, 8, size=(rows, cols))].astype(np.float64)


# ---------------------------------------------------------------- format (page constants)

def test_page_constants_and_code_bytes():
    g = json.load(open(GOLDEN))
    stages, entries, dim = g["stages"]["value"], g["codebook_entries"]["value"], g["subvector_dim"]["value"]
    assert (stages, entries, dim) == (3, 256, 8)
    # one code byte per stage per 8-weight group, each byte indexing a 256-entry codebook
    assert 2 ** 8 == entries
    bpw = stages * 8 / dim
    assert bpw == g["bits_per_weight"]["value"]
    for rows, cols in [(256, 512), (2048, 7168), (7168, 2048)]:
        codes = synth.matrix_codes(1, 0, 0, synth.SINGLE, rows, cols)
        assert codes.dtype == np.uint8 and codes.shape == (rows, cols // dim, stages)
        assert codes.nbytes * 8 / (rows * cols) == bpw
    ex = synth.Expert(synth.SEED_EXPERT, 0, 0, 7168, 2048)
    assert ex.record_bytes().nbytes == 16_515_072
    assert 256 * 16_515_072 == 4_227_858_432
    assert 92 * 64 * 16_515_072 == 97_240_743_936
    assert g["table_reads_per_row_group"]["value"] == stages
    assert g["additions_per_row_group"]["value"] == stages - 1


# ---------------------------------------------------------------- decode + matvec

def test_digit_encoding_decodes_exactly():
    rng = np.random.default_rng(1)
    rows, cols = 37, 64
    W = _digit_matrix(rng, rows, cols)
    codes = _digit_encode(W)
    cb = _digit_codebooks()
    assert np.array_equal(oracle.dequant(codes, cb, rows, cols), W)
    x = rng.integers(-3, 4, size=cols).astype(np.float64)
    assert np.array_equal(oracle.gemv(codes, cb, rows, cols, x), W @ x)
    xr = rng.standard_normal(cols)
    np.testing.assert_allclose(oracle.gemv(codes, cb, rows, cols, xr), W @ xr, rtol=1e-13, atol=1e-12)


def test_stage0_only_reduces_to_dense_matmul():
    rng = np.random.default_rng(2)
    rows, cols = 20, 48
    # dense W whose 8-vectors come from a pool of 256 distinct vectors
    pool = rng.standard_normal((256, 8)).astype(np.float32)
    pick = rng.integers(0, 256, size=(rows, cols // 8))
    W = pool[pick].reshape(rows, cols).astype(np.float64)
    cb = np.zeros((3, 256, 8), dtype=np.float32)
    cb[0] = pool
    codes = np.zeros((rows, cols // 8, 3), dtype=np.uint8)
    codes[:, :, 0] = pick
    codes[:, :, 1:] = rng.integers(0, 256, size=(rows, cols // 8, 2))  # indexes zero vectors
    x = rng.standard_normal(cols)
    np.testing.assert_allclose(oracle.gemv(codes, cb, rows, cols, x), W @ x, rtol=1e-13, atol=1e-13)


def test_linearity_and_power_of_two_scaling():
    codes = synth.matrix_codes(5, 0, 0, synth.SINGLE, 64, 256)
    cb = synth.matrix_codebooks(5, 0, 0, synth.SINGLE)
    x1 = synth.activation_f32(5, 1, 256).astype(np.float64)
    x2 = synth.activation_f32(5, 2, 256).astype(np.float64)
    y = oracle.gemv(codes, cb, 64, 256, 0.75 * x1 - 2.5 * x2)
    y1, y2 = oracle.gemv(codes, cb, 64, 256, x1), oracle.gemv(codes, cb, 64, 256, x2)
    np.testing.assert_allclose(y, 0.75 * y1 - 2.5 * y2, rtol=1e-12, atol=1e-12)
    ys = oracle.gemv(codes, (cb * np.float32(8.0)).astype(np.float32), 64, 256, x1)
    assert np.array_equal(ys, 8.0 * y1)


def test_codebook_relabelling_invariance():
    rng = np.random.default_rng(3)
    codes = synth.matrix_codes(6, 0, 0, synth.SINGLE, 32, 128)
    cb = synth.matrix_codebooks(6, 0, 0, synth.SINGLE)
    x = synth.activation_f32(6, 0, 128)
    cb2 = np.empty_like(cb)
    codes2 = np.empty_like(codes)
    for s in range(3):
        perm = rng.permutation(256)          # new entry i holds old entry perm[i]
        inv = np.argsort(perm)               # old code c -> new code inv[c]
        cb2[s] = cb[s][perm]
        codes2[:, :, s] = inv[codes[:, :, s]]
    assert np.array_equal(oracle.gemv(codes2, cb2, 32, 128, x), oracle.gemv(codes, cb, 32, 128, x))


def test_row_selection_matches_full():
    codes = synth.matrix_codes(7, 0, 0, synth.SINGLE, 100, 80)
    cb = synth.matrix_codebooks(7, 0, 0, synth.SINGLE)
    x = synth.activation_f32(7, 0, 80)
    full = oracle.gemv(codes, cb, 100, 80, x)
    sel = np.array([99, 0, 17, 17, 50])
    assert np.array_equal(oracle.gemv(codes, cb, 100, 80, x, rowsel=sel), full[sel])


# ---------------------------------------------------------------- partial-dot tables

def test_lut_closed_form_on_digit_codebooks():
    cb = _digit_codebooks()
    x = np.tile(2.0 ** np.arange(8), 3)          # every group sees (1, 2, 4, ..., 128)
    T = oracle.lut(cb, x)
    c = np.arange(256, dtype=np.float64)
    for g in range(3):
        assert np.array_equal(T[g, 0], 16 * c)
        assert np.array_equal(T[g, 1], 4 * c)
        assert np.array_equal(T[g, 2], c)


def test_lut_brute_force_all_code_triples():
    cb = synth.matrix_codebooks(8, 0, 0, synth.SINGLE).astype(np.float64)
    xg = synth.activation_f32(8, 0, 8).astype(np.float64)
    T = oracle.lut(cb.astype(np.float32), xg)[0]            # [3, 256]
    table_sum = T[0][:, None, None] + T[1][None, :, None] + T[2][None, None, :]
    # decoded sub-vector for every (c0, c1, c2), then its dot with x_g
    d0, d1, d2 = cb[0] @ xg, cb[1] @ xg, cb[2] @ xg
    assert np.abs(T[0] - d0).max() < 1e-14 * 8
    dense = np.einsum("abcj,j->abc", cb[0][:, None, None, :] + cb[1][None, :, None, :]
                      + cb[2][None, None, :, :], xg, optimize=True)
    assert np.abs(table_sum - dense).max() <= 1e-13 * np.abs(dense).max()
    del d1, d2


def test_lut_form_equals_decode_exactly_on_small_integers():
    rng = np.random.default_rng(4)
    rows, cols = 50, 96
    cb = rng.integers(-4, 5, size=(3, 256, 8)).astype(np.float32)
    codes = rng.integers(0, 256, size=(rows, cols // 8, 3)).astype(np.uint8)
    x = rng.integers(-3, 4, size=cols).astype(np.float64)
    y_dec = oracle.gemv(codes, cb, rows, cols, x)
    y_lut = oracle.gemv_via_lut(codes, oracle.lut(cb, x), rows, cols)
    assert np.array_equal(y_dec, y_lut)
    W = oracle.dequant(codes, cb, rows, cols)
    assert np.array_equal(W @ x, y_dec)


def test_lut_form_equals_decode_on_random_data():
    codes = synth.matrix_codes(synth.SEED_MATVEC, 0, 0, synth.SINGLE, 256, 512)
    cb = synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)
    x = synth.activation_f32(synth.SEED_MATVEC, 0, 512)
    y_dec = oracle.gemv(codes, cb, 256, 512, x)
    y_lut = oracle.gemv_via_lut(codes, oracle.lut(cb, x), 256, 512)
    assert np.linalg.norm(y_dec - y_lut) <= 1e-12 * np.linalg.norm(y_dec)


# ---------------------------------------------------------------- SwiGLU expert

def _digit_expert(rng, H, I):
    Wg, Wu, Wd = _digit_matrix(rng, I, H), _digit_matrix(rng, I, H), _digit_matrix(rng, H, I)
    # centre the weights so activations stay moderate: subtract via codebooks is not possible,
    # so scale x instead (the expert is linear in each matrix)
    cb = _digit_codebooks()
    ex = {"hidden": H, "inter": I, "gate": (_digit_encode(Wg), cb), "up": (_digit_encode(Wu), cb),
          "down": (_digit_encode(Wd), cb)}
    return ex, Wg, Wu, Wd


def test_expert_matches_dense_torch_swiglu():
    rng = np.random.default_rng(5)
    H, I = 64, 40
    ex, Wg, Wu, Wd = _digit_expert(rng, H, I)
    x = rng.standard_normal(H) * 0.01
    y = oracle.expert(ex, x)
    xt = torch.tensor(x, dtype=torch.float64)
    ref = torch.tensor(Wd) @ (torch.nn.functional.silu(torch.tensor(Wg) @ xt) * (torch.tensor(Wu) @ xt))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.expert(ex, np.zeros(H)), np.zeros(H))
    sel = np.array([3, 63, 0])
    np.testing.assert_allclose(oracle.expert(ex, x, rowsel=sel), y[sel], rtol=0, atol=0)


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    for z in (-30.0, -2.5, -1e-3, 0.5, 3.0, 40.0):
        assert abs(oracle.silu(z) - z * scipy.special.expit(z)) <= 1e-15 * max(1.0, abs(z))
    assert abs(oracle.silu(60.0) / 60.0 - 1.0) < 1e-20 + 1e-15
    assert abs(oracle.silu(-60.0)) < 1e-20
    # odd-even identity of z*sigmoid(z): silu(z) - silu(-z) = z
    for z in (0.3, 1.7, 9.0):
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) < 1e-14 * max(1.0, z)


# ---------------------------------------------------------------- router

def test_router_logits_match_numpy_on_widened_bf16():
    bits = synth.router_bf16_bits(synth.SEED_LAYER, 0, 64, 512)
    X = np.stack([synth.activation_f32(synth.SEED_LAYER, t, 512) for t in range(3)]).astype(np.float64)
    L = oracle.router_logits(bits, X)
    Wf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(L, X @ Wf.T, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("E,k", [(256, 16), (64, 16), (16, 16), (10, 1), (300, 7)])
def test_topk_invariants(E, k):
    rng = np.random.default_rng(E * 31 + k)
    logits = rng.standard_normal(E) * 1.7
    ids, gates, gaps = oracle.topk(logits, k)
    assert len(set(ids.tolist())) == k and ids.min() >= 0 and ids.max() < E
    order = np.lexsort((np.arange(E), -logits))
    assert np.array_equal(ids, order[:k])
    if k < E:
        assert logits[ids].min() >= np.delete(logits, ids).max()
        assert gaps[0] == logits[order[k - 1]] - logits[order[k]]
    assert (gates > 0).all() and abs(gates.sum() - 1.0) < 1e-12
    assert (np.diff(gates) <= 0).all()
    np.testing.assert_allclose(gates, scipy.special.softmax(logits[ids]), rtol=1e-13)
    if k == E:
        np.testing.assert_allclose(gates, scipy.special.softmax(logits)[ids], rtol=1e-13)
    if k == 1:
        assert gates[0] == 1.0


def test_topk_exact_ties_prefer_lower_id():
    logits = np.array([0.5, 2.0, 1.0, 2.0, 1.0, 1.0, -3.0, 2.0])
    ids, gates, gaps = oracle.topk(logits, 5)
    assert ids.tolist() == [1, 3, 7, 2, 4]
    assert gates[0] == gates[1] == gates[2] and gates[3] == gates[4]
    assert gaps == (0.0, 0.0)


def test_topk_softmax_renormalisation_equals_softmax_then_renormalise():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal(256) * 1.7
    ids, gates, _ = oracle.topk(logits, 16)
    p = scipy.special.softmax(logits)
    np.testing.assert_allclose(gates, p[ids] / p[ids].sum(), rtol=1e-13)


# ---------------------------------------------------------------- MoE composition

def _small_expert(seed, e, H, I):
    ex = synth.Expert(seed, 0, e, H, I)
    return {"hidden": H, "inter": I, "gate": (ex.codes(synth.GATE), ex.codebooks(synth.GATE)),
            "up": (ex.codes(synth.UP), ex.codebooks(synth.UP)),
            "down": (ex.codes(synth.DOWN), ex.codebooks(synth.DOWN))}


def test_moe_layer_k1_and_duplicate_experts():
    H, I, E = 64, 32, 8
    experts = {e: _small_expert(11, e, H, I) for e in range(E)}
    bits = synth.router_bf16_bits(11, 0, E, H)
    x = synth.activation_f32(11, 0, H).astype(np.float64)
    y1, ids1, g1, _ = oracle.moe_layer(lambda e: experts[e], bits, x, 1)
    assert g1[0] == 1.0
    assert np.array_equal(y1, oracle.expert(experts[int(ids1[0])], x))
    # every id maps to the same expert: output = (sum of gates) * expert = expert (gates sum to 1)
    y4, ids4, g4, _ = oracle.moe_layer(lambda e: experts[0], bits, x, 4)
    np.testing.assert_allclose(y4, oracle.expert(experts[0], x), rtol=1e-13, atol=1e-12)
    # residual is added once
    r = np.arange(H, dtype=np.float64)
    yr, _, _, _ = oracle.moe_layer(lambda e: experts[e], bits, x, 3, residual=r)
    y3, _, _, _ = oracle.moe_layer(lambda e: experts[e], bits, x, 3)
    np.testing.assert_allclose(yr - r, y3, rtol=1e-13, atol=1e-12)


def test_moe_layer_weighs_each_expert_by_its_own_gate():
    """Experts whose outputs live on disjoint coordinates: expert e's down matrix has one nonzero
    row, row e (every other row's codes select all-zero entries), so coordinate e of the layer's
    output is gate(e) * expert_e(x)[e] for a selected e and 0 otherwise.  The gates come from scipy's
    softmax over the kept logits and the selection from numpy's lexsort of the logits, so a gate
    applied to another rank's expert, a dropped or repeated expert, or a wrong normalisation fails."""
    H, I, E, k = 64, 32, 12, 5
    bits = synth.router_bf16_bits(13, 0, E, H)
    x = synth.activation_f32(13, 0, H).astype(np.float64)
    experts = {}
    for e in range(E):
        ex = _small_expert(13, e, H, I)
        dc, dcb = ex["down"]
        dc = np.array(dc, dtype=np.uint8).reshape(H, I // 8, 3)
        dcb = np.array(dcb, dtype=np.float32).reshape(3, 256, 8)
        dcb[:, 0, :] = 0.0                                  # entry 0 of every stage is the zero vector
        keep = dc[e].copy()
        dc[:] = 0
        dc[e] = np.where(keep == 0, 1, keep)                # row e: nonzero entries only
        ex["down"] = (dc, dcb)
        experts[e] = ex
    y, ids, gates, _ = oracle.moe_layer(lambda e: experts[e], bits, x, k)
    L = oracle.router_logits(bits, x[None, :])[0]
    order = np.lexsort((np.arange(E), -L))[:k]
    assert np.array_equal(np.sort(ids), np.sort(order))
    g = scipy.special.softmax(L[order])
    for e in range(E):
        own = oracle.expert(experts[e], x)
        assert np.count_nonzero(own) == 1 and own[e] != 0.0
        if e in order:
            want = g[list(order).index(e)] * own[e]
            assert abs(y[e] - want) <= 1e-13 * abs(want), (e, y[e], want)
        else:
            assert y[e] == 0.0


def test_gemv_and_expert_batch_equal_single_token_calls():
    """Several tokens at once give each token exactly what a one-token call gives (the oracle's
    per-token sums do not depend on the other tokens); row selection keeps that."""
    H, I = 96, 40
    ex = _small_expert(13, 3, H, I)
    X = np.stack([synth.activation_f32(13, t, H).astype(np.float64) for t in range(5)])
    X[2] *= -3.0
    codes, cb = ex["gate"]
    Yg = oracle.gemv_batch(codes, cb, I, H, X)
    Ye = oracle.expert_batch(ex, X)
    sel = np.array([0, 17, 95, 3])
    Yes = oracle.expert_batch(ex, X, rowsel=sel)
    for t in range(X.shape[0]):
        assert np.array_equal(Yg[t], oracle.gemv(codes, cb, I, H, X[t]))
        assert np.array_equal(Ye[t], oracle.expert(ex, X[t]))
        assert np.array_equal(Yes[t], Ye[t][sel])
    # and the batch form is the dense product on the dequantised weights
    np.testing.assert_allclose(Yg, X @ oracle.dequant(codes, cb, I, H).T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("E,k", [(6, 3), (8, 1), (5, 5)])
def test_moe_chunk_equals_moe_layer_token_by_token(E, k):
    """The chunk form (experts rebuilt once, applied to all their tokens, pairs scattered back with
    their gates) gives each token moe_layer's output: same ids and gates, same sum up to the order of
    the fp64 additions; with few experts every expert serves several tokens, and a token subset
    returns those rows only."""
    H, I, T = 64, 32, 7
    experts = {e: _small_expert(17, e, H, I) for e in range(E)}
    get = lambda e: experts[e]
    bits = synth.router_bf16_bits(17, 0, E, H)
    X = np.stack([synth.activation_f32(17, 100 + t, H).astype(np.float64) for t in range(T)])
    R = np.stack([synth.activation_f32(17, 200 + t, H).astype(np.float64) for t in range(T)])
    for residual in (None, R):
        Y, ids, gates = oracle.moe_chunk(get, bits, X, k, residual=residual)
        for t in range(T):
            y1, ids1, g1, _ = oracle.moe_layer(get, bits, X[t], k, residual=None if residual is None else R[t])
            assert np.array_equal(ids[t], ids1) and np.array_equal(gates[t], g1)
            np.testing.assert_allclose(Y[t], y1, rtol=1e-13, atol=1e-12 * np.abs(y1).max())
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert counts.max() >= 2          # some expert serves several tokens
    sub = np.array([5, 0, 3])
    Ys, _, _ = oracle.moe_chunk(get, bits, X, k, residual=R, tokens=sub)
    Yall, _, _ = oracle.moe_chunk(get, bits, X, k, residual=R)
    np.testing.assert_allclose(Ys, Yall[sub], rtol=1e-13, atol=1e-12 * np.abs(Yall).max())


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_matches_torch_and_closed_form():
    h = synth.activation_f32(12, 0, 7168).astype(np.float64) * 3.0
    eps = 1e-6
    out = oracle.rmsnorm(h, eps)
    ref = torch.nn.functional.rms_norm(torch.tensor(h), (h.size,), eps=eps).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)
    ms = np.mean(h * h)
    assert abs(np.sqrt(np.mean(out * out)) - np.sqrt(ms / (ms + eps))) < 1e-14
    np.testing.assert_allclose(oracle.rmsnorm(7.0 * h, 0.0), oracle.rmsnorm(h, 0.0), rtol=1e-14)


# ---------------------------------------------------------------- CRC-32

def test_crc32_check_value_and_zlib():
    import zlib
    assert oracle.crc32(b"123456789") == 0xCBF43926   # the catalogued check value of CRC-32
    assert oracle.crc32(b"") == 0
    rng = np.random.default_rng(7)
    for n in (1, 3, 1023, 1024, 65537, 300001):
        buf = rng.integers(0, 256, n, dtype=np.uint8)
        assert oracle.crc32(buf) == zlib.crc32(buf.tobytes()), n
    # a single flipped bit anywhere changes the value
    buf = rng.integers(0, 256, 4096, dtype=np.uint8)
    c = oracle.crc32(buf)
    for pos in (0, 1000, 4095):
        b2 = buf.copy()
        b2[pos] ^= 0x10
        assert oracle.crc32(b2) != c


# ---------------------------------------------------------------- RVQ encoder

def test_rvq_encode_recovers_digit_codes():
    """With digit codebooks (16, 4, 1) x bits, w = 16a + 4b + c: the nearest stage-0 entry takes
    bit a in every column (16 + [0, 5] is nearer 16 than 0; [0, 5] nearer 0), and so on down the
    stages, so the greedy residual search must return exactly the bit-extraction codes."""
    rng = np.random.default_rng(11)
    rows, cols = 37, 96
    W = (16 * rng.integers(0, 2, (rows, cols)) + 4 * rng.integers(0, 2, (rows, cols))
         + rng.integers(0, 2, (rows, cols))).astype(np.float32)
    codes = oracle.rvq_encode(W, _digit_codebooks())
    assert np.array_equal(codes, _digit_encode(W))
    np.testing.assert_array_equal(oracle.dequant(codes, _digit_codebooks(), rows, cols), W)


def test_rvq_encode_exact_entries_and_reencode():
    rng = np.random.default_rng(12)
    cb = rng.standard_normal((3, 256, 8)).astype(np.float32) * np.float32(0.5) ** np.arange(3)[:, None, None]
    cb[1, 77] = 0.0
    cb[2, 201] = 0.0
    # a sub-vector equal to a stage-0 entry: that entry, then the zero entries of stages 1 and 2
    picks = rng.integers(0, 256, 12)
    W = cb[0, picks].reshape(3, 32)
    codes = oracle.rvq_encode(W, cb)
    assert np.array_equal(codes[:, :, 0].reshape(-1), picks)
    assert np.all(codes[:, :, 1] == 77) and np.all(codes[:, :, 2] == 201)
    # encoding a decode returns the same codes when every stage's pick is the unique nearest
    # (stages far apart in scale: 1, 1e-2, 1e-4)
    cb2 = rng.standard_normal((3, 256, 8)).astype(np.float32) * np.array([1.0, 1e-2, 1e-4], np.float32)[:, None, None]
    c0 = rng.integers(0, 256, (20, 6, 3)).astype(np.uint8)
    W2 = oracle.dequant(c0, cb2, 20, 48).astype(np.float32)
    assert np.array_equal(oracle.rvq_encode(W2, cb2), c0)


def test_rvq_encode_brute_force_and_margins():
    """Every decision against a numpy brute force along the oracle's own path (all 256 distances of
    the fp64 residual, the first index of the minimum), and the reported margins: the best and
    second-best distance and the input's squared norm at each stage."""
    rng = np.random.default_rng(14)
    cb = (rng.standard_normal((3, 256, 8)) * np.array([1.0, 0.5, 0.25])[:, None, None]).astype(np.float32)
    W = rng.standard_normal((9, 64)).astype(np.float32)
    codes, m = oracle.rvq_encode(W, cb, margins=True)
    V = W.reshape(-1, 8).astype(np.float64)
    C = codes.reshape(-1, 3)
    M = m.reshape(-1, 3, 3)
    for s in range(3):
        D = ((V[:, None, :] - cb[s].astype(np.float64)[None]) ** 2).sum(axis=2)
        best = np.argmin(D, axis=1)
        assert np.array_equal(C[:, s], best), s
        Ds = np.sort(D, axis=1)
        np.testing.assert_allclose(M[:, s, 0], Ds[:, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(M[:, s, 1], Ds[:, 1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(M[:, s, 2], (V ** 2).sum(axis=1), rtol=1e-12)
        V = V - cb[s][best].astype(np.float64)
    assert np.array_equal(oracle.rvq_encode(W, cb), codes)


def test_rvq_encode_exact_tie_takes_lower_index():
    """Two entries at exactly the same distance (mirror images about the sub-vector): the lower
    index wins, at every stage, and the reported gap is exactly zero."""
    cb = np.full((3, 256, 8), 100.0, dtype=np.float32)
    for s in range(3):
        cb[s, 200] = 1.0
        cb[s, 31] = -1.0            # |0 - 1| == |0 - (-1)|: a tie between entries 31 and 200
    W = np.zeros((1, 8), dtype=np.float32)
    codes, m = oracle.rvq_encode(W, cb, margins=True)
    # stage 0 picks 31 (lower index); the residual is then +1, nearest entry 200 (distance 0)
    assert codes[0, 0, 0] == 31 and m[0, 0, 0, 0] == m[0, 0, 0, 1] == 8.0
    assert codes[0, 0, 1] == 200 and m[0, 0, 1, 0] == 0.0


# ---------------------------------------------------------------- RVQ codebook fit (residual k-means)

def _lattice_data(seed):
    """Sub-vectors S0[c0] + S1[c1] + S2[c2] over the full product of 256 x 8 x 5 entries, shuffled.
    S0: 1024 x distinct integer vectors (clusters far apart); S1 = {+-v1..+-v4} (components +-8, +-16),
    S2 = {0, +-u1, +-u2} (components +-0.5, +-1): both of mean zero, so each stage's clusters have
    their stage entry as exact mean, and every value and sum is exact in fp32 and fp64."""
    rng = np.random.default_rng(seed)
    S0 = set()
    while len(S0) < 256:
        S0.add(tuple(rng.integers(-3, 4, 8)))
    S0 = 1024.0 * np.array(sorted(S0), dtype=np.float64)
    v = rng.choice([-16.0, -8.0, 8.0, 16.0], size=(4, 8))
    S1 = np.concatenate([v, -v])
    u = rng.choice([-1.0, -0.5, 0.5, 1.0], size=(2, 8))
    S2 = np.concatenate([np.zeros((1, 8)), u, -u])
    assert len({tuple(r) for r in S1}) == 8 and len({tuple(r) for r in S2}) == 5
    digits = np.array([(a, b, c) for a in range(256) for b in range(8) for c in range(5)])
    digits = digits[rng.permutation(len(digits))]
    X = S0[digits[:, 0]] + S1[digits[:, 1]] + S2[digits[:, 2]]
    return X.astype(np.float32).reshape(160, 512), digits, (S0, S1, S2)


def _first_with(digits, **want):
    cols = {"s0": 0, "s1": 1, "s2": 2}
    m = np.ones(len(digits), bool)
    for k, v in want.items():
        m &= digits[:, cols[k]] == v
    return int(np.flatnonzero(m)[0])


@pytest.mark.parametrize("iters", [1, 3])
def test_rvq_fit_recovers_a_separated_balanced_lattice(iters):
    """Stage 0 starts each centroid at a member away from its cluster's centre (S0[k] + v1 + u1) and
    must reach the exact centre in one Lloyd iteration (the mean of 40 members); stages 1 and 2
    start at residuals equal to their entries (repeated over the 256 centroids, the copies with higher
    index staying empty), which only the correct residual makes exact.  Codes = the digits, and the
    fitted codebooks rebuild every sub-vector exactly."""
    W, digits, (S0, S1, S2) = _lattice_data(21)
    init = np.zeros((3, 256), np.int32)
    for c in range(256):
        init[0, c] = _first_with(digits, s0=c, s1=0, s2=1)
        init[1, c] = _first_with(digits, s1=c % 8, s2=0)
        init[2, c] = _first_with(digits, s2=c % 5)
    cb, codes = oracle.rvq_fit(W, iters, init)
    assert np.array_equal(cb[0], S0.astype(np.float32))
    assert np.array_equal(cb[1], S1[np.arange(256) % 8].astype(np.float32))
    assert np.array_equal(cb[2], S2[np.arange(256) % 5].astype(np.float32))
    assert np.array_equal(codes.reshape(-1, 3), digits)
    rebuilt = (cb[0][codes[..., 0]] + cb[1][codes[..., 1]] + cb[2][codes[..., 2]]).reshape(W.shape)
    assert np.array_equal(rebuilt, W)
    # no iteration: the centroids are the chosen sub-vectors themselves
    cb0, _ = oracle.rvq_fit(W, 0, init)
    assert np.array_equal(cb0[0], W.reshape(-1, 8)[init[0]])


def _gauss_fit_input(seed, rows=125, cols=320, dup=40):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((rows, cols)).astype(np.float32)
    n = rows * cols // 8
    init = np.stack([rng.choice(n, 256, replace=False) for _ in range(3)]).astype(np.int32)
    init[0, 256 - dup:] = init[0, :dup]          # repeated starts: those copies begin empty
    return W, init


@pytest.mark.parametrize("K", [1, 2, 5])
def test_rvq_fit_update_is_the_mean_of_the_previous_assignment(K):
    """Lloyd's update, checked against an exact sum: the stage-0 centroids after K iterations are the
    means (math.fsum, correctly rounded, within one fp32 ulp) of the sub-vectors that the last
    assignment of a (K-1)-iteration run gave them; a centroid without members keeps its value."""
    import math
    W, init = _gauss_fit_input(5)
    X = W.reshape(-1, 8).astype(np.float64)
    cbp, codesp = oracle.rvq_fit(W, K - 1, init)
    cb, _ = oracle.rvq_fit(W, K, init)
    a = codesp.reshape(-1, 3)[:, 0]
    empty = 0
    for c in range(256):
        m = np.flatnonzero(a == c)
        if len(m) == 0:
            empty += 1
            assert np.array_equal(cb[0, c], cbp[0, c])
            continue
        exact = np.array([math.fsum(X[m, j]) / len(m) for j in range(8)], dtype=np.float32)
        ulp = np.spacing(np.abs(exact))
        assert np.all(np.abs(cb[0, c] - exact) <= ulp), c
    if K == 1:
        assert empty >= 40   # the repeated starts lose every tie to their lower-index twins


def test_rvq_fit_initialises_each_stage_from_its_residual():
    """With no iteration, stage s's centroids are the sub-vectors init[s] of what stages < s left,
    rounded to fp32 (the residual itself is exact: formed in fp64 from the earlier stages' codes and
    centroids, numpy here)."""
    W, init = _gauss_fit_input(6)
    cb, codes = oracle.rvq_fit(W, 0, init)
    R = W.reshape(-1, 8).astype(np.float64)
    c = codes.reshape(-1, 3)
    for s in range(3):
        assert np.array_equal(cb[s], R[init[s]].astype(np.float32)), s
        R = R - cb[s][c[:, s]].astype(np.float64)


def test_rvq_fit_codes_are_the_encoding_with_the_fitted_codebooks():
    """The last assignment of each stage is the residual encoder's decision (pinned above): the fit's
    codes equal rvq_encode of W with the fitted codebooks, bit for bit."""
    W, init = _gauss_fit_input(7)
    cb, codes = oracle.rvq_fit(W, 4, init)
    assert np.array_equal(codes, oracle.rvq_encode(W, cb))


def test_rvq_fit_distortion_never_increases():
    """Lloyd's monotonicity: the stage-0 squared error does not grow with the iteration count, and
    the three-stage error is far below stage 0's."""
    W, init = _gauss_fit_input(8)
    X = W.reshape(-1, 8).astype(np.float64)
    prev = None
    for it in range(7):
        cb, codes = oracle.rvq_fit(W, it, init)
        c = codes.reshape(-1, 3)
        d0 = float(np.sum((X - cb[0][c[:, 0]]) ** 2))
        if prev is not None:
            assert d0 <= prev * (1 + 1e-6), it
        prev = d0
    d3 = float(np.sum((X - cb[0][c[:, 0]] - cb[1][c[:, 1]] - cb[2][c[:, 2]]) ** 2))
    assert d3 < 0.5 * d0
