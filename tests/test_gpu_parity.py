"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances (relative L2 over the whole output unless stated):
  fp32 tables: 1e-5;  fp16 tables: 2e-3;  router ids: bit-exact;
  gates: 1e-6 relative;  logits (fp64 on both sides): 1e-12 relative.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
import synth
from quant_checks import compare_with_oracle_codes
from workloads import (HIDDEN, INTER, LAYER_EXPERTS, MATVEC_COLS, MATVEC_ROWS, TOP_K, oracle_expert, pack_spec,
                       rel_l2, router, upload_bank)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-5, "f16": 2e-3}


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def packed_matrix(seed, rows, cols, matrix=synth.SINGLE, expert=0):
    codes = synth.matrix_codes(seed, 0, expert, matrix, rows, cols)
    cb = synth.matrix_codebooks(seed, 0, expert, matrix)
    packed = rvq.pack_codes(to_dev(codes), rows, cols)
    return codes, cb, packed, to_dev(cb)


# ---------------------------------------------------------------- packing (byte permutation, exact)

@pytest.mark.parametrize("rows,cols", [(256, 512), (1, 8), (65, 136), (300, 800), (2048, 7168), (7168, 2048)])
def test_pack_matches_layout_spec(rows, cols):
    say(f"pack {rows}x{cols}")
    codes = synth.matrix_codes(0xA1, 0, 0, synth.SINGLE, rows, cols)
    packed = rvq.pack_codes(to_dev(codes), rows, cols).cpu().numpy()
    assert np.array_equal(packed, pack_spec(codes, rows, cols))


# ---------------------------------------------------------------- partial-dot tables

def test_lut_build_f32_matvec_config():
    say("lut f32 256x512")
    x = synth.activation_f32(synth.SEED_MATVEC, 0, MATVEC_COLS)
    cb = synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)
    lut, e = rvq.lut_build(to_dev(x), to_dev(cb), "f32")
    T = oracle.lut(cb, x)
    absT = oracle.lut(np.abs(cb), np.abs(x))          # sum_j |C_s[c][j] x_j|
    got = lut.cpu().numpy().astype(np.float64)
    assert int(e.item()) == 0
    assert (np.abs(got - T) <= 8 * 2.0 ** -24 * absT + 1e-30).all()


@pytest.mark.parametrize("cols,scale", [(512, 1.0), (7168, 1.0), (2048, 3.0e4), (136, 1e-3)])
def test_lut_build_f16(cols, scale):
    say(f"lut f16 cols={cols} scale={scale}")
    x = (synth.activation_f32(0xB2, 0, cols) * np.float32(scale)).astype(np.float32)
    cb = synth.matrix_codebooks(0xB2, 0, 0, synth.SINGLE)
    lut, e = rvq.lut_build(to_dev(x), to_dev(cb), "f16")
    e = int(e.item())
    got = lut.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    T = oracle.lut(cb, x)
    assert np.abs(T).max() * 2.0 ** -e < 65504
    absT = oracle.lut(np.abs(cb), np.abs(x))
    err = np.abs(got * 2.0 ** e - T)
    # fp16 rounding (half ulp = 2^-11 relative), fp32 dot error, and subnormal spacing 2^-24 (scaled)
    bound = 2.0 ** -11 * np.abs(T) + 16 * 2.0 ** -24 * absT + 2.0 ** (e - 24)
    assert (err <= bound).all()


# ---------------------------------------------------------------- single-matrix GEMV

@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_gemv_matvec_config(dtype):
    say(f"gemv 256x512 {dtype}")
    codes, cb, packed, cbd = packed_matrix(synth.SEED_MATVEC, MATVEC_ROWS, MATVEC_COLS)
    x = synth.activation_f32(synth.SEED_MATVEC, 0, MATVEC_COLS)
    y = rvq.expert_gemv(packed, cbd, MATVEC_ROWS, MATVEC_COLS, to_dev(x), dtype).cpu().numpy()
    ref = oracle.gemv(codes, cb, MATVEC_ROWS, MATVEC_COLS, x)
    err = rel_l2(y, ref)
    say(f"  rel-L2 {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rows,cols", [(1, 8), (7, 120), (64, 128), (65, 136), (300, 264), (129, 800), (5, 8 * 33)])
def test_gemv_ragged_shapes(rows, cols, dtype):
    say(f"gemv {rows}x{cols} {dtype}")
    codes, cb, packed, cbd = packed_matrix(0xC3 + rows, rows, cols)
    x = synth.activation_f32(0xC3, rows, cols)
    y = rvq.expert_gemv(packed, cbd, rows, cols, to_dev(x), dtype).cpu().numpy()
    ref = oracle.gemv(codes, cb, rows, cols, x)
    assert rel_l2(y, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_gemv_full_size_sampled(dtype):
    rows, cols = INTER, HIDDEN
    say(f"gemv {rows}x{cols} {dtype}")
    codes, cb, packed, cbd = packed_matrix(synth.SEED_EXPERT, rows, cols, synth.GATE)
    x = synth.activation_f32(synth.SEED_EXPERT, 0, cols)
    y = rvq.expert_gemv(packed, cbd, rows, cols, to_dev(x), dtype).cpu().numpy()
    ref = oracle.gemv(codes, cb, rows, cols, x)
    assert rel_l2(y, ref) <= TOL[dtype]


def test_gemv_is_deterministic():
    say("gemv determinism")
    codes, cb, packed, cbd = packed_matrix(0xD4, 2048, 7168)
    x = to_dev(synth.activation_f32(0xD4, 0, 7168))
    a = rvq.expert_gemv(packed, cbd, 2048, 7168, x, "f32")
    b = rvq.expert_gemv(packed, cbd, 2048, 7168, x, "f32")
    assert torch.equal(a, b)


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("E,H,k", [(LAYER_EXPERTS, HIDDEN, TOP_K), (64, HIDDEN, TOP_K), (300, 1000, 7), (16, 64, 16),
                                   (4096, 512, 64)])   # the largest expert count and k accepted
def test_router_topk_matches_oracle(E, H, k):
    say(f"router E={E} H={H} k={k}")
    bits, w = router(synth.SEED_LAYER, 0, E, H)
    X = np.stack([synth.activation_f32(synth.SEED_LAYER, t, H) for t in range(8)])
    ids, gates, logits = rvq.router_topk(w, to_dev(X), k)
    ids, gates, logits = ids.cpu().numpy(), gates.cpu().numpy(), logits.cpu().numpy()
    L = oracle.router_logits(bits, X)
    np.testing.assert_allclose(logits, L, rtol=1e-12, atol=1e-12 * np.abs(L).max())
    for t in range(X.shape[0]):
        ids_o, gates_o, _ = oracle.topk(L[t], k)
        assert np.array_equal(ids[t], ids_o), (t, ids[t], ids_o)
        np.testing.assert_allclose(gates[t], gates_o, rtol=1e-6)


def test_router_bf16_tokens():
    say("router bf16 x")
    E, H, k = LAYER_EXPERTS, HIDDEN, TOP_K
    bits, w = router(synth.SEED_LAYER, 0, E, H)
    xb = np.stack([synth.activation_bf16_bits(synth.SEED_CHUNK, t, H) for t in range(16)])
    xt = to_dev(xb.view(np.int16)).view(torch.bfloat16)
    ids, gates, logits = rvq.router_topk(w, xt, k)
    L = oracle.router_logits(bits, synth.bf16_bits_to_f32(xb))
    for t in range(16):
        ids_o, gates_o, _ = oracle.topk(L[t], k)
        assert np.array_equal(ids[t].cpu().numpy(), ids_o)
        np.testing.assert_allclose(gates[t].cpu().numpy(), gates_o, rtol=1e-6)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E,H,T", [(37, 7168, 7), (256, 264, 5), (8, 7168, 64)])
def test_router_tiles_equal_one_token(x_dtype, E, H, T):
    """Several tokens at once (4-expert x 4-token tiles) give every token the logits, ids and gates
    of a one-token call bit for bit, with experts and tokens ragged against the tiles, and agree
    with the oracle's fp64 logits to rounding."""
    say(f"router tiles E={E} H={H} T={T} {x_dtype}")
    bits = synth.router_bf16_bits(0x7A ^ E, 0, E, H)
    w = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    if x_dtype == "f32":
        X = np.stack([synth.activation_f32(0x7A, t, H) for t in range(T)])
        Xd, Xo = to_dev(X), X.astype(np.float64)
    else:
        Xb = np.stack([synth.activation_bf16_bits(0x7A, t, H) for t in range(T)])
        Xd = to_dev(Xb.view(np.int16)).view(torch.bfloat16)
        Xo = (Xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = min(16, E)
    ids, gates, logits = rvq.router_topk(w, Xd, k)
    for t in range(T):
        ids1, gates1, logits1 = rvq.router_topk(w, Xd[t], k)
        assert torch.equal(logits[t], logits1[0]), t
        assert torch.equal(ids[t], ids1[0]) and torch.equal(gates[t], gates1[0]), t
    lo = oracle.router_logits(bits, Xo)
    np.testing.assert_allclose(logits.cpu().numpy(), lo, rtol=1e-12, atol=1e-12 * np.abs(lo).max())


def test_router_exact_ties_and_edge_k():
    say("router ties")
    E, H = 12, 32
    bits = synth.router_bf16_bits(0xE5, 0, E, H)
    bits[5] = bits[2]          # identical rows -> identical logits -> lower id first
    bits[9] = bits[2]
    w = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    x = synth.activation_f32(0xE5, 0, H)
    for k in (1, 3, E):
        ids, gates, logits = rvq.router_topk(w, to_dev(x), k)
        ids_o, gates_o, _ = oracle.topk(oracle.router_logits(bits, x[None, :])[0], k)
        assert np.array_equal(ids[0].cpu().numpy(), ids_o)
        np.testing.assert_allclose(gates[0].cpu().numpy(), gates_o, rtol=1e-6)
        if k == 1:
            assert gates[0, 0].item() == 1.0
    l = logits[0].cpu().numpy()
    assert l[5] == l[2] == l[9]


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_matches_oracle():
    say("rmsnorm")
    X = np.stack([synth.activation_f32(0xF6, t, HIDDEN) * np.float32(0.1 * (t + 1)) for t in range(4)])
    out = rvq.rmsnorm(to_dev(X), 1e-6).cpu().numpy()
    for t in range(4):
        ref = oracle.rmsnorm(X[t].astype(np.float64), 1e-6)
        assert rel_l2(out[t], ref) <= 1e-6


# ---------------------------------------------------------------- one SwiGLU expert (k = 1)

@pytest.fixture(scope="module")
def expert_bank():
    say("upload single-expert bank (7168/2048)")
    bank = upload_bank(synth.SEED_EXPERT, 0, 4)
    return bank


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_single_expert_decode(expert_bank, dtype):
    say(f"expert 7168/2048 {dtype}")
    x = synth.activation_f32(synth.SEED_EXPERT, 0, HIDDEN)
    for e in (0, 3):
        ids = torch.tensor([e], dtype=torch.int32, device=DEV)
        gates = torch.ones(1, dtype=torch.float32, device=DEV)
        y = rvq.moe_layer_forward(expert_bank, to_dev(x), ids, gates, dtype=dtype).cpu().numpy()
        ref = oracle.expert(oracle_expert(synth.SEED_EXPERT, 0, e), x)
        err = rel_l2(y, ref)
        say(f"  expert {e} rel-L2 {err:.3e}")
        assert err <= TOL[dtype]


def test_single_expert_layer_equals_three_gemvs(expert_bank):
    """Cross-path: the fused layer (k = 1) and three standalone GEMVs with a host-side SwiGLU agree."""
    say("expert cross-path")
    x = to_dev(synth.activation_f32(synth.SEED_EXPERT, 1, HIDDEN))
    b = expert_bank
    e = 1
    def mat(m, rows, cols):
        off = b.matrix_offset(e, m)
        return b.codes[off:off + rvq.packed_bytes(rows, cols)], b.codebooks[e, m].contiguous()
    g = rvq.expert_gemv(*mat(0, INTER, HIDDEN), INTER, HIDDEN, x)
    u = rvq.expert_gemv(*mat(1, INTER, HIDDEN), INTER, HIDDEN, x)
    h = (g.double() * torch.sigmoid(g.double()) * u.double()).float()
    y3 = rvq.expert_gemv(*mat(2, HIDDEN, INTER), HIDDEN, INTER, h)
    y1 = rvq.moe_layer_forward(b, x, torch.tensor([e], dtype=torch.int32, device=DEV),
                               torch.ones(1, device=DEV))
    assert rel_l2(y1.cpu().numpy(), y3.cpu().numpy()) <= 2e-6


def test_invalid_expert_id_sets_status_and_is_skipped(expert_bank):
    say("invalid expert id")
    x = to_dev(synth.activation_f32(synth.SEED_EXPERT, 2, HIDDEN))
    ws = rvq.make_moe_workspace(expert_bank, 1, 2, "f32")
    assert rvq.check_device_status(ws) == 0
    gates = torch.tensor([0.75, 0.25], device=DEV)
    y_bad = rvq.moe_layer_forward(expert_bank, x, torch.tensor([2, 99], dtype=torch.int32, device=DEV), gates,
                                  workspace=ws)
    assert rvq.check_device_status(ws) == rvq._lib.RVQ_ERR_EXPERT_ID
    assert rvq.check_device_status(ws) == 0          # cleared
    y_one = rvq.moe_layer_forward(expert_bank, x, torch.tensor([2], dtype=torch.int32, device=DEV),
                                  torch.tensor([0.75], device=DEV))
    assert torch.equal(y_bad, y_one)
    assert rvq.check_device_status(ws) == 0


# ---------------------------------------------------------------- one MoE layer (256 experts, top-16)

@pytest.fixture(scope="module")
def layer_bank():
    say("upload 256-expert layer bank (4.2 GB)")
    bank = upload_bank(synth.SEED_LAYER, 0, LAYER_EXPERTS)
    bits, w = router(synth.SEED_LAYER, 0, LAYER_EXPERTS, HIDDEN)
    return bank, bits, w


def _layer_oracle_getter(seed=None, H=HIDDEN, I=INTER):
    seed = synth.SEED_LAYER if seed is None else seed
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(seed, 0, e, H, I)
        return cache[e]
    return get


def _rows_match_oracle(get, bits, X, R, y, ids, gates, tokens, k, dtype):
    """Rows `tokens` of a batch output against the oracle's layer, token by token: the same ids, gates
    to 1e-6, and the MoE part (output minus residual) within the table precision's tolerance."""
    for t in tokens:
        r = None if R is None else R[t]
        y_ref, ids_ref, gates_ref, _ = oracle.moe_layer(get, bits, X[t], k, residual=r)
        assert np.array_equal(ids[t], ids_ref), t
        np.testing.assert_allclose(gates[t], gates_ref, rtol=1e-6)
        base = 0.0 if r is None else r
        err = rel_l2(y[t] - base, y_ref - base)
        say(f"  token {t}: rel-L2 {err:.3e} against the oracle")
        assert err <= TOL[dtype], t


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_moe_layer_decode(layer_bank, dtype):
    bank, bits, w = layer_bank
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, dtype)
    cache = {}
    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(synth.SEED_LAYER, 0, e)
        return cache[e]
    for t in (0, 1):
        say(f"moe layer token {t} {dtype}")
        x = synth.activation_f32(synth.SEED_LAYER, t, HIDDEN)
        r = synth.activation_f32(synth.SEED_LAYER, 1000 + t, HIDDEN)
        xd = to_dev(x)
        ids, gates, _ = rvq.router_topk(w, xd, TOP_K)
        y = rvq.moe_layer_forward(bank, xd, ids[0], gates[0], residual=to_dev(r), dtype=dtype, workspace=ws)
        y = y.cpu().numpy()
        y_ref, ids_ref, gates_ref, gaps = oracle.moe_layer(get, bits, x, TOP_K, residual=r)
        assert np.array_equal(ids[0].cpu().numpy(), ids_ref)
        np.testing.assert_allclose(gates[0].cpu().numpy(), gates_ref, rtol=1e-6)
        err = rel_l2(y - r, y_ref - r)           # the MoE part alone
        say(f"  rel-L2 {err:.3e} (boundary gap {gaps[0]:.2e})")
        assert err <= TOL[dtype]
        assert rel_l2(y, y_ref) <= TOL[dtype]
    assert rvq.check_device_status(ws) == 0


def test_moe_layer_is_deterministic(layer_bank):
    say("moe layer determinism")
    bank, bits, w = layer_bank
    x = to_dev(synth.activation_f32(synth.SEED_LAYER, 5, HIDDEN))
    ids, gates, _ = rvq.router_topk(w, x, TOP_K)
    a = rvq.moe_layer_forward(bank, x, ids[0], gates[0])
    b = rvq.moe_layer_forward(bank, x, ids[0], gates[0])
    assert torch.equal(a, b)


def test_topk_ties_across_blocks(layer_bank):
    """Top-k of 256 logits with many exact ties inside and across the 64-expert blocks of the
    selection (router rows repeated with period 37, and a group of rows set to the largest one):
    rvq_router_topk equals the oracle's order (logit desc, lower id first) for k = 1, 16, 64, and the
    top-k inside the gate/up kernel (rvq_moe_decode_routed, fp32 tables) gives the same ids and gates."""
    say("top-k ties across blocks (256 experts)")
    bank, bits0, _ = layer_bank
    E = LAYER_EXPERTS
    bits = bits0.copy()
    for j in range(37, E):
        bits[j] = bits[j % 37]
    x = synth.activation_f32(synth.SEED_LAYER, 41, HIDDEN)
    lo = oracle.router_logits(bits, x[None, :])[0]
    top = int(np.argmax(lo))
    for j in (3, 70, 130, 200, 255):
        bits[j] = bits[top]              # ties at the top, in four different blocks
    w = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    xd = to_dev(x)
    lo = oracle.router_logits(bits, x[None, :])[0]
    assert len(np.unique(lo)) == 37
    for k in (1, 16, 64):
        ids, gates, logits = rvq.router_topk(w, xd, k)
        ids_o, gates_o, _ = oracle.topk(lo, k)
        assert np.array_equal(ids[0].cpu().numpy(), ids_o), k
        np.testing.assert_allclose(gates[0].cpu().numpy(), gates_o, rtol=1e-6)
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, "f32")
    y, ids_r, gates_r, _ = rvq.moe_decode_routed(bank, w, xd, TOP_K, dtype="f32", workspace=ws)
    ids2, gates2, _ = rvq.router_topk(w, xd, TOP_K)
    assert torch.equal(ids_r, ids2[0]) and torch.equal(gates_r, gates2[0])
    assert torch.equal(y, rvq.moe_layer_forward(bank, xd, ids2[0], gates2[0], dtype="f32", workspace=ws))
    assert rvq.check_device_status(ws) == 0


def test_topk_all_logits_equal(layer_bank):
    """All 256 router rows equal, so all logits are equal: every expert is a candidate with the same
    key, and the selection's exact fixup of equal keys decides the whole order (by id alone: ids
    0 .. k-1, each gate 1/k, as the oracle gives), for fp32 and fp16 tables; the two-call form agrees
    bit for bit."""
    say("top-k: all logits equal")
    bank, bits0, _ = layer_bank
    bits = np.repeat(bits0[:1], LAYER_EXPERTS, axis=0)
    x = synth.activation_f32(synth.SEED_LAYER, 47, HIDDEN)
    lo = oracle.router_logits(bits, x[None, :])[0]
    assert len(np.unique(lo)) == 1
    ids_o, gates_o, _ = oracle.topk(lo, TOP_K)
    assert list(ids_o) == list(range(TOP_K))
    w = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    xd = to_dev(x)
    for dtype in ("f32", "f16"):
        ws = rvq.make_moe_workspace(bank, 1, TOP_K, dtype)
        y, ids_r, gates_r, _ = rvq.moe_decode_routed(bank, w, xd, TOP_K, dtype=dtype, workspace=ws)
        assert np.array_equal(ids_r.cpu().numpy(), ids_o), dtype
        np.testing.assert_allclose(gates_r.cpu().numpy(), gates_o, rtol=1e-6)
        ids2, gates2, _ = rvq.router_topk(w, xd, TOP_K)
        assert torch.equal(ids_r, ids2[0]) and torch.equal(gates_r, gates2[0])
        assert torch.equal(y, rvq.moe_layer_forward(bank, xd, ids2[0], gates2[0], dtype=dtype, workspace=ws))
        assert rvq.check_device_status(ws) == 0


def near_tie_router(bits0, x, h0, gaps):
    """Router rows, copies of the top row of bits0 on x, raised by gaps[i] bf16 ulps at element h0
    (positive there), at ids 10, 100, 200, ...: their logits differ by a few ulps of w[h0] times x[h0]."""
    lo = oracle.router_logits(bits0, x[None, :])[0]
    top = int(np.argmax(lo))
    bits = bits0.copy()
    ids = [j for j in (10, 100, 200, 250) if j != top][:len(gaps)]
    for j, d in zip(ids, gaps):
        bits[j] = bits[top]
        bits[j, h0] = bits[top, h0] + d
    return bits, ids, top


def test_topk_orders_logits_equal_in_fp32_by_fp64(layer_bank):
    """Logits that round to the same fp32 value but differ in fp64 keep their fp64 order, not their
    id order: the selection compares 32-bit keys of the fp32-rounded logits first and must decide
    equal keys in fp64 (then by id).  Copies of the top router row at three ids, the later ones
    raised at one element by 1 and 2 bf16 ulps times a small x there, so the larger logits sit at the
    larger ids; rvq_router_topk (one-pass ranks for E = 256, two passes for
    E = 4096) and the routed decode's in-kernel top-k must give the oracle's order."""
    say("top-k: logits equal in fp32, distinct in fp64")
    bank, bits0, _ = layer_bank
    x = synth.activation_f32(synth.SEED_LAYER, 43, HIDDEN)
    lo0 = oracle.router_logits(bits0, x[None, :])[0]
    top = int(np.argmax(lo0))
    row = (bits0[top].astype(np.uint32) << 16).view(np.float32)
    h0 = int(np.flatnonzero((row > 0) & (np.abs(x) > 0))[-1])
    found = ids_t = None
    for scale in 2.0 ** -np.arange(8, 40):
        xs = x.copy()
        xs[h0] = np.float32(scale)
        bits, ids_t, _ = near_tie_router(bits0, xs, h0, [0, 1, 2])
        lo = oracle.router_logits(bits, xs[None, :])[0]
        l = lo[ids_t]
        if l[0] < l[1] < l[2] and len(set(np.float32(l).tolist())) == 1 and np.float32(l[0]) == np.float32(lo[top]):
            found = (xs, bits, lo, ids_t)
            break
    assert found is not None
    xs, bits, lo, ids_t = found
    xd = to_dev(xs)
    w = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    for k in (1, 2, 4, 16):
        ids, gates, logits = rvq.router_topk(w, xd, k)
        ids_o, gates_o, _ = oracle.topk(lo, k)
        assert np.array_equal(ids[0].cpu().numpy(), ids_o), (k, ids[0].cpu().numpy(), ids_o)
        np.testing.assert_allclose(gates[0].cpu().numpy(), gates_o, rtol=1e-6)
    assert list(oracle.topk(lo, 2)[0]) == ids_t[:0:-1]   # the larger logits at the larger ids come first
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, "f32")
    y, ids_r, gates_r, _ = rvq.moe_decode_routed(bank, w, xd, TOP_K, dtype="f32", workspace=ws)
    ids_o, gates_o, _ = oracle.topk(lo, TOP_K)
    assert np.array_equal(ids_r.cpu().numpy(), ids_o)
    np.testing.assert_allclose(gates_r.cpu().numpy(), gates_o, rtol=1e-6)
    assert rvq.check_device_status(ws) == 0
    # 4096 experts (the two-pass form): the same 256 rows repeated, near-ties at the top of each copy
    big = np.concatenate([bits] * 16)
    wb = to_dev(big.view(np.int16)).view(torch.bfloat16)
    lb = oracle.router_logits(big, xs[None, :])[0]
    for k in (3, 16, 64):
        ids, gates, _ = rvq.router_topk(wb, xd, k)
        ids_o, gates_o, _ = oracle.topk(lb, k)
        assert np.array_equal(ids[0].cpu().numpy(), ids_o), k
        np.testing.assert_allclose(gates[0].cpu().numpy(), gates_o, rtol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_routed_decode_matches_two_calls_and_oracle(layer_bank, dtype):
    """rvq_moe_decode_routed (top-k taken inside the gate/up kernel, for fp32 and fp16 tables) gives
    the ids and gates of rvq_router_topk bit for bit, the output of rvq_moe_layer_forward on them bit
    for bit, and the oracle's layer within tolerance."""
    bank, bits, w = layer_bank
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, dtype)
    cache = {}
    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(synth.SEED_LAYER, 0, e)
        return cache[e]
    for t in (2, 3):
        say(f"routed decode token {t} {dtype}")
        x = synth.activation_f32(synth.SEED_LAYER, t, HIDDEN)
        r = synth.activation_f32(synth.SEED_LAYER, 1000 + t, HIDDEN)
        xd, rd = to_dev(x), to_dev(r)
        y, ids, gates, logits = rvq.moe_decode_routed(bank, w, xd, TOP_K, residual=rd, dtype=dtype, workspace=ws)
        ids2, gates2, logits2 = rvq.router_topk(w, xd, TOP_K)
        y2 = rvq.moe_layer_forward(bank, xd, ids2[0], gates2[0], residual=rd, dtype=dtype, workspace=ws)
        assert torch.equal(logits, logits2[0])
        assert torch.equal(ids, ids2[0])
        assert torch.equal(gates, gates2[0])
        assert torch.equal(y, y2)
        y_ref, ids_ref, gates_ref, _ = oracle.moe_layer(get, bits, x, TOP_K, residual=r)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        np.testing.assert_allclose(gates.cpu().numpy(), gates_ref, rtol=1e-6)
        assert rel_l2(y.cpu().numpy() - r, y_ref - r) <= TOL[dtype]
    assert rvq.check_device_status(ws) == 0


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_block_decode_matches_norm_then_routed_and_oracle(layer_bank, dtype):
    """rvq_moe_block_decode (RMSNorm folded into the router kernel) equals rvq_rmsnorm followed by
    rvq_moe_decode_routed(x = n, residual = h) bit for bit, also in place (h_out aliasing h), and the
    oracle's pre-norm block within tolerance."""
    bank, bits, w = layer_bank
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, dtype)
    cache = {}
    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(synth.SEED_LAYER, 0, e)
        return cache[e]
    for t, scale in ((4, 3.5), (5, 0.02)):
        say(f"block decode token {t} {dtype}")
        h = synth.activation_f32(synth.SEED_LAYER, 2000 + t, HIDDEN) * np.float32(scale)
        hd = to_dev(h)
        y, ids, gates, logits = rvq.moe_block_decode(bank, w, hd, TOP_K, 1e-6, dtype=dtype, workspace=ws)
        n = rvq.rmsnorm(hd[None, :], 1e-6)[0]
        y2, ids2, gates2, logits2 = rvq.moe_decode_routed(bank, w, n, TOP_K, residual=hd, dtype=dtype, workspace=ws)
        assert torch.equal(logits, logits2) and torch.equal(ids, ids2) and torch.equal(gates, gates2)
        assert torch.equal(y, y2)
        hin = hd.clone()
        y3, ids3, _, _ = rvq.moe_block_decode(bank, w, hin, TOP_K, 1e-6, dtype=dtype, h_out=hin, workspace=ws)
        assert torch.equal(hin, y) and torch.equal(ids3, ids)
        n_ref = oracle.rmsnorm(h.astype(np.float64), 1e-6)
        y_ref, ids_ref, gates_ref, gaps = oracle.moe_layer(get, bits, n_ref, TOP_K, residual=h)
        # the kernels route on n rounded to fp32, which moves a logit by at most 2^-24 sum |w n|; the
        # kept experts and their order are then unique while every gap exceeds twice that
        wf = (np.asarray(bits, dtype=np.uint32).reshape(-1, HIDDEN) << 16).view(np.float32).astype(np.float64)
        assert min(gaps) > 2.0 * 2.0 ** -24 * float((np.abs(wf) @ np.abs(n_ref)).max())
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        np.testing.assert_allclose(gates.cpu().numpy(), gates_ref, rtol=1e-5)
        assert rel_l2(y.cpu().numpy() - h, y_ref - h) <= TOL[dtype]
    assert rvq.check_device_status(ws) == 0


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_batch_decode_equals_single_token_calls(layer_bank, dtype):
    """rvq_moe_batch_decode runs T tokens' pairs in the same launches, each chunked as for one token:
    rows 0 and T-1 against the oracle's layer, every row equal to a single-token
    rvq_moe_layer_forward bit for bit, y may alias the residual, and the workspace is reusable across
    batch sizes."""
    bank, bits, w = layer_bank
    T = 5
    say(f"batch decode T={T} {dtype}")
    X = np.stack([synth.activation_f32(synth.SEED_LAYER, 40 + t, HIDDEN) for t in range(T)])
    R = np.stack([synth.activation_f32(synth.SEED_LAYER, 1040 + t, HIDDEN) for t in range(T)])
    xd, rd = to_dev(X), to_dev(R)
    ids, gates, _ = rvq.router_topk(w, xd, TOP_K)
    ws = rvq.make_batch_workspace(bank, T, TOP_K, dtype)
    y = rvq.moe_batch_decode(bank, xd, ids, gates, residual=rd, dtype=dtype, workspace=ws)
    _rows_match_oracle(_layer_oracle_getter(), bits, X, R, y.cpu().numpy(), ids.cpu().numpy(),
                       gates.cpu().numpy(), (0, T - 1), TOP_K, dtype)
    for t in range(T):
        y1 = rvq.moe_layer_forward(bank, xd[t], ids[t], gates[t], residual=rd[t], dtype=dtype, workspace=ws)
        assert torch.equal(y[t], y1), t
    yin = rd[:3].clone()
    rvq.moe_batch_decode(bank, xd[:3], ids[:3], gates[:3], residual=yin, dtype=dtype, y=yin, workspace=ws)
    assert torch.equal(yin, y[:3])
    assert rvq.check_device_status(ws) == 0


@pytest.mark.parametrize("k,T", [(1, 6), (2, 4), (1, 48)])
def test_batch_decode_few_experts_per_token(layer_bank, k, T):
    """k = 1 and k = 2 on the 256-expert layer: few pairs per token, so gate/up leaves more partial
    sums per row than the down kernel reads (the partial-sum kernel runs) and the down kernel may take
    one row block per streamer wave.  With 48 one-expert tokens the batch has pairs enough for down's
    four-block row split while a single-token call takes one row block per wave: the rows differ, the
    sums must not.  Rows against the oracle (all of them, or 6 of the 48), and every row bit-equal to
    single-token calls."""
    bank, bits, w = layer_bank
    X = np.stack([synth.activation_f32(synth.SEED_LAYER, 4000 + 10 * k + t, HIDDEN) for t in range(T)])
    xd = to_dev(X)
    ids, gates, _ = rvq.router_topk(w, xd, k)
    get = _layer_oracle_getter()
    rows = range(T) if T <= 8 else (0, 1, 17, 30, 46, 47)
    for dtype in ("f32", "f16"):
        say(f"batch decode T={T} k={k} {dtype}")
        y = rvq.moe_batch_decode(bank, xd, ids, gates, dtype=dtype)
        _rows_match_oracle(get, bits, X, None, y.cpu().numpy(), ids.cpu().numpy(), gates.cpu().numpy(),
                           rows, k, dtype)
        for t in range(T):
            assert torch.equal(y[t], rvq.moe_layer_forward(bank, xd[t], ids[t], gates[t], dtype=dtype)), t


@pytest.mark.parametrize("H,I,E,k", [
    (1024, 2048, 8, 4),    # no wave-specialised down: tokens run one after another
    (3584, 2048, 4, 2),    # both wave-specialised kernels (one K-tile per workgroup)
])
def test_batch_decode_other_shapes(H, I, E, k):
    say(f"batch decode H={H} I={I} E={E} k={k}")
    seed = synth.SEED_EXPERT ^ (H * 131 + I)
    bank = upload_bank(seed, 0, E, H, I)
    bits, w = router(seed, 0, E, H)
    T = 3
    X = np.stack([synth.activation_f32(seed, 200 + t, H) for t in range(T)])
    xd = to_dev(X)
    ids, gates, _ = rvq.router_topk(w, xd, k)
    get = _layer_oracle_getter(seed, H, I)
    for dtype in ("f32", "f16"):
        y = rvq.moe_batch_decode(bank, xd, ids, gates, dtype=dtype)
        _rows_match_oracle(get, bits, X, None, y.cpu().numpy(), ids.cpu().numpy(), gates.cpu().numpy(),
                           range(T), k, dtype)
        for t in range(T):
            assert torch.equal(y[t], rvq.moe_layer_forward(bank, xd[t], ids[t], gates[t], dtype=dtype)), (dtype, t)


def test_batch_decode_at_max_tokens(layer_bank):
    """The largest batch (256 tokens x top-16 = 4096 pairs in one set of launches): two rows against
    the oracle, sampled rows equal single-token calls bit for bit."""
    bank, bits, w = layer_bank
    T = 256
    say(f"batch decode T={T} f16")
    X = np.stack([synth.activation_f32(synth.SEED_LAYER, 3000 + t, HIDDEN) for t in range(T)])
    xd = to_dev(X)
    ids, gates, _ = rvq.router_topk(w, xd, TOP_K)
    ws = rvq.make_batch_workspace(bank, T, TOP_K, "f16")
    y = rvq.moe_batch_decode(bank, xd, ids, gates, dtype="f16", workspace=ws)
    _rows_match_oracle(_layer_oracle_getter(), bits, X, None, y.cpu().numpy(), ids.cpu().numpy(),
                       gates.cpu().numpy(), (1, 254), TOP_K, "f16")
    for t in (0, 1, 100, 254, 255):
        y1 = rvq.moe_layer_forward(bank, xd[t], ids[t], gates[t], dtype="f16", workspace=ws)
        assert torch.equal(y[t], y1), t
    assert rvq.check_device_status(ws) == 0


def test_batch_decode_invalid_id_is_skipped(expert_bank):
    """An id outside [0, E) in one token of a batch sets RVQ_ERR_EXPERT_ID and contributes zero,
    as in a single-token call; the other tokens are unaffected."""
    bank = expert_bank
    say("batch decode with an invalid id")
    X = to_dev(np.stack([synth.activation_f32(synth.SEED_EXPERT, 60 + t, HIDDEN) for t in range(2)]))
    ids = torch.tensor([[0, 1], [1, 99]], dtype=torch.int32, device="cuda")
    gates = torch.tensor([[0.25, 0.75], [0.5, 0.5]], dtype=torch.float32, device="cuda")
    ws = rvq.make_batch_workspace(bank, 2, 2, "f32")
    y = rvq.moe_batch_decode(bank, X, ids, gates, workspace=ws)
    assert rvq.check_device_status(ws) == 6
    for t in range(2):
        y1 = rvq.moe_layer_forward(bank, X[t], ids[t], gates[t], workspace=ws)
        assert torch.equal(y[t], y1)
    assert rvq.check_device_status(ws) == 6


def record_payload(bank, e):
    n = 2 * bank.gate_bytes + bank.down_bytes
    return bank.codes[e * bank.stride: e * bank.stride + n].cpu().numpy()


def test_bank_crc32_matches_oracle(expert_bank):
    """CRC-32 of each record's packed code payload, bit-exact against the oracle's bitwise CRC of the
    same bytes; a flipped byte changes only that record's value (and matches the oracle again)."""
    bank = expert_bank
    say("bank crc32 (4 experts, 16.5 MB records)")
    crc = rvq.bank_crc32(bank).cpu().numpy().view(np.uint32)
    for e in range(bank.E):
        assert int(crc[e]) == oracle.crc32(record_payload(bank, e)), e
    pos = 2 * bank.stride + 12_345_679
    saved = bank.codes[pos].clone()
    bank.codes[pos] ^= 0x40
    try:
        crc2 = rvq.bank_crc32(bank).cpu().numpy().view(np.uint32)
        assert int(crc2[2]) != int(crc[2]) and int(crc2[2]) == oracle.crc32(record_payload(bank, 2))
        assert all(int(crc2[e]) == int(crc[e]) for e in (0, 1, 3))
    finally:
        bank.codes[pos] = saved
    torch.cuda.synchronize()


def test_bank_crc32_ragged_and_layer(layer_bank):
    """A shape whose records end in a partial 64 KiB block (72 KiB payloads), and sampled experts of
    the 256-expert layer bank."""
    say("bank crc32 ragged shape and layer samples")
    small = upload_bank(synth.SEED_EXPERT ^ 77, 0, 3, 256, 200)
    crc = rvq.bank_crc32(small).cpu().numpy().view(np.uint32)
    for e in range(3):
        assert int(crc[e]) == oracle.crc32(record_payload(small, e)), e
    bank = layer_bank[0]
    crc = rvq.bank_crc32(bank).cpu().numpy().view(np.uint32)
    for e in (0, 97, 255):
        assert int(crc[e]) == oracle.crc32(record_payload(bank, e)), e


def _digit_setup(rows, cols, seed):
    rng = np.random.default_rng(seed)
    W = (16 * rng.integers(0, 2, (rows, cols)) + 4 * rng.integers(0, 2, (rows, cols))
         + rng.integers(0, 2, (rows, cols))).astype(np.float32)
    bits = ((np.arange(256)[:, None] >> np.arange(8)[None, :]) & 1).astype(np.float32)
    cb = np.stack([16.0 * bits, 4.0 * bits, bits]).astype(np.float32)
    Wi = W.astype(np.int64)
    codes = np.zeros((rows, cols // 8, 3), dtype=np.uint8)
    for s_, d in enumerate(((Wi >> 4) & 1, (Wi >> 2) & 1, Wi & 1)):
        codes[:, :, s_] = (d.reshape(rows, cols // 8, 8) << np.arange(8)).sum(axis=2).astype(np.uint8)
    return W, cb, codes


@pytest.mark.parametrize("rows,cols", [(256, 512), (100, 264), (1, 8)])
def test_rvq_encode_matches_oracle(rows, cols):
    """GPU residual encoding (fp32 decisions) against the oracle's fp64 decisions: every group equal
    except where the oracle's best and second-best distances lie within the fp32 rounding bound of
    each other, and those groups are nearest-entry picks along their own path (quant_checks.py).
    Weights near the code lattice (a decode plus noise) and plain Gaussian weights; the digit case
    recovers the codes built by bit extraction exactly."""
    say(f"rvq encode {rows}x{cols}")
    cb = synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)
    rng = np.random.default_rng(rows * 31 + cols)
    c0 = rng.integers(0, 256, (rows, cols // 8, 3)).astype(np.uint8)
    W1 = (oracle.dequant(c0, cb, rows, cols) + 0.05 * rng.standard_normal((rows, cols))).astype(np.float32)
    W2 = rng.standard_normal((rows, cols)).astype(np.float32)
    cbd = to_dev(cb)
    for W in (W1, W2):
        got = rvq.rvq_encode(to_dev(W), cbd).cpu().numpy()
        want, margins = oracle.rvq_encode(W, cb, margins=True)
        flipped = compare_with_oracle_codes(W, cb, got, want, margins)
        assert flipped <= max(1, got.size // 3000)
    Wd, cbdig, codes = _digit_setup(rows, cols, rows + cols)
    assert np.array_equal(rvq.rvq_encode(to_dev(Wd), to_dev(cbdig)).cpu().numpy(), codes)


def test_rvq_encode_full_size_sampled():
    """A 2048 x 7168 gate matrix (decode of its codes plus noise): sampled rows against the oracle (as
    above), and the round trip through the packed decode path (encode -> pack -> table GEMV) against
    the oracle's GEMV of the recovered codes."""
    say("rvq encode 2048x7168")
    rows, cols = INTER, HIDDEN
    ex = synth.Expert(synth.SEED_EXPERT, 0, 1, HIDDEN, INTER)
    cb = ex.codebooks(synth.GATE)
    rng = np.random.default_rng(5)
    W = (oracle.dequant(ex.codes(synth.GATE), cb, rows, cols) + 0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    codes = rvq.rvq_encode(to_dev(W), to_dev(cb)).cpu().numpy()
    for r in (0, 1, 777, 2047):
        want, margins = oracle.rvq_encode(W[r:r + 1], cb, margins=True)
        assert compare_with_oracle_codes(W[r:r + 1], cb, codes[r:r + 1], want, margins) <= 1, r
    x = synth.activation_f32(synth.SEED_EXPERT, 3, cols)
    packed = rvq.pack_codes(torch.from_numpy(codes).cuda(), rows, cols)
    y = rvq.expert_gemv(packed, to_dev(cb), rows, cols, to_dev(x), "f32").cpu().numpy()
    assert rel_l2(y, oracle.gemv(codes, cb, rows, cols, x)) <= 1e-5


def test_graph_replays_match_eager(layer_bank):
    """The benchmark replays HIP graphs of the decode entry points: every replay, with new inputs
    copied in eagerly between replays, equals an eager call on the same inputs bit for bit (routed
    step, pre-norm block in place, and a 3-token batch)."""
    bank, bits, w = layer_bank
    say("graph replays vs eager")
    k = TOP_K
    ws = rvq.make_moe_workspace(bank, 1, k, "f32")
    wsb = rvq.make_batch_workspace(bank, 3, k, "f32")
    xin = torch.empty(HIDDEN, dtype=torch.float32, device="cuda")
    hblk = torch.empty_like(xin)
    y = torch.empty_like(xin)
    ids = torch.empty(k, dtype=torch.int32, device="cuda")
    gates = torch.empty(k, dtype=torch.float32, device="cuda")
    logits = torch.empty(LAYER_EXPERTS, dtype=torch.float64, device="cuda")
    xb = torch.empty(3, HIDDEN, dtype=torch.float32, device="cuda")
    idsb = torch.empty(3, k, dtype=torch.int32, device="cuda")
    gatesb = torch.empty(3, k, dtype=torch.float32, device="cuda")
    yb = torch.empty(3, HIDDEN, dtype=torch.float32, device="cuda")

    def routed():
        rvq.moe_decode_routed(bank, w, xin, k, y=y, ids=ids, gates=gates, logits=logits, workspace=ws)

    def block():
        rvq.moe_block_decode(bank, w, hblk, k, 1e-6, h_out=hblk, ids=ids, gates=gates, logits=logits, workspace=ws)

    def batch():
        rvq.moe_batch_decode(bank, xb, idsb, gatesb, y=yb, workspace=wsb)

    def inputs(t):
        xs = np.stack([synth.activation_f32(synth.SEED_LAYER, 500 + 4 * t + j, HIDDEN) for j in range(4)])
        return to_dev(xs)
    X0 = inputs(0)
    xin.copy_(X0[0]); hblk.copy_(X0[1]); xb.copy_(X0[1:])
    ib, gb, _ = rvq.router_topk(w, xb, k)
    idsb.copy_(ib); gatesb.copy_(gb)
    routed(); block(); batch()
    torch.cuda.synchronize()
    graphs = []
    for fn in (routed, block, batch):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    for t in range(1, 5):
        X = inputs(t)
        ib, gb, _ = rvq.router_topk(w, X[1:], k)
        # eager references on the same inputs
        ref_y, ref_ids, _, _ = rvq.moe_decode_routed(bank, w, X[0], k, workspace=ws)
        ref_h, _, _, _ = rvq.moe_block_decode(bank, w, X[1], k, 1e-6, workspace=ws)
        ref_b = rvq.moe_batch_decode(bank, X[1:], ib, gb, workspace=wsb)
        xin.copy_(X[0]); hblk.copy_(X[1]); xb.copy_(X[1:]); idsb.copy_(ib); gatesb.copy_(gb)
        graphs[0].replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(ids, ref_ids), t
        graphs[1].replay()
        torch.cuda.synchronize()
        assert torch.equal(hblk, ref_h), t
        graphs[2].replay()
        torch.cuda.synchronize()
        assert torch.equal(yb, ref_b), t
    assert rvq.check_device_status(ws) == 0 and rvq.check_device_status(wsb) == 0


def test_routed_decode_small_expert_count():
    """Top-k inside the gate/up kernel with fewer experts than wave lanes, k = 1 and k = E."""
    E, k_all = 5, 5
    say("routed decode, 5 experts")
    bank = upload_bank(synth.SEED_EXPERT, 7, E)
    bits, w = router(synth.SEED_EXPERT, 7, E, HIDDEN)
    x = to_dev(synth.activation_f32(synth.SEED_EXPERT, 70, HIDDEN))
    for k in (1, k_all):
        y, ids, gates, _ = rvq.moe_decode_routed(bank, w, x, k)
        ids2, gates2, _ = rvq.router_topk(w, x, k)
        assert torch.equal(ids, ids2[0]) and torch.equal(gates, gates2[0])
        assert torch.equal(y, rvq.moe_layer_forward(bank, x, ids2[0], gates2[0]))


def test_block_decode_few_experts_and_unaligned_h():
    """The norm-folding router's loop form (taken when a workgroup writes more than 256 elements of
    n, here 1434 with 5 experts, and when h is not 16-byte aligned) equals rvq_rmsnorm followed by
    the routed decode bit for bit, as its one-round form does on the full layer."""
    E, k = 5, 3
    say("block decode, 5 experts, h aligned and offset by one float")
    bank = upload_bank(synth.SEED_EXPERT, 7, E)
    _, w = router(synth.SEED_EXPERT, 7, E, HIDDEN)
    ws = rvq.make_moe_workspace(bank, 1, k, "f32")
    buf = torch.empty(HIDDEN + 4, dtype=torch.float32, device="cuda")
    h = torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT, 71, HIDDEN))
    for off in (0, 1):
        hd = buf[off:off + HIDDEN]
        hd.copy_(h)
        y, ids, gates, logits = rvq.moe_block_decode(bank, w, hd, k, 1e-6, workspace=ws)
        n = rvq.rmsnorm(hd[None, :], 1e-6)[0]
        y2, ids2, gates2, logits2 = rvq.moe_decode_routed(bank, w, n, k, residual=hd, workspace=ws)
        assert torch.equal(logits, logits2) and torch.equal(ids, ids2) and torch.equal(gates, gates2), off
        assert torch.equal(y, y2), off
    assert rvq.check_device_status(ws) == 0


# ---------------------------------------------------------------- other layer shapes

@pytest.mark.parametrize("H,I,E,k", [
    (256, 128, 8, 4),      # one-K-tile-per-workgroup kernels (gate/up rows != 2048)
    (264, 200, 6, 3),      # ragged: 33 groups, 200 rows (partial row block), both fallbacks
    (1024, 2048, 8, 4),    # wave-specialised gate/up, fallback down (16 row blocks of H)
    (3584, 2048, 4, 2),    # both wave-specialised kernels, 2 row chunks of down
    (256, 128, 64, 64),    # the largest k: every expert selected
    (1024, 2048, 64, 64),  # the largest k through the wave-specialised gate/up (and its in-kernel ranking)
    (256, 2048, 300, 16),  # in-kernel top-k over a ragged expert count (300: 4 whole waves and a part)
    (128, 2048, 768, 16),  # the most experts the in-kernel top-k takes (a thread per expert)
])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_moe_layer_other_shapes(H, I, E, k, dtype):
    say(f"moe layer H={H} I={I} E={E} k={k} {dtype}")
    seed = synth.SEED_EXPERT ^ (H * 131 + I)
    bank = upload_bank(seed, 0, E, H, I)
    bits, w = router(seed, 0, E, H)
    cache = {}
    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(seed, 0, e, H, I)
        return cache[e]
    ws = rvq.make_moe_workspace(bank, 1, k, dtype)
    for t in (0, 1):
        x = synth.activation_f32(seed, t, H)
        r = synth.activation_f32(seed, 100 + t, H)
        xd, rd = to_dev(x), to_dev(r)
        ids, gates, _ = rvq.router_topk(w, xd, k)
        y = rvq.moe_layer_forward(bank, xd, ids[0], gates[0], residual=rd, dtype=dtype, workspace=ws)
        y_ref, ids_ref, _, _ = oracle.moe_layer(get, bits, x, k, residual=r)
        assert np.array_equal(ids[0].cpu().numpy(), ids_ref)
        err = rel_l2(y.cpu().numpy() - r, y_ref - r)
        say(f"  rel-L2 {err:.3e}")
        assert err <= TOL[dtype]
        y2, ids2, gates2, _ = rvq.moe_decode_routed(bank, w, xd, k, residual=rd, dtype=dtype, workspace=ws)
        assert torch.equal(ids2, ids[0]) and torch.equal(gates2, gates[0]) and torch.equal(y2, y)
    assert rvq.check_device_status(ws) == 0


def test_bounded_waits_give_up_and_report(layer_bank):
    """Failure path of the wave-specialised kernels, forced from the host: with their bounded waits cut
    to zero polls in one workspace they still finish (every access stays in bounds) and that workspace
    reports RVQ_ERR_DEVICE_STALL, while a second workspace used in between keeps the default and gives
    the exact result; the default limit then brings back the exact result in the first as well."""
    say("bounded waits cut to zero polls")
    bank, bits, w = layer_bank
    x = to_dev(synth.activation_f32(synth.SEED_LAYER, 9, HIDDEN))
    ids, gates, _ = rvq.router_topk(w, x, TOP_K)
    ws = rvq.make_moe_workspace(bank, 1, TOP_K, "f32")
    other = rvq.make_moe_workspace(bank, 1, TOP_K, "f32")
    ref = rvq.moe_layer_forward(bank, x, ids[0], gates[0], workspace=ws)
    assert rvq.check_device_status(ws) == 0
    rvq.set_wait_limit(ws, 0)
    rvq.moe_layer_forward(bank, x, ids[0], gates[0], workspace=ws)
    assert rvq.check_device_status(ws) == 8  # RVQ_ERR_DEVICE_STALL
    assert torch.equal(rvq.moe_layer_forward(bank, x, ids[0], gates[0], workspace=other), ref)
    assert rvq.check_device_status(other) == 0
    rvq.set_wait_limit(ws, -1)
    again = rvq.moe_layer_forward(bank, x, ids[0], gates[0], workspace=ws)
    assert rvq.check_device_status(ws) == 0
    assert torch.equal(again, ref)
    rvq.set_wait_limit(ws, 0)
    rvq.workspace_init(ws)              # a zero-filled header is the default limit again
    assert torch.equal(rvq.moe_layer_forward(bank, x, ids[0], gates[0], workspace=ws), ref)
    assert rvq.check_device_status(ws) == 0

def test_stream_read_reference_sizes():
    """rvq_stream_read (the bench's read-rate reference: one workgroup per CU over a contiguous part,
    16 loads in flight per thread) on sizes that do not split evenly: parts ending inside a batch of
    loads, fewer 16-byte pieces than a workgroup's threads, and more workgroups than the CUs could
    each fill.  It writes nothing but its sink word, which no input here can reach (all-zero and
    all-ones data fold to 0)."""
    say("stream read reference sizes")
    for nbytes in (16, 4096, 65536 + 48, (1 << 20) + 16 * 37, 48 << 20):
        for fill in (0, 255):
            src = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
            sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
            rvq.stream_read(src, sink)
            torch.cuda.synchronize()
            assert int(sink.item()) == 7, (nbytes, fill)
