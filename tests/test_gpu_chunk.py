"""Chunked prefill through one MoE layer (T tokens at once): bucketing by expert, RVQ groups decoded
into MFMA operands, grouped expert GEMMs, gated combine; against the fp64 oracle.

Tile precision and bound: fp16 tiles (weights summed in fp16 from fp16 codebooks, h scaled per pair
by a power of two) must meet rel-L2 <= 2e-3.  bf16 tiles round the weights and h to bf16 (8-bit
significand).  One such rounding of a value with a log-uniform significand has relative standard
deviation 2^-7 * sqrt(E[(1/m)^2]) / sqrt(12) = 2^-7 * 0.736 / 3.46 = 1.66e-3 (m in [1, 2)); the
output sees four independent ones in a chain (gate weights, up weights, h, down weights; x is bf16
already), each carried into the output at about its own relative size because the sums average
independent errors, so rel-L2 ~ sqrt(4) * 1.66e-3 = 3.3e-3 (measured 3.3e-3).  bf16 is held to 4e-3,
1.2x that expectation; it is also reported against 2e-3, which only the fp16 tiles meet.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
import synth
from workloads import CHUNK_TOKENS, HIDDEN, INTER, LAYER_EXPERTS, TOP_K, oracle_expert, rel_l2, router, upload_bank

pytestmark = pytest.mark.gpu
TOL = {"f16": 2e-3, "bf16": 4e-3}


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def chunk_x(seed, T, H):
    bits = np.stack([synth.activation_bf16_bits(seed, t, H) for t in range(T)])
    return bits, torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def run_case(seed, E, H, I, T, k, dtype, tokens=None, residual=False, bank=None, rt=None):
    if bank is None:
        bank = upload_bank(seed, 0, E, H, I)
    bits, w = rt if rt is not None else router(seed, 0, E, H)
    xb, xt = chunk_x(seed, T, H)
    res = synth.normal_f32(seed, synth.tensor_id(synth.KIND_ACT_F32, 7, 0), T * H).reshape(T, H) if residual else None
    ids, gates, _ = rvq.router_topk(w, xt, k)
    y = rvq.moe_layer_forward(bank, xt, ids, gates, residual=None if res is None else torch.from_numpy(res).cuda(),
                              dtype=dtype)
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(seed, 0, e, H, I)
        return cache[e]
    Y, ids_o, gates_o = oracle.moe_chunk(get, bits, synth.bf16_bits_to_f32(xb), k, residual=res, tokens=tokens)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_allclose(gates.cpu().numpy(), gates_o, rtol=1e-6)
    got = y.cpu().numpy()
    if tokens is not None:
        got = got[np.asarray(tokens)]
    err = rel_l2(got, Y)
    say(f"  {dtype}: rel-L2 {err:.3e}")
    return err, bank, y, ids, gates, xt


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunk_small_layer(dtype):
    say(f"chunk E=32 H=512 I=256 T=64 k=4 {dtype}")
    err = run_case(0xC1, 32, 512, 256, 64, 4, dtype)[0]
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunk_crowded_experts_and_residual(dtype):
    """8 experts, top-2 of 200 tokens: about 50 tokens per expert, some over the 64-token pass."""
    say(f"chunk E=8 H=256 I=128 T=200 k=2 {dtype}")
    err = run_case(0xC2, 8, 256, 128, 200, 2, dtype, residual=True)[0]
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("H,I", [(192, 128), (128, 192)])
def test_chunk_odd_row_block_count(dtype, H, I):
    """Three 64-row blocks: H = 192 makes down take one row block per step, I = 192 makes gate/up take
    one row block of each matrix per step (an even count takes two, as in the other cases); a K of 192
    also leaves a partial K-tile (gate/up for H = 192, down for I = 192)."""
    say(f"chunk E=8 H={H} I={I} T=40 k=2 {dtype}")
    err = run_case(0xC5, 8, H, I, 40, 2, dtype, residual=True)[0]
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunk_expert_count_not_a_multiple_of_8(dtype):
    """12 experts: the expert kernels take the experts in id order, XCD-major (the deal by pair count
    needs the experts to split evenly over the 8 XCDs), with the same results."""
    say(f"chunk E=12 H=256 I=128 T=40 k=3 {dtype}")
    err = run_case(0xC6, 12, 256, 128, 40, 3, dtype, residual=True)[0]
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunk_smallest(dtype):
    """The smallest chunk (2 tokens, top-2 of 16 experts): at most 4 experts have a pair, the other
    work items end at once, and each pass holds one or two pairs of a 16-pair block."""
    say(f"chunk E=16 H=256 I=128 T=2 k=2 {dtype}")
    err = run_case(0xC7, 16, 256, 128, 2, 2, dtype, residual=True)[0]
    assert err <= TOL[dtype]


def test_chunk_at_max_tokens():
    """The largest chunk accepted (4096 tokens; 8 experts, so about 1000 pairs per expert)."""
    say("chunk E=8 H=256 I=128 T=4096 k=2 f16")
    err = run_case(0xC4, 8, 256, 128, 4096, 2, "f16")[0]
    assert err <= TOL["f16"]


def test_chunk_is_deterministic():
    say("chunk determinism")
    _, bank, y, ids, gates, xt = run_case(0xC3, 16, 256, 128, 48, 3, "f16")
    y2 = rvq.moe_layer_forward(bank, xt, ids, gates, dtype="f16")
    assert torch.equal(y, y2)


def test_chunk_invalid_expert_id_sets_status():
    say("chunk invalid id")
    E, H, I, T, k = 8, 256, 128, 16, 2
    bank = upload_bank(0xC4, 0, E, H, I)
    _, xt = chunk_x(0xC4, T, H)
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    ids[:, 1] = 1
    ids[3, 1] = 77
    gates = torch.full((T, k), 0.5, device="cuda")
    ws = rvq.make_moe_workspace(bank, T, k, "f16")
    y = rvq.moe_layer_forward(bank, xt, ids, gates, dtype="f16", workspace=ws)
    assert rvq.check_device_status(ws) == rvq._lib.RVQ_ERR_EXPERT_ID
    ids[3, 1] = 1
    y_ok = rvq.moe_layer_forward(bank, xt, ids, gates, dtype="f16", workspace=ws)
    assert rvq.check_device_status(ws) == 0
    # the token with the bad id keeps only its valid expert's share
    assert torch.equal(y[:3], y_ok[:3]) and torch.equal(y[4:], y_ok[4:])


@pytest.fixture(scope="module")
def layer():
    say("upload 256-expert layer bank (4.2 GB)")
    return upload_bank(synth.SEED_LAYER, 0, LAYER_EXPERTS), router(synth.SEED_LAYER, 0, LAYER_EXPERTS, HIDDEN)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunk_512_tokens_full_layer(layer, dtype):
    """512 bf16 tokens through the 256-expert layer; all routing checked, 24 sampled tokens' outputs
    (all 7168 each) compared."""
    bank, rt = layer
    tokens = list(range(0, CHUNK_TOKENS, CHUNK_TOKENS // 24))[:24]
    say(f"chunk 512 tokens x 256 experts {dtype}")
    seed = synth.SEED_LAYER
    bits, w = rt
    xb = np.stack([synth.activation_bf16_bits(synth.SEED_CHUNK, t, HIDDEN) for t in range(CHUNK_TOKENS)])
    xt = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    ids, gates, _ = rvq.router_topk(w, xt, TOP_K)
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=LAYER_EXPERTS)
    say(f"  tokens per expert: min {counts.min()} max {counts.max()} mean {counts.mean():.1f}")
    y = rvq.moe_layer_forward(bank, xt, ids, gates, dtype=dtype).cpu().numpy()
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(seed, 0, e)
        return cache[e]
    Y, ids_o, gates_o = oracle.moe_chunk(get, bits, synth.bf16_bits_to_f32(xb), TOP_K, tokens=tokens)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_allclose(gates.cpu().numpy(), gates_o, rtol=1e-6)
    err = rel_l2(y[np.asarray(tokens)], Y)
    say(f"  {dtype}: rel-L2 {err:.3e} over {len(tokens)} tokens")
    assert err <= TOL[dtype]
