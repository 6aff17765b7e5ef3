"""92-layer expert stack, batch-1 decode (64 experts per layer, top-16, RMSNorm + residual between
layers, no attention): the HIP path against the fp64 oracle.

  h <- x_t;  for each layer l:  n = rmsnorm(h);  (ids, gates) = route_l(n);  h <- h + MoE_l(n)

Checks per decode step (the layer-by-layer comparison against an independent reference that the
WASTE pages describe for their own engine):
  * layer-wise: each GPU layer is given the oracle's own inputs for that layer (inputs flow
    oracle -> GPU only): RMSNorm of the oracle's h_l (rel-L2 <= 1e-6), the router on the oracle's
    n_l (ids bit-exact: both sides accumulate logits in fp64; gates 1e-6), and the MoE output on
    the oracle's n_l, ids and gates (rel-L2 <= 1e-5 with fp32 tables, 2e-3 with fp16 tables).
  * end-to-end: the GPU runs all 92 layers on its own (norm, router, layer as three calls; the
    fused block call must give the same final h bit for bit).  Its ids must equal the oracle's at every
    layer except where the oracle's own top-k boundary is a near-tie (gap < TAU); after such a
    divergence the step is not compared further.  92 routed layers amplify rounding-level
    differences about 400x (measured below: the oracle's own final h under a one-ulp change of x),
    so the end-to-end drift is reported and held to a sanity limit only.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
import synth
from workloads import RMS_EPS, TOP_K, Stack, rel_l2

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "f16": 2e-3}
# Largest oracle logit gap at which the free-running GPU may order experts differently.
TAU = {"f32": 1e-3, "f16": 5e-2}
SANITY = {"f32": 1e-3, "f16": 5e-2}


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.fixture(scope="module")
def stack():
    say("upload 92-layer stack (92 x 64 experts, 97 GB of codes)")
    return Stack()


def oracle_step(stack, x):
    """The oracle's trajectory: per layer (h_in, n, ids, gates, boundary gap, MoE output); final h."""
    h = np.asarray(x, dtype=np.float64)
    trace = []
    for l in range(stack.L):
        n = oracle.rmsnorm(h, RMS_EPS)
        cache = {}

        def get(e, l=l):
            if e not in cache:
                cache[e] = stack.oracle_expert(l, e)
            return cache[e]
        y, ids, gates, gaps = oracle.moe_layer(get, stack.router_bits[l], n, TOP_K)
        trace.append((h, n, ids, gates, gaps[0], y))
        h = h + y
    return h, trace


def gpu_free_step(stack, x, dtype, ws):
    h = dev32(x)
    ids_all = []
    for l in range(stack.L):
        n = rvq.rmsnorm(h, RMS_EPS)
        ids, gates, _ = rvq.router_topk(stack.routers[l], n, TOP_K)
        h = rvq.moe_layer_forward(stack.banks[l], n, ids[0], gates[0], residual=h, dtype=dtype, workspace=ws)
        ids_all.append(ids[0])
    return h.cpu().numpy(), [i.cpu().numpy() for i in ids_all]


def gpu_block_step(stack, x, dtype, ws):
    """The same free run through rvq_moe_block_decode (one call per layer, updated in place)."""
    h = dev32(x)
    for l in range(stack.L):
        rvq.moe_block_decode(stack.banks[l], stack.routers[l], h, TOP_K, RMS_EPS, dtype=dtype, h_out=h,
                             workspace=ws)
    return h.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_stack_decode_steps(stack, dtype):
    ws = rvq.make_moe_workspace(stack.banks[0], 1, TOP_K, dtype)
    flips = 0
    for t in (0, 1):
        x = synth.activation_f32(synth.SEED_STACK, t, stack.H)
        say(f"stack step {t} {dtype}: oracle trajectory")
        h_ref, trace = oracle_step(stack, x)
        if t == 0 and dtype == "f32":
            sign = np.where(synth.uniform_bytes(0x51, 1, stack.H) & 1, 1.0, -1.0)
            xp = np.nextafter(x, (x.astype(np.float64) + sign).astype(np.float32))
            h_p, _ = oracle_step(stack, xp)
            say(f"  oracle sensitivity to a 1-ulp input change: final h rel-L2 {rel_l2(h_p, h_ref):.3e}")
        say(f"stack step {t} {dtype}: layer-wise GPU on the oracle's inputs")
        worst = 0.0
        for l, (h_in, n, ids, gates, gap, y) in enumerate(trace):
            n_gpu = rvq.rmsnorm(dev32(h_in), RMS_EPS).cpu().numpy()
            assert rel_l2(n_gpu, n) <= 1e-6, l
            ids_g, gates_g, _ = rvq.router_topk(stack.routers[l], dev32(n), TOP_K)
            assert np.array_equal(ids_g[0].cpu().numpy(), ids), (l, gap)
            np.testing.assert_allclose(gates_g[0].cpu().numpy(), gates, rtol=1e-6)
            y_gpu = rvq.moe_layer_forward(stack.banks[l], dev32(n), dev32(ids).int(), dev32(gates),
                                          dtype=dtype, workspace=ws).cpu().numpy()
            err = rel_l2(y_gpu, y)
            worst = max(worst, err)
            assert err <= TOL[dtype], (l, err)
        say(f"  layer-wise MoE output: worst rel-L2 over 92 layers {worst:.3e}")
        say(f"stack step {t} {dtype}: end-to-end GPU")
        h_free, ids_gpu = gpu_free_step(stack, x, dtype, ws)
        assert np.array_equal(gpu_block_step(stack, x, dtype, ws), h_free)
        diverged = False
        for l in range(stack.L):
            ids_o, gap = trace[l][2], trace[l][4]
            if not np.array_equal(ids_gpu[l], ids_o):
                same_set = set(ids_gpu[l].tolist()) == set(ids_o.tolist())
                assert same_set or gap < TAU[dtype], (l, ids_gpu[l], ids_o, gap)
                if not same_set:
                    flips += 1
                    diverged = True
                    say(f"  layer {l}: top-k boundary near-tie (oracle gap {gap:.2e}); rest of step not compared")
                    break
        if not diverged:
            drift = rel_l2(h_free, h_ref)
            say(f"  end-to-end final h rel-L2 {drift:.3e} (drift)")
            assert drift <= SANITY[dtype]
    assert rvq.check_device_status(ws) == 0
    say(f"  near-tie divergences: {flips}")
