"""rvq_moe_decode_routed_scratch, the routed decode step that allocates nothing (its partial sums in the
library's static per-device array): through the C ABI, two calls in a row, the second on a smaller
layer, each equal bit for bit to rvq_moe_decode_routed with a workspace on the same inputs; layouts
past the array's 24 MiB are refused before anything runs; the caller's status words receive the
device status."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import rvq_quantized_moe_amd as rvq
import synth
from workloads import router, upload_bank

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def scratch_call(bank, w, x, k, dtype, residual, status):
    L = rvq.lib()
    dev = x.device
    y = torch.empty(bank.H, dtype=torch.float32, device=dev)
    ids = torch.empty(k, dtype=torch.int32, device=dev)
    gates = torch.empty(k, dtype=torch.float32, device=dev)
    logits = torch.empty(bank.E, dtype=torch.float64, device=dev)
    desc = bank.desc()
    st = L.rvq_moe_decode_routed_scratch(ctypes.byref(desc), _p(w), _p(x), k, _p(residual), _p(y), _p(ids), _p(gates),
                                         _p(logits), rvq._lib._table_dtype(dtype), _p(status),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, y, ids, gates, logits


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_scratch_decode_equals_workspace_decode(dtype):
    status = torch.zeros(64, dtype=torch.int32, device="cuda")   # 256 bytes
    assert status.data_ptr() % 256 == 0
    cases = [(synth.SEED_LAYER, 256, 7168, 2048, 16), (synth.SEED_EXPERT ^ 0x77, 32, 1024, 2048, 4)]
    for n, (seed, E, H, I, k) in enumerate(cases):   # the second call: a smaller layer
        say(f"scratch decode call {n}: E={E} H={H} I={I} k={k} {dtype}")
        bank = upload_bank(seed, 0, E, H, I)
        _, w = router(seed, 0, E, H)
        x = torch.from_numpy(synth.activation_f32(seed, 500 + n, H)).cuda()
        r = torch.from_numpy(synth.activation_f32(seed, 600 + n, H)).cuda()
        st, y, ids, gates, logits = scratch_call(bank, w, x, k, dtype, r, status)
        assert st == 0, rvq.status_string(st)
        ref = rvq.moe_decode_routed(bank, w, x, k, residual=r, dtype=dtype)
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(ids, ref[1]) and torch.equal(gates, ref[2])
        assert torch.equal(logits, ref[3])
        assert rvq.check_device_status(status) == 0
        del bank
        torch.cuda.empty_cache()


def test_scratch_decode_refuses_layouts_past_its_array():
    say("scratch decode: k = 64 at 7168/2048 needs more than 24 MiB")
    bank = rvq.ExpertBank(64, 7168, 2048, device="cuda")
    _, w = router(synth.SEED_LAYER, 0, 64, 7168)
    x = torch.zeros(7168, dtype=torch.float32, device="cuda")
    status = torch.zeros(64, dtype=torch.int32, device="cuda")
    st, *_ = scratch_call(bank, w, x, 64, "f32", None, status)
    assert st == rvq._lib.RVQ_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_scratch_decode_reports_device_status():
    """The caller's status words: the bounded waits cut to zero polls through word 1 give
    RVQ_ERR_DEVICE_STALL in word 0; cleared, and with the default limit, the exact result again."""
    seed, E, H, I, k = synth.SEED_EXPERT ^ 0x78, 32, 1024, 2048, 4
    say("scratch decode: forced stall through the status words")
    bank = upload_bank(seed, 0, E, H, I)
    _, w = router(seed, 0, E, H)
    x = torch.from_numpy(synth.activation_f32(seed, 1, H)).cuda()
    status = torch.zeros(64, dtype=torch.int32, device="cuda")
    ok = scratch_call(bank, w, x, k, "f32", None, status)
    assert ok[0] == 0 and rvq.check_device_status(status) == 0
    rvq.set_wait_limit(status, 0)
    assert scratch_call(bank, w, x, k, "f32", None, status)[0] == 0
    assert rvq.check_device_status(status) == 8     # RVQ_ERR_DEVICE_STALL
    rvq.set_wait_limit(status, -1)
    again = scratch_call(bank, w, x, k, "f32", None, status)
    assert again[0] == 0 and rvq.check_device_status(status) == 0
    assert torch.equal(again[1], ok[1])
