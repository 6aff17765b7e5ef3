"""Host-side contract of librvq.so, runnable without a GPU: the library loads,
exports every entry point include/rvq.h declares, and rejects invalid
arguments with the documented status before anything is enqueued (fake
non-NULL device pointers are used; no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

import rvq_quantized_moe_amd as rvq
from rvq_quantized_moe_amd import _lib
from workloads import pack_spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rvq.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WS, EXPERT_ID, HIP = range(8)
FAKE = 0x7f0000000000          # 256-byte aligned, never dereferenced by the validators
FAKE2 = 0x7f0000100000


@pytest.fixture(scope="module")
def L():
    return rvq.lib()


def test_exports_every_declared_symbol(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(rvq_[a-z0-9_]+)\s*\(", text))
    assert declared, "no declarations found"
    assert set(_lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(10):
        txt = rvq.status_string(s)
        assert txt.startswith("RVQ_")
    assert "unknown" in rvq.status_string(99)


def test_packed_bytes(L):
    assert rvq.packed_bytes(2048, 7168) == 5_505_024 == 2048 * 7168 * 3 // 8
    assert rvq.packed_bytes(7168, 2048) == 5_505_024
    assert rvq.packed_bytes(256, 512) == 49_152
    assert rvq.packed_bytes(1, 8) == 3072
    assert rvq.packed_bytes(65, 8 * 17) == 2 * 2 * 3072
    assert L.rvq_packed_bytes(0, 8) == 0 and L.rvq_packed_bytes(4, 12) == 0
    assert L.rvq_bank_record_bytes(7168, 2048) == 16_515_072
    for rows, cols in [(1, 8), (65, 136), (256, 512), (300, 800)]:
        assert pack_spec(np.zeros((rows, cols // 8, 3), np.uint8), rows, cols).size == rvq.packed_bytes(rows, cols)


def test_pack_spec_is_a_zero_padded_permutation():
    rng = np.random.default_rng(0)
    rows, cols = 70, 8 * 21
    codes = rng.integers(1, 256, size=(rows, cols // 8, 3)).astype(np.uint8)
    p = pack_spec(codes, rows, cols)
    assert np.array_equal(np.sort(p[p != 0]), np.sort(codes.reshape(-1)))
    # first KiB of the first slab = rows 0..63, bytes 0..15 of each row's run
    assert np.array_equal(p[:1024].reshape(64, 16), codes.reshape(rows, -1)[:64, :16])


def test_pack_validation(L):
    s = None
    assert L.rvq_pack_codes(None, 4, 8, FAKE, s) == NULL
    assert L.rvq_pack_codes(FAKE, 4, 8, None, s) == NULL
    assert L.rvq_pack_codes(FAKE, 0, 8, FAKE2, s) == SHAPE
    assert L.rvq_pack_codes(FAKE, 4, 12, FAKE2, s) == SHAPE
    assert L.rvq_pack_codes(FAKE, 4, 0, FAKE2, s) == SHAPE
    assert L.rvq_pack_codes(FAKE, 4, 8, FAKE2 + 8, s) == ALIGN


def test_lut_validation(L):
    s = None
    assert L.rvq_lut_build(None, 8, FAKE, 0, FAKE2, FAKE2, s) == NULL
    assert L.rvq_lut_build(FAKE, 8, FAKE, 0, FAKE2, None, s) == NULL
    assert L.rvq_lut_build(FAKE, 9, FAKE, 0, FAKE2, FAKE2, s) == SHAPE
    assert L.rvq_lut_build(FAKE, 8, FAKE, 2, FAKE2, FAKE2, s) == DTYPE
    assert L.rvq_lut_build(FAKE, 8, FAKE + 4, 0, FAKE2, FAKE2, s) == ALIGN


def _matrix(rows, cols, codes=FAKE, cb=FAKE2):
    return ctypes.byref(_lib.Matrix(codes, cb, rows, cols))


def test_gemv_validation(L):
    s = None
    need = L.rvq_expert_gemv_workspace_bytes(256, 512, 0)
    assert need == 4 * 256 * 4
    assert L.rvq_expert_gemv_workspace_bytes(256, 512, 1) == 2 * 256 * 4
    assert L.rvq_expert_gemv_workspace_bytes(256, 500, 0) == 0
    assert L.rvq_expert_gemv(None, FAKE, 0, FAKE, FAKE, need, s) == NULL
    assert L.rvq_expert_gemv(_matrix(256, 512, codes=None), FAKE, 0, FAKE, FAKE, need, s) == NULL
    assert L.rvq_expert_gemv(_matrix(256, 512), FAKE, 0, FAKE, None, need, s) == NULL
    assert L.rvq_expert_gemv(_matrix(0, 512), FAKE, 0, FAKE, FAKE, need, s) == SHAPE
    assert L.rvq_expert_gemv(_matrix(256, 511), FAKE, 0, FAKE, FAKE, need, s) == SHAPE
    assert L.rvq_expert_gemv(_matrix(256, 512), FAKE, 2, FAKE, FAKE, need, s) == DTYPE
    assert L.rvq_expert_gemv(_matrix(256, 512, codes=FAKE + 8), FAKE, 0, FAKE, FAKE, need, s) == ALIGN
    assert L.rvq_expert_gemv(_matrix(256, 512), FAKE, 0, FAKE, FAKE + 16, need, s) == ALIGN
    assert L.rvq_expert_gemv(_matrix(256, 512), FAKE, 0, FAKE, FAKE, need - 1, s) == WS


def test_router_validation(L):
    s = None
    a = (FAKE, FAKE2)
    assert L.rvq_router_topk(None, FAKE, 0, 1, 256, 7168, 16, FAKE, FAKE, FAKE, s) == NULL
    assert L.rvq_router_topk(*a, 0, 1, 256, 7168, 16, FAKE, FAKE, None, s) == NULL
    assert L.rvq_router_topk(*a, 0, 1, 256, 7168, 257, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.rvq_router_topk(*a, 0, 1, 256, 7168, 0, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.rvq_router_topk(*a, 0, 1, 5000, 7168, 16, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.rvq_router_topk(*a, 0, 1, 256, 7168, 65, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.rvq_router_topk(*a, 0, 0, 256, 7168, 16, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.rvq_router_topk(*a, 1, 1, 256, 7168, 16, FAKE, FAKE, FAKE, s) == DTYPE
    assert L.rvq_router_topk(FAKE + 1, FAKE2, 0, 1, 256, 7168, 16, FAKE, FAKE, FAKE, s) == ALIGN
    assert L.rvq_router_topk(*a, 0, 1, 256, 7168, 16, FAKE, FAKE, FAKE + 4, s) == ALIGN


def _bank(E=256, H=7168, I=2048, stride=16_515_072, codes=FAKE, cb=FAKE2):
    return ctypes.byref(_lib.BankDesc(codes, cb, stride, E, H, I))


def test_moe_workspace_size(L):
    n = L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 0)
    assert n == 256 + 16 * 2 * 56 * 2048 * 4 + 16 * 16 * 7168 * 4 + 7168 * 4   # + RMSNorm(h) of the block
    # partials are sized for 16-group K-tiles whatever the table precision
    assert L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 1) == n
    assert L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 2) == 0
    assert L.rvq_moe_layer_workspace_bytes(None, 1, 16, 0) == 0


def test_moe_validation(L):
    s = None
    n = L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 0)
    args = (FAKE, 0, 1, FAKE, FAKE, 16, None, FAKE, 0, FAKE, n, s)
    assert L.rvq_moe_layer_forward(None, *args) == NULL
    assert L.rvq_moe_layer_forward(_bank(codes=None), *args) == NULL
    assert L.rvq_moe_layer_forward(_bank(stride=16_515_072 + 8), *args) == ALIGN
    assert L.rvq_moe_layer_forward(_bank(stride=16_515_072 - 256), *args) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(E=0), *args) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(H=7170), *args) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 0, FAKE, FAKE, 16, None, FAKE, 0, FAKE, n, s) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 1, FAKE, FAKE, 65, None, FAKE, 0, FAKE, n, s) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 2, 1, FAKE, FAKE, 16, None, FAKE, 0, FAKE, n, s) == DTYPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 1, FAKE, FAKE, 16, None, FAKE, 2, FAKE, n, s) == DTYPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 1, FAKE, FAKE, 16, None, FAKE, 0, FAKE + 64, n, s) == ALIGN
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 1, FAKE, FAKE, 16, None, FAKE, 0, FAKE, n - 1, s) == WS
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, 1, None, FAKE, 16, None, FAKE, 0, FAKE, n, s) == NULL


def test_batch_decode_workspace_and_validation(L):
    """rvq_moe_batch_decode: the workspace holds the decode layout for T * k pairs; every check
    returns before anything is enqueued."""
    s = None
    q = L.rvq_moe_batch_decode_workspace_bytes
    n = q(_bank(), 4, 16, 0)
    assert n == 256 + 64 * 2 * 56 * 2048 * 4 + 64 * 16 * 7168 * 4 + 7168 * 4
    assert q(_bank(), 1, 16, 0) == L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 0)
    assert q(_bank(), 4, 16, 1) == n and q(_bank(), 4, 16, 2) == 0
    assert q(_bank(), 0, 16, 0) == 0 and q(_bank(), 257, 16, 0) == 0 and q(_bank(), 4, 65, 0) == 0
    assert q(None, 4, 16, 0) == 0
    f = L.rvq_moe_batch_decode
    ok = [FAKE, 4, FAKE, FAKE, 16, None, FAKE, 0, FAKE, n, s]

    def call(bank=None, **kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(bank if bank is not None else _bank(), *a)
    assert f(None, *ok) == NULL
    assert call(a0=None) == NULL and call(a2=None) == NULL and call(a6=None) == NULL and call(a8=None) == NULL
    assert call(_bank(E=0)) == SHAPE
    assert call(a1=0) == SHAPE and call(a1=257) == SHAPE     # T
    assert call(a4=0) == SHAPE and call(a4=65) == SHAPE      # k
    assert call(a7=2) == DTYPE                              # bf16 tables: no
    assert call(a0=FAKE + 2) == ALIGN and call(a8=FAKE + 64) == ALIGN
    assert call(a9=n - 1) == WS


def test_bank_crc32_validation(L):
    """rvq_bank_crc32: one word per 64 KiB block of every record in the workspace; every check returns
    before anything is enqueued."""
    q = L.rvq_bank_crc32_workspace_bytes
    n = q(_bank())
    assert n == 256 * 252 * 4   # 256 records; 16,515,072-byte payloads are 252 blocks of 64 KiB
    assert q(None) == 0 and q(_bank(E=0)) == 0
    f = L.rvq_bank_crc32
    assert f(None, FAKE, FAKE, n, None) == NULL
    assert f(_bank(), None, FAKE, n, None) == NULL and f(_bank(), FAKE, None, n, None) == NULL
    assert f(_bank(), FAKE + 2, FAKE, n, None) == ALIGN and f(_bank(), FAKE, FAKE + 64, n, None) == ALIGN
    assert f(_bank(), FAKE, FAKE, n - 1, None) == WS
    assert f(_bank(E=0), FAKE, FAKE, n, None) == SHAPE


def test_pool_validation(L):
    """Expert pool entry points: every argument check returns before any HIP call."""
    out = ctypes.c_void_p()
    c = L.rvq_pool_create
    ok = [FAKE, FAKE2, 16_515_072, 32, 7168, 2048, FAKE, FAKE2, 8]
    assert c(*ok, None) == NULL
    assert c(None, *ok[1:], ctypes.byref(out)) == NULL
    assert c(*ok[:6], None, *ok[7:], ctypes.byref(out)) == NULL
    assert c(*ok[:8], 0, ctypes.byref(out)) == SHAPE                      # no slots
    assert c(*ok[:3], 0, *ok[4:], ctypes.byref(out)) == SHAPE             # no experts
    assert c(*ok[:2], 16_515_072 - 256, *ok[3:], ctypes.byref(out)) == SHAPE
    assert c(*ok[:6], FAKE + 16, *ok[7:], ctypes.byref(out)) == ALIGN     # slot codes 256-aligned
    assert out.value is None
    ids = (ctypes.c_int32 * 2)(0, 1)
    assert L.rvq_pool_acquire(None, ids, 2, ids, None) == NULL
    assert L.rvq_pool_prefetch(None, ids, 2) == NULL
    v = ctypes.c_int64()
    assert L.rvq_pool_stats(None, ctypes.byref(v), ctypes.byref(v), ctypes.byref(v), ctypes.byref(v)) == NULL
    assert L.rvq_pool_destroy(None) == NULL


def test_routed_decode_validation(L):
    """Every check of rvq_moe_decode_routed returns before anything is enqueued."""
    s = None
    n = L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 0)
    f = L.rvq_moe_decode_routed
    ok = [FAKE, FAKE, 16, None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, n, s]

    def call(bank=None, **kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(bank if bank is not None else _bank(), *a)
    assert f(None, *ok) == NULL
    assert call(a0=None) == NULL                          # router weights
    assert call(a4=None) == NULL                          # y
    assert call(a7=None) == NULL                          # logits
    assert call(_bank(E=0)) == SHAPE
    assert call(a2=0) == SHAPE and call(a2=65) == SHAPE   # k
    assert call(a8=2) == DTYPE                            # bf16 tables: no
    assert call(a7=FAKE + 4) == ALIGN                     # logits are fp64
    assert call(a9=FAKE + 64) == ALIGN                    # workspace
    assert call(a10=n - 1) == WS


def test_block_decode_validation(L):
    s = None
    n = L.rvq_moe_layer_workspace_bytes(_bank(), 1, 16, 0)
    f = L.rvq_moe_block_decode
    ok = [FAKE, FAKE, 16, 1e-6, FAKE, FAKE, FAKE, FAKE, 0, FAKE, n, s]

    def call(bank=None, **kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(bank if bank is not None else _bank(), *a)
    assert f(None, *ok) == NULL
    assert call(a1=None) == NULL and call(a4=None) == NULL
    assert call(a3=-1.0) == SHAPE and call(a2=0) == SHAPE
    assert call(a8=2) == DTYPE
    assert call(a7=FAKE + 4) == ALIGN
    assert call(a10=n - 1) == WS


def test_chunk_workspace_and_validation(L):
    """T > 1 selects the chunk path: bf16 tokens, f16 or bf16 tiles."""
    s = None
    E, H, I, T, k = 256, 7168, 2048, 512, 16
    n = L.rvq_moe_layer_workspace_bytes(_bank(), T, k, 1)
    P = T * k
    up = lambda v: (v + 255) // 256 * 256
    # status, expert offsets, the expert order, pair token/position/h-scale, h (fp32), y rows (fp32),
    # the tokens and h as the tiles' 16-bit operands
    assert n == (256 + up((E + 1) * 4) + up(E * 4) + 3 * up(P * 4) + up(P * I * 4) + up(P * H * 4) + up(T * H * 2)
                 + up(P * I * 2))
    assert L.rvq_moe_layer_workspace_bytes(_bank(), T, k, 2) == n
    assert L.rvq_moe_layer_workspace_bytes(_bank(), T, k, 0) == 0          # fp32 tiles: no
    assert L.rvq_moe_layer_workspace_bytes(_bank(), 5000, k, 1) == 0       # too many tokens
    assert L.rvq_moe_layer_workspace_bytes(_bank(H=7176), T, k, 1) == 0    # rows not a multiple of 64
    ok = (FAKE, 2, T, FAKE, FAKE, k, None, FAKE, 1, FAKE, n, s)
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 0, T, FAKE, FAKE, k, None, FAKE, 1, FAKE, n, s) == DTYPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 2, T, FAKE, FAKE, k, None, FAKE, 0, FAKE, n, s) == DTYPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE + 2, 2, T, FAKE, FAKE, k, None, FAKE, 1, FAKE, n, s) == ALIGN
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 2, T, FAKE, FAKE, k, None, FAKE, 1, FAKE, n - 1, s) == WS
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 2, 5000, FAKE, FAKE, k, None, FAKE, 1, FAKE, n, s) == SHAPE
    assert L.rvq_moe_layer_forward(_bank(), FAKE, 2, T, FAKE, None, k, None, FAKE, 1, FAKE, n, s) == NULL
    del ok


def test_scratch_decode_validation(L):
    """The no-workspace routed decode: its arguments are checked as rvq_moe_decode_routed's, its status
    words must be given (256-byte aligned), and a layout past the static array (24 MiB) is refused."""
    s = None
    b = _bank(E=256)
    args = lambda **kw: (kw.get("bank", b), FAKE, FAKE, kw.get("k", 16), None, FAKE, FAKE, FAKE, FAKE,
                         kw.get("dtype", 0), kw.get("status", FAKE), s)
    assert L.rvq_moe_decode_routed_scratch(*args(status=None)) == NULL
    assert L.rvq_moe_decode_routed_scratch(*args(status=FAKE + 4)) == ALIGN
    assert L.rvq_moe_decode_routed_scratch(*args(dtype=2)) == DTYPE
    assert L.rvq_moe_decode_routed_scratch(*args(k=0)) == SHAPE
    assert L.rvq_moe_decode_routed_scratch(*args(k=64)) == WS          # 7168/2048 at k = 64: 88 MB of partials
    assert L.rvq_moe_layer_workspace_bytes(b, 1, 16, 0) <= 24 << 20     # the layer decode's k = 16 fits


def test_misc_validation(L):
    s = None
    assert L.rvq_rmsnorm(None, 1, 8, 1e-6, FAKE, s) == NULL
    assert L.rvq_rmsnorm(FAKE, 0, 8, 1e-6, FAKE, s) == SHAPE
    assert L.rvq_rmsnorm(FAKE, 1, 8, -1.0, FAKE, s) == SHAPE
    assert L.rvq_rmsnorm(FAKE, 1, 8, float("nan"), FAKE, s) == SHAPE
    assert L.rvq_workspace_init(None, 16, s) == NULL
    assert L.rvq_workspace_init(FAKE + 8, 16, s) == ALIGN
    assert L.rvq_check_device_status(None, s) == NULL
    assert L.rvq_workspace_set_wait_limit(None, 256, 0, s) == NULL
    assert L.rvq_workspace_set_wait_limit(FAKE + 8, 256, 0, s) == ALIGN
    assert L.rvq_workspace_set_wait_limit(FAKE, 255, 0, s) == WS
    assert L.rvq_workspace_set_wait_limit(FAKE, 256, 2 ** 31 - 1, s) == SHAPE


def test_validator_fuzz(L):
    """Random argument sets with at least one invalid field never pass validation."""
    rng = np.random.default_rng(1234)
    s = None
    bad_values = {"rows": [0, -1, -64], "cols": [0, 4, 12, 1001, -8], "dtype": [2, 3, -1, 7],
                  "align": [1, 2, 4, 8]}
    for _ in range(400):
        rows = int(rng.integers(1, 5000))
        cols = 8 * int(rng.integers(1, 1000))
        dtype = int(rng.integers(0, 2))
        codes = FAKE
        which = rng.choice(list(bad_values))
        if which == "rows":
            rows = int(rng.choice(bad_values["rows"]))
        elif which == "cols":
            cols = int(rng.choice(bad_values["cols"]))
        elif which == "dtype":
            dtype = int(rng.choice(bad_values["dtype"]))
        else:
            codes = FAKE + int(rng.choice(bad_values["align"]))
        st = L.rvq_expert_gemv(_matrix(rows, cols, codes=codes), FAKE, dtype, FAKE, FAKE, 1 << 40, s)
        assert st in (SHAPE, DTYPE, ALIGN), (which, rows, cols, dtype, st)
        st = L.rvq_pack_codes(FAKE, rows, cols, codes if which == "align" else FAKE2, s)
        if which in ("rows", "cols", "align"):
            assert st in (SHAPE, ALIGN), (which, st)


def test_stream_copy_validation(L):
    s = None
    assert L.rvq_stream_copy(None, FAKE, 16, s) == NULL
    assert L.rvq_stream_copy(FAKE, None, 16, s) == NULL
    assert L.rvq_stream_copy(FAKE, FAKE2, 17, s) == SHAPE
    assert L.rvq_stream_copy(FAKE + 4, FAKE2, 16, s) == ALIGN
    assert L.rvq_stream_copy(FAKE, FAKE2, 0, s) == OK


# ---- expert records (host-only: header layout and the read-time check) ----
REC_H, REC_I = 256, 128        # small shape: packed codes 36,864 B, record exactly 114,688 B (no padding)
RECORD = 9


def _spec_header(layer, expert, H, I, crc, codes_bytes):
    """The header as the documented layout states it, packed independently of the library."""
    import struct
    return struct.pack("<IIiiiiqqqqII", 0x45515652, 1, layer, expert, H, I, 4096, 73728, 4096 + 73728, codes_bytes,
                       crc, 0)


def _record(layer=3, expert=5, crc=0xDEADBEEF):
    rb = rvq.record_bytes(REC_H, REC_I)
    rec = np.zeros(rb, dtype=np.uint8)
    rec[:64] = np.frombuffer(rvq.record_header(layer, expert, REC_H, REC_I, crc), dtype=np.uint8)
    return rec


def test_record_layout_matches_the_documented_header(L):
    cb = L.rvq_bank_record_bytes(REC_H, REC_I)
    assert cb == 36864
    assert rvq.record_bytes(REC_H, REC_I) == 114688
    assert rvq.record_bytes(7168, 2048) == 16_592_896 == 4051 * 4096
    assert rvq.record_bytes(7168, 2048) - 77824 == L.rvq_bank_record_bytes(7168, 2048)
    assert ctypes.sizeof(rvq.RecordHeader) == 64
    assert rvq.record_header(3, 5, REC_H, REC_I, 0xDEADBEEF) == _spec_header(3, 5, REC_H, REC_I, 0xDEADBEEF, cb)
    assert rvq.record_header(91, 255, 7168, 2048, 1) == _spec_header(91, 255, 7168, 2048, 1, 16_515_072)
    h = rvq.RecordHeader()
    assert L.rvq_record_header_init(None, 0, 0, REC_H, REC_I, 0) == NULL
    assert L.rvq_record_header_init(ctypes.byref(h), -1, 0, REC_H, REC_I, 0) == SHAPE
    assert L.rvq_record_header_init(ctypes.byref(h), 0, -1, REC_H, REC_I, 0) == SHAPE
    assert L.rvq_record_header_init(ctypes.byref(h), 0, 0, REC_H, 12, 0) == SHAPE
    assert rvq.record_bytes(REC_H, 12) == 0


def test_record_check_accepts_the_standard_record(L):
    rec = _record()
    assert rvq.record_check(rec, 3, 5, REC_H, REC_I) == OK
    # the check reads the header only: payload bytes and the CRC field are not its business
    rec[4096:] = 0xA5
    assert rvq.record_check(rec, 3, 5, REC_H, REC_I) == OK
    # a record longer than the layout needs (padding after the codes) is fine
    assert rvq.record_check(np.concatenate([rec, np.zeros(4096, np.uint8)]), 3, 5, REC_H, REC_I) == OK


def test_record_check_refuses_wrong_identity_and_truncation(L):
    rec = _record()
    assert rvq.record_check(rec, 4, 5, REC_H, REC_I) == RECORD          # another layer's record
    assert rvq.record_check(rec, 3, 6, REC_H, REC_I) == RECORD          # wrongly joined: expert 5 in slot 6
    assert rvq.record_check(rec, 3, 5, 512, REC_I) == RECORD            # another shape
    assert rvq.record_check(rec[:-1], 3, 5, REC_H, REC_I) == RECORD     # truncated by one byte
    assert rvq.record_check(rec[:4096], 3, 5, REC_H, REC_I) == RECORD   # header page only
    assert rvq.record_check(rec[:63], 3, 5, REC_H, REC_I) == RECORD     # not even a header
    assert rvq.record_check(np.zeros_like(rec), 3, 5, REC_H, REC_I) == RECORD
    assert L.rvq_record_check(None, rec.size, 3, 5, REC_H, REC_I) == NULL
    assert rvq.record_check(rec, -1, 5, REC_H, REC_I) == SHAPE
    assert rvq.record_check(rec, 3, 5, REC_H, 12) == SHAPE


def test_record_check_refuses_every_single_bit_flip_of_the_checked_fields(L):
    """At a record with no padding every field the check reads is pinned: flipping any one of the 448
    bits of the first 56 bytes (magic .. codes_bytes) is refused; the CRC and reserved words are not
    checked here."""
    rec = _record()
    for byte in range(64):
        for bit in range(8):
            r = rec.copy()
            r[byte] ^= np.uint8(1 << bit)
            want = RECORD if byte < 56 else OK
            assert rvq.record_check(r, 3, 5, REC_H, REC_I) == want, (byte, bit)


def test_record_check_offset_range_edge_cases(L):
    import struct
    cb = L.rvq_bank_record_bytes(REC_H, REC_I)
    rb = rvq.record_bytes(REC_H, REC_I)

    def with_offsets(cb_off, codes_off, size=rb):
        r = np.zeros(size, dtype=np.uint8)
        r[:64] = np.frombuffer(struct.pack("<IIiiiiqqqqII", 0x45515652, 1, 3, 5, REC_H, REC_I, cb_off, 73728,
                                           codes_off, cb, 0, 0), dtype=np.uint8)
        return rvq.record_check(r, 3, 5, REC_H, REC_I)
    assert with_offsets(4096, 77824) == OK
    assert with_offsets(64, 64 + 73728) == OK                   # packed right after the header
    assert with_offsets(64 + cb, 64) == OK                      # codes first, then codebooks
    assert with_offsets(48, 77824) == RECORD                    # over the header
    assert with_offsets(4096, 77824 - 16) == RECORD             # regions overlap by 16 bytes
    assert with_offsets(4096, rb - cb + 16) == RECORD           # codes run 16 bytes past the end
    assert with_offsets(4096, 2 ** 62) == RECORD                # offset far out (no overflow)
    assert with_offsets(4096, -4096) == RECORD                  # negative offset
    assert with_offsets(2 ** 63 - 16, 77824) == RECORD          # offset + size would overflow
    assert with_offsets(4104, 77824) == RECORD                  # not 16-byte aligned


def test_record_pool_validation(L):
    out = ctypes.c_void_p()
    c = L.rvq_pool_create_records
    rb = rvq.record_bytes(7168, 2048)
    vw = L.rvq_pool_verify_workspace_bytes(7168, 2048)
    assert vw >= 256 + 2 * 256 and vw % 256 == 0
    assert L.rvq_pool_verify_workspace_bytes(7168, 12) == 0
    ok = [FAKE, rb, 0, 32, 7168, 2048, FAKE, FAKE2, 16_515_072, 8, 1, FAKE2 + 0x100000, vw]
    assert c(*ok, None) == NULL
    assert c(None, *ok[1:], ctypes.byref(out)) == NULL
    assert c(*ok[:11], None, vw, ctypes.byref(out)) == NULL                  # verify without a workspace
    assert c(*ok[:1], rb - 4096, *ok[2:], ctypes.byref(out)) == SHAPE        # records shorter than the layout
    assert c(*ok[:1], rb + 256, *ok[2:], ctypes.byref(out)) == ALIGN         # record stride not 4 KiB
    assert c(*ok[:2], -1, *ok[3:], ctypes.byref(out)) == SHAPE               # negative layer
    assert c(*ok[:9], 0, *ok[10:], ctypes.byref(out)) == SHAPE               # no slots
    assert c(*ok[:8], 16_515_072 - 256, *ok[9:], ctypes.byref(out)) == SHAPE  # slot stride below the payload
    assert c(*ok[:8], 16_515_072 + 16, *ok[9:], ctypes.byref(out)) == ALIGN   # slot stride not 256
    assert c(*ok[:11], FAKE2 + 0x100010, vw, ctypes.byref(out)) == ALIGN      # workspace alignment
    assert c(*ok[:12], vw - 1, ctypes.byref(out)) == WS
    assert out.value is None
    bad = ctypes.c_int32()
    assert L.rvq_pool_verify_status(None, ctypes.byref(bad)) == NULL


def test_fit_workspace_and_validation(L):
    ws = L.rvq_fit_workspace_bytes(2048, 7168)
    n = 2048 * 896
    runs = -(-n // 2048)
    assert ws == n * 32 + n + runs * 2048 * 8 + runs * 256 * 4
    assert L.rvq_fit_workspace_bytes(0, 8) == 0 and L.rvq_fit_workspace_bytes(4, 12) == 0
    assert L.rvq_fit_workspace_bytes(2 ** 30, 2 ** 30) == 0                # more sub-vectors than int32 indices
    init = (ctypes.c_int32 * 768)(*([0] * 768))
    f = L.rvq_fit
    ok = [FAKE, 64, 512, 3, init, FAKE2, FAKE, FAKE2 + 0x100000, L.rvq_fit_workspace_bytes(64, 512), None]
    assert f(None, *ok[1:]) == NULL
    assert f(*ok[:4], None, *ok[5:]) == NULL
    assert f(*ok[:7], None, *ok[8:]) == NULL
    assert f(*ok[:3], -1, *ok[4:]) == SHAPE
    assert f(*ok[:3], 10001, *ok[4:]) == SHAPE
    assert f(FAKE, 64, 500, *ok[3:]) == SHAPE
    bad = (ctypes.c_int32 * 768)(*([0] * 767 + [64 * 64]))               # one start past the last sub-vector
    assert f(*ok[:4], bad, *ok[5:]) == SHAPE
    neg = (ctypes.c_int32 * 768)(*([-1] + [0] * 767))
    assert f(*ok[:4], neg, *ok[5:]) == SHAPE
    assert f(*ok[:5], FAKE2 + 4, *ok[6:]) == ALIGN                         # codebooks 16-aligned
    assert f(*ok[:7], FAKE2 + 0x100010, *ok[8:]) == ALIGN                  # workspace 256-aligned
    assert f(*ok[:8], ok[8] - 1, None) == WS
