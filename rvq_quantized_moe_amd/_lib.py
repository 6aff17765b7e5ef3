"""ctypes binding of librvq.so (include/rvq.h).

Argument marshalling only: PyTorch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if librvq.so is missing, or no GPU is visible, the
calls raise.
"""
import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librvq.so")

F32, F16, BF16 = 0, 1, 2
_DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}

RVQ_OK = 0
RVQ_ERR_WORKSPACE = 5
RVQ_ERR_EXPERT_ID = 6
RVQ_ERR_RECORD = 9


class RvqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("codebooks", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class BankDesc(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("codebooks", ctypes.c_void_p), ("record_stride", ctypes.c_int64),
                ("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32)]


class RecordHeader(ctypes.Structure):
    """The 64-byte header at the start of an expert record (rvq_record_header_t)."""
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("layer", ctypes.c_int32),
                ("expert", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("codebook_offset", ctypes.c_int64), ("codebook_bytes", ctypes.c_int64),
                ("codes_offset", ctypes.c_int64), ("codes_bytes", ctypes.c_int64),
                ("payload_crc32", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None

EXPORTS = [
    "rvq_status_string", "rvq_packed_bytes", "rvq_pack_codes", "rvq_lut_build",
    "rvq_expert_gemv_workspace_bytes", "rvq_expert_gemv", "rvq_router_topk", "rvq_bank_record_bytes",
    "rvq_moe_layer_workspace_bytes", "rvq_moe_layer_forward", "rvq_moe_layer_forward_timed",
    "rvq_workspace_init", "rvq_rmsnorm", "rvq_stream_copy", "rvq_stream_read",
    "rvq_check_device_status", "rvq_moe_decode_routed", "rvq_workspace_set_wait_limit", "rvq_moe_block_decode",
    "rvq_moe_batch_decode", "rvq_moe_batch_decode_workspace_bytes", "rvq_bank_crc32", "rvq_bank_crc32_workspace_bytes",
    "rvq_encode", "rvq_pool_create", "rvq_pool_acquire", "rvq_pool_prefetch", "rvq_pool_stats", "rvq_pool_destroy",
    "rvq_record_bytes", "rvq_record_header_init", "rvq_record_check", "rvq_pool_verify_workspace_bytes",
    "rvq_pool_create_records", "rvq_pool_verify_status", "rvq_fit_workspace_bytes", "rvq_fit",
    "rvq_moe_decode_routed_scratch",
]


def lib():
    """Loads librvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rvq_quantized_moe_amd.build` "
                              "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.rvq_status_string.argtypes = [ctypes.c_int]
        L.rvq_status_string.restype = ctypes.c_char_p
        L.rvq_packed_bytes.argtypes = [i32, i32]
        L.rvq_packed_bytes.restype = sz
        L.rvq_pack_codes.argtypes = [p, i32, i32, p, p]
        L.rvq_lut_build.argtypes = [p, i32, p, i32, p, p, p]
        L.rvq_expert_gemv_workspace_bytes.argtypes = [i32, i32, i32]
        L.rvq_expert_gemv_workspace_bytes.restype = sz
        L.rvq_expert_gemv.argtypes = [ctypes.POINTER(Matrix), p, i32, p, p, sz, p]
        L.rvq_router_topk.argtypes = [p, p, i32, i32, i32, i32, i32, p, p, p, p]
        L.rvq_bank_record_bytes.argtypes = [i32, i32]
        L.rvq_bank_record_bytes.restype = sz
        L.rvq_moe_layer_workspace_bytes.argtypes = [ctypes.POINTER(BankDesc), i32, i32, i32]
        L.rvq_moe_layer_workspace_bytes.restype = sz
        L.rvq_moe_layer_forward.argtypes = [ctypes.POINTER(BankDesc), p, i32, i32, p, p, i32, p, p, i32, p, sz, p]
        L.rvq_moe_layer_forward_timed.argtypes = [ctypes.POINTER(BankDesc), p, i32, i32, p, p, i32, p, p, i32, p,
                                                  sz, p, ctypes.POINTER(ctypes.c_void_p)]
        L.rvq_workspace_init.argtypes = [p, sz, p]
        L.rvq_rmsnorm.argtypes = [p, i32, i32, ctypes.c_float, p, p]
        L.rvq_check_device_status.argtypes = [p, p]
        L.rvq_stream_copy.argtypes = [p, p, sz, p]
        L.rvq_stream_read.argtypes = [p, sz, p, p]
        L.rvq_moe_block_decode.argtypes = [ctypes.POINTER(BankDesc), p, p, i32, ctypes.c_float, p, p, p, p, i32, p,
                                           sz, p]
        L.rvq_workspace_set_wait_limit.argtypes = [p, sz, i32, p]
        L.rvq_moe_batch_decode.argtypes = [ctypes.POINTER(BankDesc), p, i32, p, p, i32, p, p, i32, p, sz, p]
        L.rvq_moe_batch_decode_workspace_bytes.argtypes = [ctypes.POINTER(BankDesc), i32, i32, i32]
        L.rvq_moe_batch_decode_workspace_bytes.restype = sz
        L.rvq_encode.argtypes = [p, i32, i32, p, p, p]
        L.rvq_encode.restype = ctypes.c_int
        L.rvq_fit_workspace_bytes.argtypes = [i32, i32]
        L.rvq_fit_workspace_bytes.restype = sz
        L.rvq_fit.argtypes = [p, i32, i32, i32, p, p, p, p, sz, p]
        L.rvq_fit.restype = ctypes.c_int
        L.rvq_bank_crc32.argtypes = [ctypes.POINTER(BankDesc), p, p, sz, p]
        L.rvq_bank_crc32.restype = ctypes.c_int
        L.rvq_bank_crc32_workspace_bytes.argtypes = [ctypes.POINTER(BankDesc)]
        L.rvq_bank_crc32_workspace_bytes.restype = sz
        i64 = ctypes.c_int64
        L.rvq_pool_create.argtypes = [p, p, i64, i32, i32, i32, p, p, i32, ctypes.POINTER(ctypes.c_void_p)]
        L.rvq_pool_acquire.argtypes = [p, p, i32, p, p]
        L.rvq_pool_prefetch.argtypes = [p, p, i32]
        L.rvq_pool_stats.argtypes = [p, p, p, p, p]
        L.rvq_pool_destroy.argtypes = [p]
        L.rvq_record_bytes.argtypes = [i32, i32]
        L.rvq_record_bytes.restype = sz
        L.rvq_record_header_init.argtypes = [ctypes.POINTER(RecordHeader), i32, i32, i32, i32, ctypes.c_uint32]
        L.rvq_record_check.argtypes = [p, i64, i32, i32, i32, i32]
        L.rvq_pool_verify_workspace_bytes.argtypes = [i32, i32]
        L.rvq_pool_verify_workspace_bytes.restype = sz
        L.rvq_pool_create_records.argtypes = [p, i64, i32, i32, i32, i32, p, p, i64, i32, i32, p, sz,
                                              ctypes.POINTER(ctypes.c_void_p)]
        L.rvq_pool_verify_status.argtypes = [p, ctypes.POINTER(i32)]
        for name in ("rvq_pool_create", "rvq_pool_acquire", "rvq_pool_prefetch", "rvq_pool_stats",
                     "rvq_pool_destroy", "rvq_record_header_init", "rvq_record_check", "rvq_pool_create_records",
                     "rvq_pool_verify_status"):
            getattr(L, name).restype = ctypes.c_int
        L.rvq_moe_decode_routed.argtypes = [ctypes.POINTER(BankDesc), p, p, i32, p, p, p, p, p, i32, p, sz, p]
        L.rvq_moe_decode_routed_scratch.argtypes = [ctypes.POINTER(BankDesc), p, p, i32, p, p, p, p, p, i32, p, p]
        for name in ("rvq_pack_codes", "rvq_lut_build", "rvq_expert_gemv", "rvq_router_topk",
                     "rvq_moe_layer_forward", "rvq_moe_layer_forward_timed", "rvq_workspace_init", "rvq_rmsnorm",
                     "rvq_check_device_status", "rvq_stream_copy", "rvq_moe_decode_routed", "rvq_moe_block_decode",
                     "rvq_moe_batch_decode", "rvq_workspace_set_wait_limit", "rvq_stream_read",
                     "rvq_moe_decode_routed_scratch"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().rvq_status_string(int(status)).decode()


def _check(status):
    if status != RVQ_OK:
        raise RvqError(status, status_string(status))


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _table_dtype(d):
    if d in ("f32", torch.float32, F32):
        return F32
    if d in ("f16", torch.float16, F16):
        return F16
    raise ValueError(f"table dtype must be f32 or f16, got {d!r}")


# ---------------------------------------------------------------------------------------------

def packed_bytes(rows, cols):
    n = lib().rvq_packed_bytes(rows, cols)
    if n == 0:
        raise ValueError(f"invalid matrix shape {rows}x{cols}")
    return n


def pack_codes(codes, rows, cols, out=None):
    """Canonical uint8 codes [rows, cols/8, 3] (device) -> packed slab layout (device uint8)."""
    _dev(codes, torch.uint8, "codes")
    if codes.numel() != rows * (cols // 8) * 3:
        raise ValueError("codes must hold 3 bytes per 8 weights")
    n = packed_bytes(rows, cols)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _dev(out, torch.uint8, "out")
    if out.numel() < n:
        raise ValueError("out too small")
    _check(lib().rvq_pack_codes(_ptr(codes), rows, cols, _ptr(out), _stream(codes)))
    return out


def lut_build(x, codebooks, dtype="f32"):
    """Partial-dot tables [cols/8, 3, 256] (fp32, or fp16 scaled by 2^-e) and e (int32 device scalar)."""
    _dev(x, torch.float32, "x")
    _dev(codebooks, torch.float32, "codebooks")
    d = _table_dtype(dtype)
    cols = x.numel()
    lut = torch.empty((cols // 8, 3, 256), dtype=torch.float32 if d == F32 else torch.float16, device=x.device)
    e = torch.empty(1, dtype=torch.int32, device=x.device)
    _check(lib().rvq_lut_build(_ptr(x), cols, _ptr(codebooks), d, _ptr(lut), _ptr(e), _stream(x)))
    return lut, e


def gemv_workspace_bytes(rows, cols, dtype="f32"):
    return lib().rvq_expert_gemv_workspace_bytes(rows, cols, _table_dtype(dtype))


def expert_gemv(packed, codebooks, rows, cols, x, dtype="f32", y=None, workspace=None):
    """y = W x through the table path for one packed RVQ matrix."""
    _dev(packed, torch.uint8, "packed")
    _dev(codebooks, torch.float32, "codebooks")
    _dev(x, torch.float32, "x")
    d = _table_dtype(dtype)
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=x.device)
    need = gemv_workspace_bytes(rows, cols, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    m = Matrix(packed.data_ptr(), codebooks.data_ptr(), rows, cols)
    _check(lib().rvq_expert_gemv(ctypes.byref(m), _ptr(x), d, _ptr(y), _ptr(workspace), workspace.numel(),
                                 _stream(x)))
    return y


def router_topk(w_router, x, k, ids=None, gates=None, logits=None):
    """Top-k routing: w_router bf16 [E, H]; x fp32 or bf16 [T, H] (or [H]).

    Returns (ids int32 [T, k], gates fp32 [T, k], logits fp64 [T, E])."""
    _dev(w_router, torch.bfloat16, "w_router")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _dev(x, x.dtype, "x")
    E, H = w_router.shape
    x2 = x.reshape(-1, H)
    T = x2.shape[0]
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    gates = torch.empty((T, k), dtype=torch.float32, device=dev) if gates is None else gates
    logits = torch.empty((T, E), dtype=torch.float64, device=dev) if logits is None else logits
    xd = F32 if x.dtype == torch.float32 else BF16
    _check(lib().rvq_router_topk(_ptr(w_router), _ptr(x2), xd, T, E, H, k, _ptr(ids), _ptr(gates), _ptr(logits),
                                 _stream(x)))
    return ids, gates, logits


def rmsnorm(x, eps=1e-6, out=None):
    _dev(x, torch.float32, "x")
    H = x.shape[-1]
    T = x.numel() // H
    out = torch.empty_like(x) if out is None else out
    _check(lib().rvq_rmsnorm(_ptr(x), T, H, float(eps), _ptr(out), _stream(x)))
    return out


def stream_copy(src, dst):
    """dst <- src (uint8 device tensors, 16-byte multiples) with the code stream's load instruction."""
    n = src.numel() * src.element_size()
    _check(lib().rvq_stream_copy(_ptr(src), _ptr(dst), n, _stream(src)))


def stream_read(src, sink):
    """Reads src (a device tensor, 16-byte multiple) with the code stream's load instruction; sink:
    a one-word int32 device tensor that is (in practice never) written."""
    n = src.numel() * src.element_size()
    _check(lib().rvq_stream_read(_ptr(src), n, _ptr(sink), _stream(src)))


def workspace_init(ws):
    _check(lib().rvq_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(ws)))


def set_wait_limit(ws, polls):
    """Polls per bounded wait of the table kernels that use workspace `ws` (< 0: the default)."""
    _check(lib().rvq_workspace_set_wait_limit(_ptr(ws), ws.numel() * ws.element_size(), int(polls), _stream(ws)))


def check_device_status(ws):
    """Synchronises the current stream; returns the sticky device status (0 = OK) and clears it."""
    return lib().rvq_check_device_status(_ptr(ws), _stream(ws))


class ExpertBank:
    """E SwiGLU experts (hidden H, inter I) resident on the device in packed layout.

    codes: uint8 [E * record_stride]; codebooks: fp32 [E, 3, 3, 256, 8] (gate, up, down)."""

    def __init__(self, num_experts, hidden, inter, device="cuda", record_stride=None):
        self.E, self.H, self.I = num_experts, hidden, inter
        rec = lib().rvq_bank_record_bytes(hidden, inter)
        if rec == 0:
            raise ValueError("invalid expert shape")
        self.record_bytes = rec
        self.stride = record_stride or ((rec + 255) // 256) * 256
        self.gate_bytes = packed_bytes(inter, hidden)
        self.down_bytes = packed_bytes(hidden, inter)
        self.codes = torch.empty(num_experts * self.stride, dtype=torch.uint8, device=device)
        self.codebooks = torch.empty((num_experts, 3, 3, 256, 8), dtype=torch.float32, device=device)
        self._staging = None

    def desc(self):
        return BankDesc(self.codes.data_ptr(), self.codebooks.data_ptr(), self.stride, self.E, self.H, self.I)

    def matrix_offset(self, e, m):
        return e * self.stride + m * self.gate_bytes

    def load_expert(self, e, gate_codes, up_codes, down_codes, codebooks):
        """Uploads one expert given canonical numpy codes ([I, H/8, 3], [I, H/8, 3], [H, I/8, 3]) and
        codebooks [3, 3, 256, 8], packing each matrix into record e."""
        dev = self.codes.device
        n = max(gate_codes.size, down_codes.size)
        if self._staging is None or self._staging.numel() < n:
            self._staging = torch.empty(n, dtype=torch.uint8, device=dev)
        for m, (c, rows, cols) in enumerate(((gate_codes, self.I, self.H), (up_codes, self.I, self.H),
                                             (down_codes, self.H, self.I))):
            st = self._staging[:c.size]
            st.copy_(torch.from_numpy(c.reshape(-1)))
            nbytes = packed_bytes(rows, cols)
            off = self.matrix_offset(e, m)
            pack_codes(st, rows, cols, out=self.codes[off:off + nbytes])
        self.codebooks[e].copy_(torch.from_numpy(codebooks))


def _layer_dtype(d, T):
    if T == 1:
        return _table_dtype(d)
    if d in ("f16", F16, torch.float16):
        return F16
    if d in ("bf16", BF16, torch.bfloat16):
        return BF16
    raise ValueError(f"chunk tile dtype must be f16 or bf16, got {d!r}")


def moe_workspace_bytes(bank, T=1, k=16, dtype="f32"):
    d = bank.desc()
    return lib().rvq_moe_layer_workspace_bytes(ctypes.byref(d), T, k, _layer_dtype(dtype, T))


def make_moe_workspace(bank, T=1, k=16, dtype="f32"):
    n = moe_workspace_bytes(bank, T, k, dtype)
    if n == 0:
        raise ValueError("unsupported MoE layer configuration")
    ws = torch.empty(n, dtype=torch.uint8, device=bank.codes.device)
    workspace_init(ws)
    return ws


def moe_layer_forward(bank, x, ids, gates, residual=None, dtype="f32", y=None, workspace=None, events=None):
    """y = [residual +] sum_i gates[i] * expert_{ids[i]}(x).

    One decode token: x fp32 [H], ids/gates [k], dtype = table precision "f32" | "f16".
    A chunk of T > 1 tokens: x bf16 [T, H], ids/gates [T, k], dtype = tile precision "f16" | "bf16";
    returns fp32 [T, H].
    events: optional sequence of 4 raw hipEvent_t handles recorded around the decode kernels."""
    _dev(ids, torch.int32, "ids")
    _dev(gates, torch.float32, "gates")
    if x.dim() == 2 and x.shape[0] > 1:
        _dev(x, torch.bfloat16, "x")
        T = x.shape[0]
        d = {"f16": F16, "bf16": BF16}[dtype]
        k = ids.shape[-1]
        out_shape = (T, bank.H)
        xd = BF16
    else:
        _dev(x, torch.float32, "x")
        T = 1
        d = _table_dtype(dtype)
        k = ids.numel()
        out_shape = (bank.H,)
        xd = F32
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    if y is None:
        y = torch.empty(out_shape, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = make_moe_workspace(bank, T, k, d)
    desc = bank.desc()
    args = (ctypes.byref(desc), _ptr(x), xd, T, _ptr(ids), _ptr(gates), k, _ptr(residual), _ptr(y), d,
            _ptr(workspace), workspace.numel(), _stream(x))
    if events is None:
        _check(lib().rvq_moe_layer_forward(*args))
    else:
        arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(int(e)) for e in events])
        _check(lib().rvq_moe_layer_forward_timed(*args, arr))
    return y


def moe_decode_routed(bank, w_router, x, k, residual=None, dtype="f32", y=None, ids=None, gates=None, logits=None,
                      workspace=None):
    """One routed decode step: router top-k of w_router (bf16 [E, H]) on x (fp32 [H]), then
    y = [residual +] sum_i gates[i] * expert_{ids[i]}(x).  Returns (y, ids, gates, logits)."""
    _dev(w_router, torch.bfloat16, "w_router")
    _dev(x, torch.float32, "x")
    E, H = w_router.shape
    if E != bank.E or H != bank.H:
        raise ValueError("router shape does not match the bank")
    dev = x.device
    d = _table_dtype(dtype)
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    y = torch.empty(H, dtype=torch.float32, device=dev) if y is None else y
    ids = torch.empty(k, dtype=torch.int32, device=dev) if ids is None else ids
    gates = torch.empty(k, dtype=torch.float32, device=dev) if gates is None else gates
    logits = torch.empty(E, dtype=torch.float64, device=dev) if logits is None else logits
    if workspace is None:
        workspace = make_moe_workspace(bank, 1, k, d)
    desc = bank.desc()
    _check(lib().rvq_moe_decode_routed(ctypes.byref(desc), _ptr(w_router), _ptr(x), k, _ptr(residual), _ptr(y),
                                       _ptr(ids), _ptr(gates), _ptr(logits), d, _ptr(workspace), workspace.numel(),
                                       _stream(x)))
    return y, ids, gates, logits


def moe_block_decode(bank, w_router, h, k, eps=1e-6, dtype="f32", h_out=None, ids=None, gates=None, logits=None,
                     workspace=None):
    """One pre-norm residual MoE block: h_out = h + MoE(RMSNorm(h)), routed by w_router (bf16 [E, H]).
    Returns (h_out, ids, gates, logits)."""
    _dev(w_router, torch.bfloat16, "w_router")
    _dev(h, torch.float32, "h")
    E, H = w_router.shape
    if E != bank.E or H != bank.H:
        raise ValueError("router shape does not match the bank")
    dev = h.device
    d = _table_dtype(dtype)
    h_out = torch.empty(H, dtype=torch.float32, device=dev) if h_out is None else h_out
    ids = torch.empty(k, dtype=torch.int32, device=dev) if ids is None else ids
    gates = torch.empty(k, dtype=torch.float32, device=dev) if gates is None else gates
    logits = torch.empty(E, dtype=torch.float64, device=dev) if logits is None else logits
    if workspace is None:
        workspace = make_moe_workspace(bank, 1, k, d)
    desc = bank.desc()
    _check(lib().rvq_moe_block_decode(ctypes.byref(desc), _ptr(w_router), _ptr(h), k, float(eps), _ptr(h_out),
                                      _ptr(ids), _ptr(gates), _ptr(logits), d, _ptr(workspace), workspace.numel(),
                                      _stream(h)))
    return h_out, ids, gates, logits


def make_batch_workspace(bank, T, k=16, dtype="f32"):
    """Zero-filled workspace for moe_batch_decode with T tokens."""
    desc = bank.desc()
    n = lib().rvq_moe_batch_decode_workspace_bytes(ctypes.byref(desc), T, k, _table_dtype(dtype))
    if n == 0:
        raise ValueError("unsupported batch decode configuration")
    ws = torch.empty(n, dtype=torch.uint8, device=bank.codes.device)
    workspace_init(ws)
    return ws


def moe_batch_decode(bank, x, ids, gates, residual=None, dtype="f32", y=None, workspace=None):
    """T decode tokens through the table path: x fp32 [T, H], ids int32 [T, k], gates fp32 [T, k];
    returns y fp32 [T, H] (y[t] as a single-token moe_layer_forward)."""
    _dev(x, torch.float32, "x")
    _dev(ids, torch.int32, "ids")
    _dev(gates, torch.float32, "gates")
    T, H = x.shape
    k = ids.shape[1]
    if H != bank.H or tuple(ids.shape) != (T, k) or tuple(gates.shape) != (T, k):
        raise ValueError("shape mismatch")
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    d = _table_dtype(dtype)
    y = torch.empty(T, H, dtype=torch.float32, device=x.device) if y is None else y
    if workspace is None:
        workspace = make_batch_workspace(bank, T, k, dtype)
    desc = bank.desc()
    _check(lib().rvq_moe_batch_decode(ctypes.byref(desc), _ptr(x), T, _ptr(ids), _ptr(gates), k,
                                      _ptr(residual) if residual is not None else None, _ptr(y), d, _ptr(workspace),
                                      workspace.numel(), _stream(x)))
    return y


def bank_crc32(bank, crc=None, workspace=None):
    """CRC-32 of every expert record's code payload: int32 tensor [E] holding the uint32 bit patterns
    (view as unsigned on the host: .cpu().numpy().view(np.uint32))."""
    desc = bank.desc()
    dev = bank.codes.device
    crc = torch.empty(bank.E, dtype=torch.int32, device=dev) if crc is None else crc
    if workspace is None:
        n = lib().rvq_bank_crc32_workspace_bytes(ctypes.byref(desc))
        if n == 0:
            raise ValueError("invalid bank")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(lib().rvq_bank_crc32(ctypes.byref(desc), _ptr(crc), _ptr(workspace), workspace.numel(),
                                _stream(bank.codes)))
    return crc


class ExpertPool:
    """Experts in pinned host memory with an LRU set of `slots` device records as the cache.

    host_codes: pinned uint8 tensor of num_experts * record_stride bytes (packed records, e.g. a
    copy of an ExpertBank's codes); host_codebooks: pinned fp32 [num_experts, 3, 3, 256, 8].
    self.bank is the device bank of the slots: pass it, with the slot ids from acquire(), to the
    decode functions."""

    def __init__(self, host_codes, host_codebooks, num_experts, hidden, inter, slots, device="cuda",
                 record_stride=None):
        if not host_codes.is_pinned() or not host_codebooks.is_pinned():
            raise ValueError("host_codes and host_codebooks must be pinned host tensors")
        self.bank = ExpertBank(slots, hidden, inter, device=device, record_stride=record_stride)
        self.host_codes, self.host_codebooks = host_codes, host_codebooks
        self.E, self.slots = num_experts, slots
        if host_codes.numel() < num_experts * self.bank.stride or host_codebooks.numel() < num_experts * 3 * 6144:
            raise ValueError("host store too small")
        handle = ctypes.c_void_p()
        _check(lib().rvq_pool_create(_ptr(host_codes), _ptr(host_codebooks), self.bank.stride, num_experts, hidden,
                                     inter, _ptr(self.bank.codes), _ptr(self.bank.codebooks), slots,
                                     ctypes.byref(handle)))
        self._h = handle

    @classmethod
    def from_records(cls, records, layer, num_experts, hidden, inter, slots, device="cuda", verify=False,
                     record_bytes_=None):
        """Pool over a pinned store of expert records (write_records layout); every copy checks its record's
        header first; verify also checks each copied payload's CRC-32 on the device (see verify_status)."""
        if not records.is_pinned():
            raise ValueError("records must be a pinned host tensor")
        rb = record_bytes_ or record_bytes(hidden, inter)
        if records.numel() < num_experts * rb:
            raise ValueError("record store too small")
        self = cls.__new__(cls)
        self.bank = ExpertBank(slots, hidden, inter, device=device)
        self.host_codes, self.host_codebooks = records, None
        self.E, self.slots = num_experts, slots
        self.verify_ws = None
        if verify:
            n = lib().rvq_pool_verify_workspace_bytes(hidden, inter)
            self.verify_ws = torch.empty(n, dtype=torch.uint8, device=device)
        handle = ctypes.c_void_p()
        _check(lib().rvq_pool_create_records(_ptr(records), rb, layer, num_experts, hidden, inter,
                                             _ptr(self.bank.codes), _ptr(self.bank.codebooks), self.bank.stride, slots,
                                             int(bool(verify)), _ptr(self.verify_ws),
                                             0 if self.verify_ws is None else self.verify_ws.numel(),
                                             ctypes.byref(handle)))
        self._h = handle
        return self

    def verify_status(self):
        """Waits for the pool's copies; -1 if every verified payload matched its header's CRC-32, else the id
        of an expert whose payload did not (the record is then cleared)."""
        bad = ctypes.c_int32(-1)
        st = lib().rvq_pool_verify_status(self._h, ctypes.byref(bad))
        if st not in (RVQ_OK, RVQ_ERR_RECORD):
            _check(st)
        return bad.value

    def acquire(self, ids):
        """ids: host int sequence [k] -> host int32 slot ids [k]; the current stream waits for copies."""
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
        out = np.empty(a.size, dtype=np.int32)
        _check(lib().rvq_pool_acquire(self._h, a.ctypes.data, a.size, out.ctypes.data, _stream(self.bank.codes)))
        return out

    def prefetch(self, ids):
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        _check(lib().rvq_pool_prefetch(self._h, a.ctypes.data, a.size))

    def stats(self):
        v = [ctypes.c_int64() for _ in range(4)]
        _check(lib().rvq_pool_stats(self._h, *[ctypes.byref(x) for x in v]))
        return {"hits": v[0].value, "misses": v[1].value, "prefetches": v[2].value, "bytes_copied": v[3].value}

    def close(self):
        if self._h:
            _check(lib().rvq_pool_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def record_bytes(hidden, inter):
    return lib().rvq_record_bytes(hidden, inter)


def record_header(layer, expert, hidden, inter, payload_crc32):
    """The 64 header bytes of an expert record in the standard layout."""
    h = RecordHeader()
    _check(lib().rvq_record_header_init(ctypes.byref(h), layer, expert, hidden, inter, payload_crc32))
    return bytes(h)


def record_check(record, layer, expert, hidden, inter):
    """Status of the read-time header check of one record (host uint8 numpy array or CPU tensor)."""
    if isinstance(record, torch.Tensor):
        if record.device.type != "cpu" or record.dtype != torch.uint8 or not record.is_contiguous():
            raise ValueError("record must be a contiguous CPU uint8 tensor")
        return lib().rvq_record_check(record.data_ptr(), record.numel(), layer, expert, hidden, inter)
    a = np.ascontiguousarray(record, dtype=np.uint8)
    return lib().rvq_record_check(a.ctypes.data, a.size, layer, expert, hidden, inter)


def write_records(bank, layer, crcs, out=None):
    """Expert records of every expert of a device ExpertBank (standard layout) in one pinned uint8 tensor
    of E * record_bytes bytes; crcs: the payload CRC-32 of each expert's codes (e.g. from bank_crc32)."""
    rb = record_bytes(bank.H, bank.I)
    out = torch.zeros(bank.E * rb, dtype=torch.uint8, pin_memory=True) if out is None else out
    codes = bank.codes.view(bank.E, bank.stride)[:, :bank.record_bytes].cpu()
    cbs = bank.codebooks.reshape(bank.E, -1).cpu().view(torch.uint8)
    for e in range(bank.E):
        rec = out[e * rb:(e + 1) * rb]
        hdr = RecordHeader.from_buffer_copy(record_header(layer, e, bank.H, bank.I, int(crcs[e])))
        rec[:64] = torch.frombuffer(bytearray(bytes(hdr)), dtype=torch.uint8)
        rec[hdr.codebook_offset:hdr.codebook_offset + hdr.codebook_bytes] = cbs[e]
        rec[hdr.codes_offset:hdr.codes_offset + hdr.codes_bytes] = codes[e]
    return out


def rvq_encode(W, codebooks, codes=None):
    """Residual RVQ codes of W (fp32 [rows, cols]) against codebooks fp32 [3, 256, 8]:
    uint8 [rows, cols/8, 3] (canonical layout)."""
    _dev(W, torch.float32, "W")
    _dev(codebooks, torch.float32, "codebooks")
    rows, cols = W.shape
    codes = torch.empty((rows, cols // 8, 3), dtype=torch.uint8, device=W.device) if codes is None else codes
    _check(lib().rvq_encode(_ptr(W), rows, cols, _ptr(codebooks), _ptr(codes), _stream(W)))
    return codes


def rvq_fit(W, iters, init_idx, codebooks=None, codes=None, workspace=None):
    """Residual k-means codebooks of W (fp32 [rows, cols], device): iters Lloyd iterations per stage from
    the residual sub-vectors init_idx (host int [3, 256]).  Returns (codebooks fp32 [3, 256, 8],
    codes uint8 [rows, cols/8, 3]); the codes equal rvq_encode(W, codebooks)."""
    _dev(W, torch.float32, "W")
    rows, cols = W.shape
    dev = W.device
    init = np.ascontiguousarray(np.asarray(init_idx, dtype=np.int32).reshape(3, 256))
    codebooks = torch.empty((3, 256, 8), dtype=torch.float32, device=dev) if codebooks is None else codebooks
    codes = torch.empty((rows, cols // 8, 3), dtype=torch.uint8, device=dev) if codes is None else codes
    if workspace is None:
        n = lib().rvq_fit_workspace_bytes(rows, cols)
        if n == 0:
            raise ValueError("invalid shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(lib().rvq_fit(_ptr(W), rows, cols, int(iters), init.ctypes.data, _ptr(codebooks), _ptr(codes),
                         _ptr(workspace), workspace.numel(), _stream(W)))
    return codebooks, codes
