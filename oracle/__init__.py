"""fp64 CPU oracle for the RVQ-LUT MoE expert forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It shares
no code with the GPU library (rvq_quantized_moe_amd) and never imports it.

The arithmetic lives in rvq_oracle.c (plain loops in double precision); this
module marshals numpy arrays and composes the per-layer steps:

  expert(x)      = down( silu(gate x) * (up x) ), every weight rebuilt as the
                   sum of its three stage code vectors
                   ("Running a 2.78-Trillion-Parameter Model on a Laptop: Inside
                   WASTE's NVMe-Streaming Engine", Technical Insight: gate, up and
                   down matrices per expert; RVQ at 3.00 bits per weight)
  route(x)       = top-k of W_r x by (logit desc, id asc), gates = softmax over
                   the k kept logits (news.hada.io topic 32035, read-ahead and
                   router-prediction section: 16 expert ids chosen per layer;
                   the starlog page, "Technical Insight": low-ranked experts
                   still matter, so none is dropped)
  moe_mix(x)     = [residual +] sum_i gate_i * expert_{id_i}(x) for given ids and gates
  moe_layer(x)   = route(x), then moe_mix
  stack step     = for each layer: n = rmsnorm(h); h += moe_layer_l(n)
  rvq_encode(W)  = codes [rows, cols/8, 3] of W by residual (stage-by-stage nearest
                   entry) quantisation, distances and residuals in fp64 (the decode's
                   inverse); optionally each decision's best and second-best distance
  crc32(bytes)   = CRC-32 (IEEE 802.3, reflected, preset and final complement) of a
                   record's code payload, bit by bit (news.hada.io topic 32035,
                   disk-streaming architecture section: optional payload crc32)
  rvq_fit(W)     = codebooks [3, 256, 8] and codes of W by residual k-means: per stage,
                   Lloyd iterations from given initial sub-vectors (nearest entry as in
                   rvq_encode; each mean one fp64 sum over its members in ascending
                   index), then the stage's codes and its residual

Parity status of each function (what pins it) is listed in tests/test_oracle_pins.py.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "librvq_oracle.so")
_SRC = os.path.join(_HERE, "rvq_oracle.c")


def build(force=False):
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                               "-Wall", "-o", _SO, _SRC, "-lm"])


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_dequant.argtypes = [p, p, i64, i64, p]
        lib.orc_gemv.argtypes = [p, p, i64, i64, p, p, i64, p, i32]
        lib.orc_gemv_batch.argtypes = [p, p, i64, i64, p, i64, p, i64, p, i32]
        lib.orc_lut.argtypes = [p, p, i64, p]
        lib.orc_gemv_via_lut.argtypes = [p, p, i64, i64, p]
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_expert_batch.argtypes = [p, p, p, p, p, p, i64, i64, p, i64, p, i64, p, i32]
        lib.orc_router_logits.argtypes = [p, p, i64, i64, i64, p, i32]
        lib.orc_topk.argtypes = [p, i64, i64, p, p, p]
        lib.orc_rmsnorm.argtypes = [p, i64, ctypes.c_double, p]
        lib.orc_rvq_encode.argtypes = [p, i64, i64, p, p, p]
        lib.orc_crc32.argtypes = [p, i64]
        lib.orc_rvq_fit.argtypes = [p, i64, i64, i32, p, p, p, i32]
        lib.orc_rvq_fit.restype = None
        lib.orc_crc32.restype = ctypes.c_uint32
        _lib = lib
    return _lib


def threads():
    """Host threads the oracle uses: every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _codes(codes, rows, cols):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    assert codes.size == rows * (cols // 8) * 3, "codes must hold 3 bytes per 8 weights"
    return codes


# ---------------------------------------------------------------------------------------------

def dequant(codes, codebooks, rows, cols):
    """Dense fp64 W [rows, cols]: W[r, 8g+j] = sum_s C_s[codes[r,g,s]][j]."""
    codes = _codes(codes, rows, cols)
    cb = _c(codebooks, np.float32)
    W = np.empty((rows, cols), dtype=np.float64)
    _load().orc_dequant(codes.ctypes.data, cb.ctypes.data, rows, cols, W.ctypes.data)
    return W


def gemv(codes, codebooks, rows, cols, x, rowsel=None):
    """y = W x in fp64 with W rebuilt weight by weight; only rows `rowsel` if given."""
    return gemv_batch(codes, codebooks, rows, cols, np.asarray(x)[None, :], rowsel)[0]


def gemv_batch(codes, codebooks, rows, cols, X, rowsel=None):
    codes = _codes(codes, rows, cols)
    cb = _c(codebooks, np.float32)
    X = _c(X, np.float64)
    assert X.ndim == 2 and X.shape[1] == cols
    sel = None if rowsel is None else _c(rowsel, np.int64)
    nout = rows if sel is None else sel.size
    Y = np.empty((X.shape[0], nout), dtype=np.float64)
    _load().orc_gemv_batch(codes.ctypes.data, cb.ctypes.data, rows, cols, X.ctypes.data, X.shape[0],
                           None if sel is None else sel.ctypes.data, 0 if sel is None else sel.size,
                           Y.ctypes.data, threads())
    return Y


def lut(codebooks, x):
    """Partial-dot tables T[g, s, c] = C_s[c] . x[8g:8g+8] in fp64, shape [cols/8, 3, 256]."""
    cb = _c(codebooks, np.float32)
    x = _c(x, np.float64)
    assert x.size % 8 == 0
    T = np.empty((x.size // 8, 3, 256), dtype=np.float64)
    _load().orc_lut(cb.ctypes.data, x.ctypes.data, x.size, T.ctypes.data)
    return T


def gemv_via_lut(codes, T, rows, cols):
    """The table form: y[r] = sum_g sum_s T[g, s, codes[r, g, s]] (used only to check the oracle itself)."""
    codes = _codes(codes, rows, cols)
    T = _c(T, np.float64)
    y = np.empty(rows, dtype=np.float64)
    _load().orc_gemv_via_lut(codes.ctypes.data, T.ctypes.data, rows, cols, y.ctypes.data)
    return y


def silu(z):
    return _load().orc_silu(float(z))


def expert_batch(ex, X, rowsel=None):
    """Y[t] = down(silu(gate X[t]) * up X[t]) in fp64.

    `ex` maps 'gate','up','down' -> (codes, codebooks) and has 'hidden', 'inter'."""
    H, I = ex["hidden"], ex["inter"]
    gc, gcb = ex["gate"]
    uc, ucb = ex["up"]
    dc, dcb = ex["down"]
    gc, uc = _codes(gc, I, H), _codes(uc, I, H)
    dc = _codes(dc, H, I)
    gcb, ucb, dcb = (_c(c, np.float32) for c in (gcb, ucb, dcb))
    X = _c(X, np.float64)
    assert X.ndim == 2 and X.shape[1] == H
    sel = None if rowsel is None else _c(rowsel, np.int64)
    nout = H if sel is None else sel.size
    Y = np.empty((X.shape[0], nout), dtype=np.float64)
    _load().orc_expert_batch(gc.ctypes.data, gcb.ctypes.data, uc.ctypes.data, ucb.ctypes.data,
                             dc.ctypes.data, dcb.ctypes.data, H, I, X.ctypes.data, X.shape[0],
                             None if sel is None else sel.ctypes.data, 0 if sel is None else sel.size,
                             Y.ctypes.data, threads())
    return Y


def expert(ex, x, rowsel=None):
    return expert_batch(ex, np.asarray(x)[None, :], rowsel)[0]


def router_logits(w_bf16_bits, X):
    """L[t, e] = sum_k Wr[e, k] X[t, k] in fp64; Wr given as bf16 bit patterns [E, H]."""
    w = _c(w_bf16_bits, np.uint16)
    X = _c(np.atleast_2d(X), np.float64)
    E, H = w.shape
    assert X.shape[1] == H
    L = np.empty((X.shape[0], E), dtype=np.float64)
    _load().orc_router_logits(w.ctypes.data, X.ctypes.data, X.shape[0], E, H, L.ctypes.data, threads())
    return L


def topk(logits, k):
    """(ids int32 [k], gates fp64 [k], (boundary gap, smallest in-set gap))."""
    l = _c(logits, np.float64)
    E = l.size
    assert 1 <= k <= E
    ids = np.empty(k, dtype=np.int32)
    gates = np.empty(k, dtype=np.float64)
    gaps = np.empty(2, dtype=np.float64)
    _load().orc_topk(l.ctypes.data, E, k, ids.ctypes.data, gates.ctypes.data, gaps.ctypes.data)
    return ids, gates, (float(gaps[0]), float(gaps[1]))


def rmsnorm(h, eps=1e-6):
    h = _c(h, np.float64)
    out = np.empty_like(h)
    _load().orc_rmsnorm(h.ctypes.data, h.size, float(eps), out.ctypes.data)
    return out


def moe_mix(get_expert, x, ids, gates, residual=None, rowsel=None):
    """[residual +] sum_i gates[i] * expert_{ids[i]}(x) for given ids and gates, in slot order (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    y = None
    for e, g in zip(np.asarray(ids).reshape(-1), np.asarray(gates, dtype=np.float64).reshape(-1)):
        yi = expert(get_expert(int(e)), x, rowsel)
        y = g * yi if y is None else y + g * yi
    if residual is not None:
        r = np.asarray(residual, dtype=np.float64)
        y = y + (r if rowsel is None else r[np.asarray(rowsel)])
    return y


def moe_layer(get_expert, router_bits, x, k, residual=None, rowsel=None):
    """One decode token through one MoE layer.

    get_expert(e) -> expert dict (see expert_batch).  Returns
    (y fp64 [H or len(rowsel)], ids, gates, gaps)."""
    x = np.asarray(x, dtype=np.float64)
    logits = router_logits(router_bits, x[None, :])[0]
    ids, gates, gaps = topk(logits, k)
    return moe_mix(get_expert, x, ids, gates, residual, rowsel), ids, gates, gaps


def moe_chunk(get_expert, router_bits, X, k, residual=None, tokens=None):
    """A chunk of tokens through one MoE layer: every token routed, then each expert rebuilt once and
    applied to all of its tokens (the token's output is the same as moe_layer's, token by token).

    X: fp64 [T, H] (exact widening of the bf16 chunk).  tokens: indices whose outputs are wanted
    (all if None).  Returns (Y fp64 [len(tokens), H], ids [T, k], gates [T, k])."""
    X = np.asarray(X, dtype=np.float64)
    T, H = X.shape
    L = router_logits(router_bits, X)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        ids[t], gates[t], _ = topk(L[t], k)
    want = np.arange(T) if tokens is None else np.asarray(tokens)
    Y = np.zeros((want.size, H), dtype=np.float64)
    by_expert = {}
    for row, t in enumerate(want):
        for i in range(k):
            by_expert.setdefault(int(ids[t, i]), []).append((row, int(t), i))
    for e in sorted(by_expert):
        pairs = by_expert[e]
        Ye = expert_batch(get_expert(e), X[[t for _, t, _ in pairs]])
        for (row, t, i), y in zip(pairs, Ye):
            Y[row] += gates[t, i] * y
    if residual is not None:
        Y += np.asarray(residual, dtype=np.float64)[want]
    return Y, ids, gates


def crc32(data):
    """CRC-32 of a byte buffer (bytes or a uint8 array)."""
    a = np.ascontiguousarray(np.frombuffer(data, dtype=np.uint8) if isinstance(data, (bytes, bytearray))
                             else np.asarray(data, dtype=np.uint8).reshape(-1))
    return int(_load().orc_crc32(a.ctypes.data, a.size))


def rvq_encode(W, codebooks, margins=False):
    """Residual quantisation of W (fp32 [rows, cols]) against codebooks [3, 256, 8] fp32:
    codes uint8 [rows, cols/8, 3].  With margins=True also returns fp64 [rows, cols/8, 3, 3]:
    per decision (best distance, second-best distance, squared norm of the stage's input)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    cb = np.ascontiguousarray(codebooks, dtype=np.float32)
    rows, cols = W.shape
    codes = np.empty((rows, cols // 8, 3), dtype=np.uint8)
    m = np.empty((rows, cols // 8, 3, 3), dtype=np.float64) if margins else None
    _load().orc_rvq_encode(W.ctypes.data, rows, cols, cb.ctypes.data, codes.ctypes.data,
                           None if m is None else m.ctypes.data)
    return (codes, m) if margins else codes


def rvq_fit(W, iters, init_idx, threads=None):
    """Residual k-means codebooks of W (fp32 [rows, cols]): iters Lloyd iterations per stage from the
    residual sub-vectors init_idx[s] (int [3, 256], row-major sub-vector indices).  Returns
    (codebooks fp32 [3, 256, 8], codes uint8 [rows, cols/8, 3])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    rows, cols = W.shape
    init = np.ascontiguousarray(init_idx, dtype=np.int32).reshape(3, 256)
    n = rows * (cols // 8)
    if init.min() < 0 or init.max() >= n:
        raise ValueError("init_idx out of range")
    cb = np.empty((3, 256, 8), dtype=np.float32)
    codes = np.empty((rows, cols // 8, 3), dtype=np.uint8)
    _load().orc_rvq_fit(W.ctypes.data, rows, cols, int(iters), init.ctypes.data, cb.ctypes.data, codes.ctypes.data,
                        int(threads or min(16, os.cpu_count() or 1)))
    return cb, codes
