"""Seeded synthetic inputs for the RVQ-LUT MoE expert path.

Holds random-number generation only (no part of the method's arithmetic):
SplitMix64 in counter mode (see synth.c for the exact definition), uniform
code bytes, Box-Muller normals rounded to fp32, and bf16 by round-to-nearest-
even from those fp32 values.  Both the GPU path's tests/benchmarks and the
fp64 oracle draw their inputs from here, so they see the same bytes.

Tensor ids pack (kind, layer, expert-or-token, matrix, sub-index) into 64 bits
so that every tensor of every configuration has its own stream and any slice
of it can be regenerated on its own.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

# Distinct streams per configuration (one seed per synthetic workload).
SEED_MATVEC = 0x52565101      # single 256x512 RVQ matvec
SEED_EXPERT = 0x52565102      # one SwiGLU expert 7168/2048
SEED_LAYER = 0x52565103       # one MoE layer, 256 experts, top-16 (decode and chunk)
SEED_CHUNK = 0x52565104       # the 512-token bf16 chunk fed to that layer
SEED_STACK = 0x52565105       # 92-layer stack, 64 experts per layer

KIND_CODES, KIND_CODEBOOK, KIND_ACT_F32, KIND_ROUTER, KIND_ACT_BF16 = 1, 2, 3, 4, 5
GATE, UP, DOWN, SINGLE = 0, 1, 2, 3

# Standard deviation of codebook stage s entries: 0.5**s (stage 0 coarse, then finer residual stages).
STAGE_STD = (1.0, 0.5, 0.25)
ROUTER_STD = 0.02


def build(force=False):
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                               "-o", _SO, src, "-lm"])


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_words.argtypes = [u64, u64, u64, u64, p]
        lib.synth_bytes.argtypes = [u64, u64, u64, u64, p, ctypes.c_int]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, ctypes.c_double, p]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ctypes.c_double, p]
        _lib = lib
    return _lib


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def tensor_id(kind, layer=0, index=0, matrix=0, sub=0):
    assert 0 <= layer < (1 << 16) and 0 <= index < (1 << 20) and 0 <= matrix < (1 << 12) and 0 <= sub < 256
    return (kind << 56) | (layer << 40) | (index << 20) | (matrix << 8) | sub


def words(seed, tid, first, n):
    out = np.empty(n, dtype=np.uint64)
    _load().synth_words(seed, tid, first, n, out.ctypes.data)
    return out


def uniform_bytes(seed, tid, n, first=0, out=None):
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == n
    _load().synth_bytes(seed, tid, first, n, out.ctypes.data, _threads())
    return out


def normal_f32(seed, tid, n, std=1.0, first=0):
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, tid, first, n, float(std), out.ctypes.data)
    return out


def normal_bf16_bits(seed, tid, n, std=1.0, first=0):
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tid, first, n, float(std), out.ctypes.data)
    return out


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- tensors of the synthetic workloads ------------------------------------------------------

def matrix_codes(seed, layer, expert, matrix, rows, cols, out=None):
    """Uniform uint8 code triples, shape [rows, cols/8, 3] (stage-minor)."""
    assert cols % 8 == 0
    n = rows * (cols // 8) * 3
    flat = uniform_bytes(seed, tensor_id(KIND_CODES, layer, expert, matrix), n,
                         out=None if out is None else out.reshape(-1))
    return flat.reshape(rows, cols // 8, 3)


def matrix_codebooks(seed, layer, expert, matrix):
    """fp32 codebooks [3 stages, 256 entries, 8 dims]; stage s entries ~ N(0, 0.5**s)."""
    cb = np.empty((3, 256, 8), dtype=np.float32)
    for s in range(3):
        cb[s] = normal_f32(seed, tensor_id(KIND_CODEBOOK, layer, expert, matrix, s), 256 * 8,
                           STAGE_STD[s]).reshape(256, 8)
    return cb


def activation_f32(seed, index, n, layer=0):
    return normal_f32(seed, tensor_id(KIND_ACT_F32, layer, index), n, 1.0)


def activation_bf16_bits(seed, index, n, layer=0):
    return normal_bf16_bits(seed, tensor_id(KIND_ACT_BF16, layer, index), n, 1.0)


def router_bf16_bits(seed, layer, num_experts, hidden):
    return normal_bf16_bits(seed, tensor_id(KIND_ROUTER, layer), num_experts * hidden,
                            ROUTER_STD).reshape(num_experts, hidden)


class Expert:
    """One SwiGLU expert's RVQ matrices: gate/up [inter x hidden], down [hidden x inter]."""

    def __init__(self, seed, layer, expert, hidden, inter):
        self.seed, self.layer, self.expert, self.hidden, self.inter = seed, layer, expert, hidden, inter

    def codes(self, matrix, out=None):
        rows, cols = (self.inter, self.hidden) if matrix in (GATE, UP) else (self.hidden, self.inter)
        return matrix_codes(self.seed, self.layer, self.expert, matrix, rows, cols, out=out)

    def codebooks(self, matrix):
        return matrix_codebooks(self.seed, self.layer, self.expert, matrix)

    def record_bytes(self):
        """The expert's three code arrays back to back (gate, up, down): 3 bytes per 8 weights."""
        n = 3 * self.hidden * self.inter * 3 // 8
        rec = np.empty(n, dtype=np.uint8)
        part = n // 3
        for m in (GATE, UP, DOWN):
            self.codes(m, out=rec[m * part:(m + 1) * part])
        return rec

    def all_codebooks(self):
        return np.stack([self.codebooks(m) for m in (GATE, UP, DOWN)])
