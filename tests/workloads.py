"""Synthetic workloads shared by the GPU tests and bench.py.

Builds device-resident expert banks and routers from the seeded generators in
`synth` (canonical codes -> upload -> rvq_pack_codes), and the matching
host-side expert descriptions for the oracle (regenerated from the same seeds,
never read back from the device).
"""
import numpy as np
import torch

import synth

# Shapes of the synthetic configurations.
MATVEC_ROWS, MATVEC_COLS = 256, 512
HIDDEN, INTER = 7168, 2048
LAYER_EXPERTS, TOP_K = 256, 16
STACK_LAYERS, STACK_EXPERTS, STACK_STEPS = 92, 64, 32
CHUNK_TOKENS = 512
RMS_EPS = 1e-6


def oracle_expert(seed, layer, e, hidden=HIDDEN, inter=INTER):
    ex = synth.Expert(seed, layer, e, hidden, inter)
    return {"hidden": hidden, "inter": inter,
            "gate": (ex.codes(synth.GATE), ex.codebooks(synth.GATE)),
            "up": (ex.codes(synth.UP), ex.codebooks(synth.UP)),
            "down": (ex.codes(synth.DOWN), ex.codebooks(synth.DOWN))}


def upload_bank(seed, layer, num_experts, hidden=HIDDEN, inter=INTER, device="cuda"):
    import rvq_quantized_moe_amd as rvq
    bank = rvq.ExpertBank(num_experts, hidden, inter, device=device)
    for e in range(num_experts):
        ex = synth.Expert(seed, layer, e, hidden, inter)
        bank.load_expert(e, ex.codes(synth.GATE), ex.codes(synth.UP), ex.codes(synth.DOWN), ex.all_codebooks())
    torch.cuda.synchronize(device)
    return bank


def router(seed, layer, num_experts, hidden=HIDDEN, device="cuda"):
    bits = synth.router_bf16_bits(seed, layer, num_experts, hidden)
    w = torch.from_numpy(bits.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return bits, w


def pack_spec(codes, rows, cols):
    """The packed slab layout of include/rvq.h written out in numpy (layout spec for tests)."""
    G = cols // 8
    nt, nrb = -(-G // 16), -(-rows // 64)
    canon = np.zeros((nrb * 64, nt * 48), dtype=np.uint8)
    canon[:rows, :3 * G] = np.asarray(codes, dtype=np.uint8).reshape(rows, 3 * G)
    # [rb, l, t, j, i] -> [t, rb, j, l, i]
    v = canon.reshape(nrb, 64, nt, 3, 16).transpose(2, 0, 3, 1, 4)
    return np.ascontiguousarray(v).reshape(-1)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


class Stack:
    """92 MoE layers (64 experts each, 7168/2048) with per-layer bf16 routers, resident on the device."""

    def __init__(self, seed=None, layers=None, experts=None, hidden=HIDDEN, inter=INTER, device="cuda"):
        import synth as _s
        self.seed = _s.SEED_STACK if seed is None else seed
        self.L = STACK_LAYERS if layers is None else layers
        self.E = STACK_EXPERTS if experts is None else experts
        self.H, self.I = hidden, inter
        self.banks, self.router_bits, self.routers = [], [], []
        for l in range(self.L):
            self.banks.append(upload_bank(self.seed, l, self.E, hidden, inter, device=device))
            bits, w = router(self.seed, l, self.E, hidden, device=device)
            self.router_bits.append(bits)
            self.routers.append(w)

    def oracle_expert(self, l, e):
        return oracle_expert(self.seed, l, e, self.H, self.I)
