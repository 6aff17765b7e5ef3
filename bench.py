"""Benchmark: one MoE layer, batch-1 decode, top-16 of 256 RVQ experts (7168/2048 SwiGLU), on one MI355X.

A step is one decode token through the whole path: router logits (fp64 accumulate) + top-16 +
renormalised softmax, then the table-path gate/up kernel, the SwiGLU + down kernel and the gated
combine, on a token drawn from a pool of 64 seeded tokens (so routing changes every step and the
256 MB last-level cache cannot hold the experts a step touches).  All 256 experts (4.23 GB of
3-bit codes) are resident in HBM before timing starts.

Prints ONE JSON line.  Roofline: the dominant kernel (gate/up, two thirds of the code bytes) is
timed with HIP events recorded around it on its own stream inside the timed region; its
algorithmic bytes per launch are the code bytes of 16 experts' gate and up matrices plus their
codebooks.  cpu_baseline: the fp64 oracle on a bounded sample of the same workload.

Also reported, not the headline: the 512-token chunked prefill (decode-to-MFMA path), one 256x512
matvec, one SwiGLU expert per token, and the 92-layer x 64-expert stack decode (97 GB resident).
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "MoE-layer decode tokens/s + code-byte HBM GB/s (% of peak), batch 1, top-16"
HBM_PEAK_GBPS = 8000.0
E, H, I, K = 256, 7168, 2048, 16
POOL = 64
STEPS_PER_GRAPH = 8        # decode steps captured in one HIP graph
CODE_BYTES_PER_TOKEN = K * 3 * (H * I * 3 // 8)          # 264,241,152
WEIGHTS_PER_TOKEN = K * 3 * H * I                         # 704,643,072
GATEUP_CODE_BYTES = K * 2 * (H * I * 3 // 8)              # 176,160,768 per gate/up launch
GATEUP_CODEBOOK_BYTES = K * 2 * 3 * 256 * 8 * 4           # 786,432
DOWN_CODE_BYTES = K * (H * I * 3 // 8)
# chip-wide lookups/s of the LDS gather the skewed table layout allows (32 distinct banks per pass),
# measured with 32-bit reads and the kernel's per-lookup code; the fp16 tables use the same layout
# and addresses with 16-bit reads, which take the same passes (this figure is assumed for them)
LDS_GATHER_RATE = {"f32": 11.2e12, "f16": 11.2e12}
KERNEL_SOURCES = ["rvq_quantized_moe_amd/csrc/kernels.hip", "rvq_quantized_moe_amd/csrc/device.hpp"]   # decode kernels


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Hip:
    """Raw HIP event API from the runtime already loaded by torch (events are handed to librvq)."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            m = re.search(r"(\S*libamdhip64\.so\S*)", line)
            if m:
                path = m.group(1)
                break
        self.L = ctypes.CDLL(path or "libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def traffic_from_profiles(dtype):
    """HBM bytes per gate/up launch from the committed rocprofv3 --pmc summary, if it was taken on
    the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"moe_gateup_{dtype}_layer256_top16_pmc.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_variant(rvq, hip, bank, w, pool, steps, warmup, dtype):
    import torch
    dev = pool.device
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    ids = torch.empty((1, K), dtype=torch.int32, device=dev)
    gates = torch.empty((1, K), dtype=torch.float32, device=dev)
    logits = torch.empty((1, E), dtype=torch.float64, device=dev)
    y = torch.empty(H, dtype=torch.float32, device=dev)
    ws = rvq.make_moe_workspace(bank, 1, K, dtype)
    L = rvq.lib()
    d = rvq._lib._table_dtype(dtype)
    desc = bank.desc()
    # arguments marshalled once; each step passes the next pool token
    xptrs = [ctypes.c_void_p(pool[i].data_ptr()) for i in range(POOL)]
    router_args = lambda xp: (ctypes.c_void_p(w.data_ptr()), xp, rvq.F32, 1, E, H, K, ctypes.c_void_p(ids.data_ptr()),
                              ctypes.c_void_p(gates.data_ptr()), ctypes.c_void_p(logits.data_ptr()), sptr)
    rargs = [router_args(xp) for xp in xptrs]
    margs = [(ctypes.byref(desc), xp, rvq.F32, 1, ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(gates.data_ptr()),
              K, None, ctypes.c_void_p(y.data_ptr()), d, ctypes.c_void_p(ws.data_ptr()), ws.numel(), sptr)
             for xp in xptrs]
    n_ev = steps
    evs = [[hip.event() for _ in range(5)] for _ in range(n_ev)]
    ev_arrays = [(ctypes.c_void_p * 4)(*ev[1:5]) for ev in evs]

    def step(i, timed):
        j = i % POOL
        if timed:
            hip.record(evs[i][0], sptr)
        st = L.rvq_router_topk(*rargs[j])
        if st:
            raise RuntimeError(rvq.status_string(st))
        if timed:
            st = L.rvq_moe_layer_forward_timed(*margs[j], ev_arrays[i])
        else:
            st = L.rvq_moe_layer_forward(*margs[j])
        if st:
            raise RuntimeError(rvq.status_string(st))

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    router_ms = np.array([hip.ms(ev[0], ev[1]) for ev in evs])
    gateup_ms = np.array([hip.ms(ev[1], ev[2]) for ev in evs])
    down_ms = np.array([hip.ms(ev[2], ev[3]) for ev in evs])
    comb_ms = np.array([hip.ms(ev[3], ev[4]) for ev in evs])
    for ev in evs:
        for e in ev:
            hip.destroy(e)
    elapsed = t1 - t0
    tok_s = steps / elapsed
    gu_s = float(np.mean(gateup_ms)) * 1e-3
    return {
        "tokens_per_s": tok_s,
        "ms_per_step": elapsed / steps * 1e3,
        "code_GBps": CODE_BYTES_PER_TOKEN * tok_s / 1e9,
        "code_frac_of_hbm_peak": CODE_BYTES_PER_TOKEN * tok_s / 1e9 / HBM_PEAK_GBPS,
        "decoded_weights_per_s": WEIGHTS_PER_TOKEN * tok_s,
        "kernel_us": {"router_topk": float(np.mean(router_ms)) * 1e3, "gateup": float(np.mean(gateup_ms)) * 1e3,
                      "swiglu_down": float(np.mean(down_ms)) * 1e3, "combine": float(np.mean(comb_ms)) * 1e3,
                      "gateup_p10": float(np.percentile(gateup_ms, 10)) * 1e3,
                      "gateup_p90": float(np.percentile(gateup_ms, 90)) * 1e3},
        "gateup_GBps": (GATEUP_CODE_BYTES + GATEUP_CODEBOOK_BYTES) / gu_s / 1e9,
        "down_GBps": DOWN_CODE_BYTES / (float(np.mean(down_ms)) * 1e-3) / 1e9,
    }


MIN_TIMED_S = 0.1          # a timed region shorter than this is extended (and the line says so)


def timed_replays(torch, graphs, steps_per_replay, steps, warmup_replays, before=None):
    """Replays `graphs` round-robin, back to back, for at least `steps` decode steps and at least
    MIN_TIMED_S of wall clock (a first pass of the requested length calibrates the count).  One event is
    recorded between consecutive replays inside the timed loop, so the per-replay intervals and the
    wall clock come from the same replays.  Returns (steps timed, seconds, per-step µs intervals)."""
    for i in range(warmup_replays):
        if before:
            before(i)
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()

    def timed(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(n):
            if before:
                before(i)
            graphs[i % len(graphs)].replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        return sec, [evs[i].elapsed_time(evs[i + 1]) * 1e3 / steps_per_replay for i in range(n)]

    n = max(1, -(-steps // steps_per_replay))
    sec, us = timed(n)
    if sec < MIN_TIMED_S:
        n = max(n, int(np.ceil(n * MIN_TIMED_S / max(sec, 1e-6) * 1.05)))
        sec, us = timed(n)
    return n * steps_per_replay, sec, us


def run_graphed(rvq, bank, w, pool, steps, warmup, dtype, routed=True, stats=None, per_graph=1):
    """The step replayed from HIP graphs, which removes host launch overhead; returns (tokens/s, steps
    timed).  Each graph holds per_graph consecutive steps (pool tokens j*per_graph ..), one after
    another on one stream, as the layers of a token follow one another inside one graph in a full
    model; per_graph = 1 adds one graph launch (about 10 µs of idle GPU) to every step.  routed: one
    rvq_moe_decode_routed call per step (router, top-k inside the gate/up kernel, experts); else
    rvq_router_topk + rvq_moe_layer_forward.  stats (dict): filled with p10/p50/p90 of the per-step
    time (µs: each replay's event interval / per_graph) from the same timed replays."""
    import torch
    dev = pool.device
    ids = torch.empty((1, K), dtype=torch.int32, device=dev)
    gates = torch.empty((1, K), dtype=torch.float32, device=dev)
    logits = torch.empty((1, E), dtype=torch.float64, device=dev)
    y = torch.empty(H, dtype=torch.float32, device=dev)
    ws = rvq.make_moe_workspace(bank, 1, K, dtype)
    torch.cuda.synchronize()
    assert POOL % per_graph == 0
    graphs = []
    side = torch.cuda.Stream()
    for j0 in range(0, POOL, per_graph):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for j in range(j0, j0 + per_graph):
                if routed:
                    rvq.moe_decode_routed(bank, w, pool[j], K, dtype=dtype, y=y, ids=ids[0], gates=gates[0],
                                          logits=logits[0], workspace=ws)
                else:
                    rvq.router_topk(w, pool[j], K, ids=ids, gates=gates, logits=logits)
                    rvq.moe_layer_forward(bank, pool[j], ids[0], gates[0], dtype=dtype, y=y, workspace=ws)
        graphs.append(g)
    n, sec, us = timed_replays(torch, graphs, per_graph, steps, max(1, -(-warmup // per_graph)))
    if stats is not None:
        stats.update(percentiles(us))
        stats["mean"] = float(np.mean(us))
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    del graphs
    return n / sec, n


def run_chunk(rvq, hip, bank, w, xt, steps, dtype):
    """Chunked prefill of the 512-token bf16 chunk through the same layer: router top-16 for all tokens,
    then the decode-to-MFMA path.  Returns tokens/s and the mean event time of the MoE part."""
    import torch
    dev = xt.device
    T = xt.shape[0]
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    gates = torch.empty((T, K), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float64, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = rvq.make_moe_workspace(bank, T, K, dtype)
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = [[hip.event() for _ in range(3)] for _ in range(steps)]

    def step(i):
        hip.record(evs[i][0], sptr)
        rvq.router_topk(w, xt, K, ids=ids, gates=gates, logits=logits)
        hip.record(evs[i][1], sptr)
        rvq.moe_layer_forward(bank, xt, ids, gates, dtype=dtype, y=y, workspace=ws)
        hip.record(evs[i][2], sptr)

    step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    router_ms = float(np.mean([hip.ms(e[0], e[1]) for e in evs]))
    moe_ms = float(np.mean([hip.ms(e[1], e[2]) for e in evs]))
    for ev in evs:
        for e in ev:
            hip.destroy(e)
    tok_s = T * steps / (t1 - t0)
    flops = 2.0 * T * K * 3 * H * I
    return {"tokens_per_s": tok_s, "ms_per_chunk": (t1 - t0) / steps * 1e3, "router_ms": router_ms,
            "moe_ms": moe_ms, "code_GBps": E * 3 * (H * I * 3 // 8) / (moe_ms * 1e-3) / 1e9,
            "mfma_TFLOPs": flops / (moe_ms * 1e-3) / 1e12, "tile_dtype": dtype}


def run_small_batch(torch, rvq, bank, w, xt, sizes=(1, 2, 4, 8, 16, 32, 64), reps=10):
    """Small-batch decode: the first T tokens of the bf16 chunk through the table path
    (rvq_moe_batch_decode, every token streaming its own experts' codes) and through the chunk path
    (rvq_moe_layer_forward, T > 1: every touched expert decoded once); tokens/s of the MoE part
    (routing computed beforehand), eager calls timed between synchronisations."""
    dev = xt.device
    res = {"T": list(sizes), "lut_f32_tokens_per_s": [], "lut_f16_tokens_per_s": [], "chunk_f16_tokens_per_s": [],
           "distinct_experts": []}

    def rate(fn, T):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return T * reps / (time.perf_counter() - t0)

    for T in sizes:
        xb = xt[:T].contiguous()
        x32 = xb.float()
        ids, gates, _ = rvq.router_topk(w, xb, K)
        res["distinct_experts"].append(int(torch.unique(ids).numel()))
        y = torch.empty(T, H, dtype=torch.float32, device=dev)
        for d in ("f32", "f16"):
            ws = rvq.make_batch_workspace(bank, T, K, d)
            res[f"lut_{d}_tokens_per_s"].append(
                rate(lambda: rvq.moe_batch_decode(bank, x32, ids, gates, dtype=d, y=y, workspace=ws), T))
            status = rvq.check_device_status(ws)
            if status:
                raise RuntimeError(rvq.status_string(status))
            del ws
        if T > 1:
            ws = rvq.make_moe_workspace(bank, T, K, "f16")
            res["chunk_f16_tokens_per_s"].append(
                rate(lambda: rvq.moe_layer_forward(bank, xb, ids, gates, dtype="f16", y=y, workspace=ws), T))
            del ws
        else:
            res["chunk_f16_tokens_per_s"].append(None)
    # one expert per token, 256 tokens: the table path's batched form with the most pairs per expert
    # slot count and down's row split chosen from all pairs
    xb = xt[:256].contiguous()
    ids1, gates1, _ = rvq.router_topk(w, xb, 1)
    y1 = torch.empty(256, H, dtype=torch.float32, device=dev)
    ws = rvq.make_batch_workspace(bank, 256, 1, "f32")
    res["k1_T256_lut_f32_tokens_per_s"] = rate(
        lambda: rvq.moe_batch_decode(bank, xb.float(), ids1, gates1, dtype="f32", y=y1, workspace=ws), 256)
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    del ws
    best_lut = [max(a, b) for a, b in zip(res["lut_f32_tokens_per_s"], res["lut_f16_tokens_per_s"])]
    cross = [T for T, c, l in zip(sizes, res["chunk_f16_tokens_per_s"], best_lut) if c is not None and c > l]
    res["chunk_faster_from_T"] = cross[0] if cross else None
    return res


def replay_rate(torch, graphs, steps, warmup, before=None):
    """Replays graphs round-robin (before(i) runs eagerly ahead of replay i); returns seconds per replay."""
    for i in range(warmup):
        if before:
            before(i)
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if before:
            before(i)
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def percentiles(us):
    return {"p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
            "p90": float(np.percentile(us, 90))}


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        fn()
    return g


def run_crc(torch, rvq, bank, reps=10):
    """Integrity check of the resident layer bank: CRC-32 of all 256 records' code payloads
    (4,227,858,432 bytes) per call; GB/s against the HBM peak."""
    ws = torch.empty(rvq.lib().rvq_bank_crc32_workspace_bytes(ctypes.byref(bank.desc())), dtype=torch.uint8,
                     device=bank.codes.device)
    crc = torch.empty(bank.E, dtype=torch.int32, device=bank.codes.device)
    rvq.bank_crc32(bank, crc=crc, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rvq.bank_crc32(bank, crc=crc, workspace=ws)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    nbytes = bank.E * (2 * bank.gate_bytes + bank.down_bytes)
    return {"ms_per_bank": sec * 1e3, "GBps": nbytes / sec / 1e9, "frac_of_hbm_peak": nbytes / sec / 1e9 / HBM_PEAK_GBPS,
            "bytes": nbytes}


def run_pool(torch, rvq, bank, w, pool_x, slots_list=(32, 128), tokens=128):
    """Layer decode with the 256 experts in pinned host memory and `slots` device records as the
    LRU cache (rvq expert pool): per token, router top-16 on the device, ids to the host, acquire
    (copies of the missing experts), decode on the slots.  Tokens/s, hit rate and the host-to-device
    copy rate over the run (copies and decode overlap only through the streams).  The same at the
    largest slot count over a store of expert records (each record's header checked on every read),
    and with the payload CRC-32 of every copied expert checked on the device as well."""
    dev = bank.codes.device
    hc = torch.empty(bank.codes.numel(), dtype=torch.uint8, pin_memory=True)
    hc.copy_(bank.codes)
    hb = torch.empty(bank.codebooks.shape, dtype=torch.float32, pin_memory=True)
    hb.copy_(bank.codebooks)
    crcs = rvq.bank_crc32(bank).cpu().numpy().view(np.uint32)
    rec = rvq.write_records(bank, 0, crcs)
    big = max(slots_list)
    variants = [(f"slots_{s}", lambda s=s: rvq.ExpertPool(hc, hb, bank.E, bank.H, bank.I, s, device=dev))
                for s in slots_list]
    variants += [(f"records{'_crc_verify' if v else ''}_slots_{big}",
                  lambda v=v: rvq.ExpertPool.from_records(rec, 0, bank.E, bank.H, bank.I, big, device=dev, verify=v))
                 for v in (False, True)]
    out = {}
    for name, make in variants:
        pool = make()
        ws = rvq.make_moe_workspace(pool.bank, 1, K, "f32")
        y = torch.empty(H, dtype=torch.float32, device=dev)
        ids = torch.empty((1, K), dtype=torch.int32, device=dev)
        gates = torch.empty((1, K), dtype=torch.float32, device=dev)
        logits = torch.empty((1, E), dtype=torch.float64, device=dev)
        sd = torch.empty(K, dtype=torch.int32, device=dev)

        def step(t):
            x = pool_x[t % pool_x.shape[0]]
            rvq.router_topk(w, x, K, ids=ids, gates=gates, logits=logits)
            slot_ids = pool.acquire(ids[0].cpu().numpy())
            sd.copy_(torch.from_numpy(slot_ids), non_blocking=False)
            rvq.moe_layer_forward(pool.bank, x, sd, gates[0], dtype="f32", y=y, workspace=ws)
        for t in range(8):
            step(t)
        torch.cuda.synchronize()
        s0 = pool.stats()
        t0 = time.perf_counter()
        for t in range(tokens):
            step(8 + t)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        s1 = pool.stats()
        status = rvq.check_device_status(ws)
        if status:
            raise RuntimeError(rvq.status_string(status))
        if pool.verify_status() != -1:
            raise RuntimeError("an expert record failed its payload CRC-32")
        hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
        out[name] = {"tokens_per_s": tokens / sec, "hit_rate": hits / max(1, hits + misses),
                                 "misses_per_token": misses / tokens,
                                 "h2d_GBps": (s1["bytes_copied"] - s0["bytes_copied"]) / sec / 1e9}
        pool.close()
        del pool, ws
    del hc, hb, rec
    return out


# fp32 VALU lane operations per second: MI355X's published fp32 vector peak (157.3 TFLOP/s) counts
# an FMA as 2 flops, i.e. 78.6 T lane operations/s (256 CUs x 128 lanes per clock x 2.4 GHz); a
# plain sub, mul, add, compare or select is one lane operation.
VALU_LANE_OPS_PEAK = 157.3e12 / 2


def run_encode(torch, rvq, dev, reps=5):
    """RVQ encoding of one 2048 x 7168 matrix (residual, stage-by-stage nearest entry, fp32 decisions):
    weights/s and the VALU rate of its distance arithmetic (3 stages x 256 entries x 8 dims x
    (sub, mul, add) per sub-vector, plus a compare and two selects per entry)."""
    import synth
    rows, cols = I, H
    cb = torch.from_numpy(synth.matrix_codebooks(synth.SEED_EXPERT, 0, 1, synth.GATE)).to(dev)
    W = torch.randn(rows, cols, device=dev, generator=torch.Generator(device=dev).manual_seed(3))
    codes = torch.empty((rows, cols // 8, 3), dtype=torch.uint8, device=dev)
    rvq.rvq_encode(W, cb, codes=codes)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rvq.rvq_encode(W, cb, codes=codes)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    ops = rows * (cols // 8) * 3 * 256 * (3 * 8 + 3)
    return {"ms": sec * 1e3, "weights_per_s": rows * cols / sec, "valu_lane_ops_per_s": ops / sec,
            "frac_of_valu_peak": ops / sec / VALU_LANE_OPS_PEAK}


def run_fit(torch, rvq, dev, iters=8, reps=2):
    """Codebook fitting of one 2048 x 7168 matrix (residual k-means, `iters` Lloyd iterations per stage
    from random starts): ms per matrix, weights/s, the VALU rate of its nearest-entry passes
    (3 x (iters + 1) passes of 256 entries x (3 x 8 + 3) lane operations per sub-vector), and the
    relative squared error of the three-stage reconstruction (Gaussian weights)."""
    rows, cols = I, H
    n = rows * cols // 8
    W = 0.02 * torch.randn(rows, cols, device=dev, generator=torch.Generator(device=dev).manual_seed(4))
    init = np.random.default_rng(4).choice(n, (3, 256)).astype(np.int32)
    ws = torch.empty(rvq.lib().rvq_fit_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    cb, codes = rvq.rvq_fit(W, iters, init, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rvq.rvq_fit(W, iters, init, codebooks=cb, codes=codes, workspace=ws)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    ops = 3 * (iters + 1) * n * 256 * (3 * 8 + 3)
    c = codes.reshape(-1, 3).long()
    rec = (cb[0][c[:, 0]] + cb[1][c[:, 1]] + cb[2][c[:, 2]]).reshape(rows, cols)
    rel = float(((rec.double() - W.double()) ** 2).sum() / (W.double() ** 2).sum())
    return {"iters": iters, "ms": sec * 1e3, "weights_per_s": rows * cols / sec,
            "assign_valu_lane_ops_per_s": ops / sec, "rel_sq_error": rel}


def run_stack_pool(torch, rvq, dev, layers=8, slots=128, tokens=12):
    """Pre-norm stack of 8 layers x 64 experts (8.5 GB of codes) held in pinned host memory behind
    a pool of `slots` device records, decoded token by token, with and without the pages' router
    look-ahead: layer l+1's router run on layer l's normalised input (before layer l's MoE), its
    16 picks, or the 8 highest-ranked, prefetched while layer l decodes.  Tokens/s, pool hit rate, and the fraction of layer l+1's
    experts that the look-ahead predicted."""
    import synth
    from workloads import RMS_EPS, Stack
    st = Stack(layers=layers, device=dev)
    E1, stride = st.E, st.banks[0].stride
    hc = torch.empty(layers * E1 * stride, dtype=torch.uint8, pin_memory=True)
    hb = torch.empty((layers * E1, 3, 3, 256, 8), dtype=torch.float32, pin_memory=True)
    for l in range(layers):
        hc[l * E1 * stride:(l + 1) * E1 * stride].copy_(st.banks[l].codes)
        hb[l * E1:(l + 1) * E1].copy_(st.banks[l].codebooks)
    routers = st.routers
    st.banks = None
    torch.cuda.empty_cache()
    xs = [torch.from_numpy(synth.activation_f32(synth.SEED_STACK, t, H)).to(dev) for t in range(tokens + 2)]
    h = torch.empty(H, dtype=torch.float32, device=dev)
    n = torch.empty_like(h)
    sd = torch.empty(K, dtype=torch.int32, device=dev)
    out = {}
    for look in (0, K, K // 2):
        pool = rvq.ExpertPool(hc, hb, layers * E1, H, I, slots, device=dev)
        ws = rvq.make_moe_workspace(pool.bank, 1, K, "f32")
        pred = {"hit": 0, "n": 0}

        def token(t):
            h.copy_(xs[t])
            nxt = None
            for l in range(layers):
                rvq.rmsnorm(h, RMS_EPS, out=n)
                ids, gates, _ = rvq.router_topk(routers[l], n, K)
                if look and l + 1 < layers:
                    p_ids, _, _ = rvq.router_topk(routers[l + 1], n, K)
                    both = torch.cat([ids[0], p_ids[0]]).cpu().numpy()
                    cur, pnext = both[:K], both[K:]
                else:
                    cur, pnext = ids[0].cpu().numpy(), None
                if nxt is not None:
                    pred["hit"] += len(set(nxt.tolist()) & set(cur.tolist()))
                    pred["n"] += K
                sd.copy_(torch.from_numpy(pool.acquire(cur + l * E1)))
                rvq.moe_layer_forward(pool.bank, n, sd, gates[0], residual=h, y=h, dtype="f32", workspace=ws)
                if pnext is not None:
                    pool.prefetch(pnext[:look] + (l + 1) * E1)   # the `look` highest-ranked picks
                nxt = pnext
        for t in range(2):
            token(t)
        torch.cuda.synchronize()
        s0 = pool.stats()
        pred["hit"] = pred["n"] = 0
        t0 = time.perf_counter()
        for t in range(tokens):
            token(2 + t)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        s1 = pool.stats()
        hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
        key = f"lookahead_top{look}" if look else "no_lookahead"
        out[key] = {"tokens_per_s": tokens / sec, "ms_per_token": sec / tokens * 1e3,
                    "hit_rate": hits / max(1, hits + misses),
                    "h2d_GBps": (s1["bytes_copied"] - s0["bytes_copied"]) / sec / 1e9}
        if look:
            out[key]["predicted_fraction"] = pred["hit"] / max(1, pred["n"])
        pool.close()
        del pool, ws
    out["config"] = {"layers": layers, "experts_per_layer": E1, "slots": slots, "host_bytes": int(hc.numel())}
    del hc, hb
    return out


def run_matvec(torch, rvq, dev, steps):
    """One 256x512 RVQ matvec (fp32 tables): microseconds per call, from a graph of 8 calls (and from
    one graph per call, beside it)."""
    import synth
    from workloads import MATVEC_COLS, MATVEC_ROWS
    R, C = MATVEC_ROWS, MATVEC_COLS
    codes = synth.matrix_codes(synth.SEED_MATVEC, 0, 0, synth.SINGLE, R, C)
    cb = torch.from_numpy(synth.matrix_codebooks(synth.SEED_MATVEC, 0, 0, synth.SINGLE)).to(dev)
    packed = rvq.pack_codes(torch.from_numpy(codes).to(dev), R, C)
    xs = [torch.from_numpy(synth.activation_f32(synth.SEED_MATVEC, t, C)).to(dev) for t in range(8)]
    y = torch.empty(R, dtype=torch.float32, device=dev)
    ws = torch.empty(max(rvq.gemv_workspace_bytes(R, C, "f32"), 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    one = [capture(torch, lambda x=x: rvq.expert_gemv(packed, cb, R, C, x, "f32", y=y, workspace=ws)) for x in xs]
    sec1 = replay_rate(torch, one, steps, 20)
    # the 8 calls in one graph, one after another (as in a full model's graph)
    def calls():
        for x in xs:
            rvq.expert_gemv(packed, cb, R, C, x, "f32", y=y, workspace=ws)
    sec = replay_rate(torch, [capture(torch, calls)], max(1, steps // len(xs)), 3) / len(xs)
    return {"us_per_call": sec * 1e6, "code_GBps": R * C * 3 / 8 / sec / 1e9, "us_per_call_one_per_graph": sec1 * 1e6}


def run_expert(torch, rvq, bank, pool, steps):
    """One SwiGLU expert (7168/2048, fp32 tables) per token: the layer forward with k = 1, rotating
    over 32 of the resident experts so that no expert stays cached; microseconds per token, from
    graphs of STEPS_PER_GRAPH tokens (and from one graph per token, beside it)."""
    dev = pool.device
    ids = [torch.tensor([e], dtype=torch.int32, device=dev) for e in range(0, 256, 8)]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    y = torch.empty(H, dtype=torch.float32, device=dev)
    ws = rvq.make_moe_workspace(bank, 1, 1, "f32")
    torch.cuda.synchronize()
    graphs = [capture(torch, lambda j=j: rvq.moe_layer_forward(bank, pool[j % POOL], ids[j], one, dtype="f32", y=y,
                                                               workspace=ws)) for j in range(len(ids))]
    sec1 = replay_rate(torch, graphs, steps, 20)
    # STEPS_PER_GRAPH tokens in one graph, one after another (as in a full model's graph)
    def tokens(j0):
        for j in range(j0, j0 + STEPS_PER_GRAPH):
            rvq.moe_layer_forward(bank, pool[j % POOL], ids[j], one, dtype="f32", y=y, workspace=ws)
    multi = [capture(torch, lambda j0=j0: tokens(j0)) for j0 in range(0, len(ids), STEPS_PER_GRAPH)]
    sec = replay_rate(torch, multi, max(1, steps // STEPS_PER_GRAPH), 3) / STEPS_PER_GRAPH
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    return {"us_per_token": sec * 1e6, "code_GBps": 3 * (H * I * 3 // 8) / sec / 1e9,
            "us_per_token_one_per_graph": sec1 * 1e6}


def run_stack(torch, rvq, dev, dtype):
    """92-layer stack decode (64 experts per layer, top-16, pre-norm residual blocks): 32 steps of
    fresh tokens, each step one graph of 92 block decodes (RMSNorm folded into the router)."""
    import synth
    from workloads import RMS_EPS, STACK_STEPS, Stack
    print("[bench] uploading the 92-layer stack (97 GB of codes)", file=sys.stderr, flush=True)
    st = Stack(device=dev)
    xin = torch.empty(H, dtype=torch.float32, device=dev)
    h = torch.empty(H, dtype=torch.float32, device=dev)
    ids = torch.empty(K, dtype=torch.int32, device=dev)
    gates = torch.empty(K, dtype=torch.float32, device=dev)
    logits = torch.empty(st.E, dtype=torch.float64, device=dev)
    ws = rvq.make_moe_workspace(st.banks[0], 1, K, dtype)
    xs = [torch.from_numpy(synth.activation_f32(synth.SEED_STACK, t, H)).to(dev) for t in range(STACK_STEPS)]

    def step():
        h.copy_(xin)
        for l in range(st.L):
            rvq.moe_block_decode(st.banks[l], st.routers[l], h, K, RMS_EPS, dtype=dtype, h_out=h, ids=ids,
                                 gates=gates, logits=logits, workspace=ws)
    torch.cuda.synchronize()
    g = capture(torch, step)
    n, total, us = timed_replays(torch, [g], 1, STACK_STEPS * 3, 4, before=lambda i: xin.copy_(xs[i % STACK_STEPS]))
    sec = total / n
    per_token = percentiles(us)
    status = rvq.check_device_status(ws)
    if status:
        raise RuntimeError(rvq.status_string(status))
    code = st.L * K * 3 * (H * I * 3 // 8)
    del st
    torch.cuda.empty_cache()
    return {"tokens_per_s": 1.0 / sec, "ms_per_token": sec * 1e3, "code_GBps": code / sec / 1e9,
            "code_frac_of_hbm_peak": code / sec / 1e9 / HBM_PEAK_GBPS, "table_dtype": dtype,
            "tokens_timed": n, "token_us": per_token}


def stream_copy_peak(torch, rvq, dev):
    """Read+write GB/s of rvq_stream_copy over 1 GiB (the code stream's load instruction); its
    rocprofv3 FETCH_SIZE/WRITE_SIZE per dispatch (1 GiB each) calibrate the counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(2):
        rvq.stream_copy(a, b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 10
    for _ in range(reps):
        rvq.stream_copy(a, b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del a, b
    return 2 * n / dt / 1e9


def stream_read_peak(torch, rvq, bank, reps=10):
    """Read-only GB/s of rvq_stream_read over the resident bank's 4.23 GB of codes (the code stream's
    load instruction, nothing written): the achievable rate of the table kernels' bound."""
    sink = torch.zeros(1, dtype=torch.int32, device=bank.codes.device)
    src = bank.codes[:bank.E * bank.stride]
    for _ in range(2):
        rvq.stream_read(src, sink)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rvq.stream_read(src, sink)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return src.numel() / dt / 1e9


def cpu_baseline(budget_s):
    """The fp64 oracle, as it stands, on a bounded sample: whole tokens of the same layer."""
    import oracle
    import synth
    from workloads import oracle_expert
    bits = synth.router_bf16_bits(synth.SEED_LAYER, 0, E, H)
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = oracle_expert(synth.SEED_LAYER, 0, e)
        return cache[e]

    n, busy = 0, 0.0
    while n == 0 or (busy < budget_s and n < 16 * POOL):   # tokens past the GPU pool's 64 are new seeds
        x = synth.activation_f32(synth.SEED_LAYER, n, H)
        # the codes of the selected experts are regenerated outside the timed part
        l = oracle.router_logits(bits, x[None, :])[0]
        for e in oracle.topk(l, K)[0]:
            get(int(e))
        t0 = time.perf_counter()
        oracle.moe_layer(get, bits, x, K)
        busy += time.perf_counter() - t0
        n += 1   # the cache ends up holding all 256 experts (4.2 GB of host memory)
    return {"value": n / busy, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{n} decode tokens of the same 256-expert top-16 layer (router + 16 full experts, "
                      f"all 7168 outputs), fp64, {busy:.1f} s of CPU time; input generation excluded",
            "code_GBps": CODE_BYTES_PER_TOKEN * n / busy / 1e9,
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--dtype", choices=["f32", "f16"], default="f32", help="table precision of the headline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the other table precision")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-chunk", action="store_true", help="skip the 512-token chunked-prefill measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (one matvec, one expert, the 92-layer stack)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the row-split sharding is designed, not run)", file=sys.stderr)
        sys.exit(2)

    import torch
    import rvq_quantized_moe_amd as rvq
    import synth
    from workloads import router, upload_bank

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] uploading 256-expert bank ({E} x 16.5 MB)", file=sys.stderr, flush=True)
    bank = upload_bank(synth.SEED_LAYER, 0, E, H, I, device=dev)
    _, w = router(synth.SEED_LAYER, 0, E, H, device=dev)
    pool = torch.from_numpy(np.stack([synth.activation_f32(synth.SEED_LAYER, t, H) for t in range(POOL)])).to(dev)
    hip = Hip()
    print("[bench] stream copy and read peaks", file=sys.stderr, flush=True)
    copy_gbps = stream_copy_peak(torch, rvq, dev)
    read_gbps = stream_read_peak(torch, rvq, bank)
    print(f"[bench] timing {args.steps} steps ({args.dtype} tables)", file=sys.stderr, flush=True)
    kernel_steps = max(args.steps, 200)   # per-kernel event timings: at least 200 samples
    main_res = run_variant(rvq, hip, bank, w, pool, kernel_steps, args.warmup, args.dtype)
    print("[bench] graph replay", file=sys.stderr, flush=True)
    step_pct = {}
    graph_tok_s, steps_timed = run_graphed(rvq, bank, w, pool, args.steps, args.warmup, args.dtype, stats=step_pct,
                                           per_graph=STEPS_PER_GRAPH)
    one_step_pct = {}
    graph_one_step, _ = run_graphed(rvq, bank, w, pool, args.steps, args.warmup, args.dtype, stats=one_step_pct)
    graph_two_call, _ = run_graphed(rvq, bank, w, pool, args.steps, args.warmup, args.dtype, routed=False,
                                    per_graph=STEPS_PER_GRAPH)
    variants = {}
    if not args.no_variants:
        other = "f16" if args.dtype == "f32" else "f32"
        print(f"[bench] timing {args.steps} steps ({other} tables)", file=sys.stderr, flush=True)
        variants[other] = run_variant(rvq, hip, bank, w, pool, kernel_steps, args.warmup, other)
        variants[other]["graph_replay_tokens_per_s"] = run_graphed(rvq, bank, w, pool, args.steps, args.warmup, other,
                                                                   per_graph=STEPS_PER_GRAPH)[0]
    chunk = None
    if not args.no_chunk:
        print("[bench] chunked prefill (512 tokens)", file=sys.stderr, flush=True)
        xb = np.stack([synth.activation_bf16_bits(synth.SEED_CHUNK, t, H) for t in range(512)])
        xt = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        chunk = {d: run_chunk(rvq, hip, bank, w, xt, 20, d) for d in ("f16", "bf16")}
        print("[bench] small-batch decode: table path vs chunk path", file=sys.stderr, flush=True)
        chunk["small_batch_decode"] = run_small_batch(torch, rvq, bank, w, xt)
    extra = None
    if not args.no_extra:
        print("[bench] one matvec, one expert", file=sys.stderr, flush=True)
        extra = {"matvec_256x512_f32": run_matvec(torch, rvq, dev, 2000),
                 "expert_7168x2048_f32": run_expert(torch, rvq, bank, pool, 1000),
                 "bank_crc32_256x16.5MB": run_crc(torch, rvq, bank),
                 "rvq_encode_2048x7168": run_encode(torch, rvq, dev),
                 "rvq_fit_2048x7168": run_fit(torch, rvq, dev)}
        print("[bench] expert pool (experts in pinned host memory)", file=sys.stderr, flush=True)
        extra["layer_decode_expert_pool_host_backed"] = run_pool(torch, rvq, bank, w, pool)
        del bank
        torch.cuda.empty_cache()
        extra["stack_92x64_top16_" + args.dtype] = run_stack(torch, rvq, dev, args.dtype)
        print("[bench] 8-layer stack behind an expert pool, router look-ahead", file=sys.stderr, flush=True)
        extra["stack_8x64_host_backed_pool"] = run_stack_pool(torch, rvq, dev)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_budget)

    gu_us = main_res["kernel_us"]["gateup"]
    achieved = (GATEUP_CODE_BYTES + GATEUP_CODEBOOK_BYTES) / (gu_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": graph_tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "steps_requested": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 / graph_tok_s,
        "step_us": step_pct,
        "value_from_step_us_mean": 1e6 / step_pct["mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": "moe_layer_decode", "experts": E, "hidden": H, "inter": I, "top_k": K, "batch": 1,
                   "table_dtype": args.dtype, "accumulate": "f32", "router_accumulate": "f64",
                   "resident_code_bytes": E * 3 * (H * I * 3 // 8), "token_pool": POOL},
        "code_GBps": CODE_BYTES_PER_TOKEN * graph_tok_s / 1e9,
        "code_frac_of_hbm_peak": CODE_BYTES_PER_TOKEN * graph_tok_s / 1e9 / HBM_PEAK_GBPS,
        "code_frac_of_stream_read": CODE_BYTES_PER_TOKEN * graph_tok_s / 1e9 / read_gbps,
        "stream_read_GBps": read_gbps,
        "stream_copy_GBps": copy_gbps,
        "decoded_weights_per_s": WEIGHTS_PER_TOKEN * graph_tok_s,
        "timing": f"value: HIP-graph replays, each graph holding {STEPS_PER_GRAPH} consecutive decode steps "
                  "(one rvq_moe_decode_routed call per token, pool tokens in order), as the layers of a token "
                  "run inside one graph in a full model, replayed back to back for the requested steps or, if "
                  f"those take under {MIN_TIMED_S * 1e3:.0f} ms, for as many more as reach it (steps = steps "
                  "timed); step_us: the same replays' event intervals / steps per graph; "
                  "graph_one_step_per_graph_tokens_per_s: one graph per step, which adds one graph launch to "
                  "every step; kernel_us and roofline: HIP events around each kernel of the two-call form "
                  f"(rvq_router_topk, rvq_moe_layer_forward_timed) in an eager pass of {kernel_steps} steps; "
                  "stream_read_GBps: rvq_stream_read over the resident bank's codes (read only, the code "
                  "stream's loads)",
        "graph_one_step_per_graph_tokens_per_s": graph_one_step,
        "step_us_one_step_per_graph": one_step_pct,
        "graph_two_call_tokens_per_s": graph_two_call,
        "eager_tokens_per_s": main_res["tokens_per_s"],
        "kernel_us": main_res["kernel_us"],
        "roofline": {"bound": "hbm", "kernel": "k_table_ws_f32<gate/up>" if args.dtype == "f32" else "k_table_ws_f16<gate/up>", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profiles(args.dtype),
                     "algorithmic_bytes_per_launch": GATEUP_CODE_BYTES + GATEUP_CODEBOOK_BYTES},
        # the table kernels' LDS ceiling: one lookup per code byte, at the skewed layout's gather rate
        "lds_gather": {"kernel": "gate/up", "lookups_per_s": GATEUP_CODE_BYTES / (gu_us * 1e-6),
                       "ceiling_lookups_per_s": LDS_GATHER_RATE[args.dtype],
                       "frac": GATEUP_CODE_BYTES / (gu_us * 1e-6) / LDS_GATHER_RATE[args.dtype]},
        "cpu_baseline": cpu,
        "variants": variants,
        "chunk_prefill_512": chunk,
        "other_workloads": extra,
        "kernel_source_sha256_16": kernel_source_hash(),
        "device": {"name": torch.cuda.get_device_name(dev), "arch": torch.cuda.get_device_properties(dev).gcnArchName,
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
                   "hip": torch.version.hip, "torch": torch.__version__},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
