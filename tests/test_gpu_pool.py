"""Expert pool (experts in pinned host memory, an LRU set of device slots): decoding through the
pool's slots gives the all-resident result bit for bit, and the hit/miss accounting follows the
LRU policy, computed independently here.  Over a store of expert records, every read checks the
record's header and, with verify on, the payload's CRC-32 against the oracle's."""
import sys

import numpy as np
import pytest
import torch

import oracle
import rvq_quantized_moe_amd as rvq
import synth
from workloads import HIDDEN, INTER, oracle_expert, rel_l2, router, upload_bank

pytestmark = pytest.mark.gpu
E_POOL = 24
SEED_POOL = synth.SEED_EXPERT ^ 0x5
_ORACLE_EXPERTS = {}


def oracle_get(e):
    """The pool's experts as the oracle sees them, regenerated from their seeds (never read back)."""
    if e not in _ORACLE_EXPERTS:
        _ORACLE_EXPERTS[e] = oracle_expert(SEED_POOL, 0, e)
    return _ORACLE_EXPERTS[e]


def assert_matches_oracle(y, x, ids, gates):
    """A pool decode against the oracle's mix of the same experts and gates (fp32 tables: 1e-5)."""
    y_ref = oracle.moe_mix(oracle_get, np.asarray(x, dtype=np.float64), np.asarray(ids), np.asarray(gates))
    err = rel_l2(y, y_ref)
    say(f"  rel-L2 {err:.3e} against the oracle")
    assert err <= 1e-5


def say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def lru_model(slots, events):
    """Counts of the pool's policy: events are ("acquire", ids) or ("prefetch", ids)."""
    stamp, clock, hits, misses, pre, latest = {}, 0, 0, 0, 0, set()

    def victim(excl):
        if len(stamp) < slots:
            return None
        cands = [e for e in stamp if e not in excl]
        return min(cands, key=stamp.get) if cands else -1
    for kind, ids in events:
        if kind == "acquire":
            cur = set()
            for e in ids:
                if e in stamp:
                    if e not in cur:
                        hits += 1
                    cur.add(e)
                    clock += 1
                    stamp[e] = clock
            for e in ids:
                if e not in stamp:
                    misses += 1
                    v = victim(cur)
                    if v is not None:
                        del stamp[v]
                    clock += 1
                    stamp[e] = clock
                    cur.add(e)
            latest = cur
        else:
            for e in ids:
                if e in stamp:
                    continue
                v = victim(latest)
                if v == -1:
                    break
                if v is not None:
                    del stamp[v]
                clock += 1
                stamp[e] = clock
                pre += 1
    return hits, misses, pre


@pytest.fixture(scope="module")
def store():
    say(f"upload {E_POOL} experts and copy them to pinned host memory")
    bank = upload_bank(SEED_POOL, 0, E_POOL)
    hc = torch.empty(bank.codes.numel(), dtype=torch.uint8, pin_memory=True)
    hc.copy_(bank.codes)
    hb = torch.empty(bank.codebooks.shape, dtype=torch.float32, pin_memory=True)
    hb.copy_(bank.codebooks)
    bits, w = router(SEED_POOL, 0, E_POOL, HIDDEN)
    return bank, hc, hb, w


@pytest.mark.parametrize("slots,k,prefetch", [(10, 4, False), (4, 4, False), (12, 4, True)])
def test_pool_decode_matches_resident_bank(store, slots, k, prefetch):
    """slots = k evicts on almost every step (copies must wait for the previous step's kernels);
    with prefetch the next token's experts are copied while the current one decodes.  Every decode
    equals the resident bank bit for bit; the first and last against the oracle's routed layer."""
    bank, hc, hb, w = store
    say(f"pool slots={slots} k={k} prefetch={prefetch}")
    bits = synth.router_bf16_bits(SEED_POOL, 0, E_POOL, HIDDEN)
    pool = rvq.ExpertPool(hc, hb, E_POOL, HIDDEN, INTER, slots)
    ws = rvq.make_moe_workspace(bank, 1, k, "f32")
    wsp = rvq.make_moe_workspace(pool.bank, 1, k, "f32")
    events = []
    xs = [torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT ^ 0x5, 300 + t, HIDDEN)).cuda() for t in range(10)]
    routes = [rvq.router_topk(w, x, k) for x in xs]
    host_ids = [r[0][0].cpu().numpy() for r in routes]
    try:
        for t in range(len(xs)):
            ids, gates, _ = routes[t]
            slot_ids = pool.acquire(host_ids[t])
            events.append(("acquire", [int(e) for e in host_ids[t]]))
            sd = torch.from_numpy(slot_ids).cuda()
            y = rvq.moe_layer_forward(pool.bank, xs[t], sd, gates[0], dtype="f32", workspace=wsp)
            if prefetch and t + 1 < len(xs):
                pool.prefetch(host_ids[t + 1])
                events.append(("prefetch", [int(e) for e in host_ids[t + 1]]))
            ref = rvq.moe_layer_forward(bank, xs[t], ids[0], gates[0], dtype="f32", workspace=ws)
            assert torch.equal(y, ref), t
            if t in (0, len(xs) - 1):
                y_ref, ids_ref, g_ref, _ = oracle.moe_layer(oracle_get, bits, xs[t].cpu().numpy(), k)
                assert np.array_equal(host_ids[t], ids_ref)
                assert rel_l2(y.cpu().numpy(), y_ref) <= 1e-5, t
        st = pool.stats()
        hits, misses, pre = lru_model(slots, events)
        assert (st["hits"], st["misses"], st["prefetches"]) == (hits, misses, pre)
        assert st["bytes_copied"] == (misses + pre) * (bank.record_bytes + 3 * 6144 * 4)
        assert rvq.check_device_status(wsp) == 0
    finally:
        pool.close()


def test_pool_rejects_bad_ids(store):
    bank, hc, hb, w = store
    pool = rvq.ExpertPool(hc, hb, E_POOL, HIDDEN, INTER, 4)
    try:
        with pytest.raises(rvq.RvqError):
            pool.acquire([0, E_POOL])
        with pytest.raises(rvq.RvqError):
            pool.acquire([0, 1, 2, 3, 4])   # more experts than slots
        assert pool.stats()["misses"] == 0
    finally:
        pool.close()


def test_pool_two_layer_lookahead_matches_resident(store):
    """The pages' look-ahead on a 2-layer pre-norm stack over the pool (the 24 experts as 2 layers of
    12): layer 1's router run early on layer 0's normalised input, its picks prefetched while layer
    0 decodes; the final h equals the all-resident computation bit for bit."""
    bank, hc, hb, _ = store
    say("pool: 2-layer stack with router look-ahead")
    E1, k = 12, 4
    routers = [router(synth.SEED_EXPERT ^ 0x6, l, E1, HIDDEN)[1] for l in range(2)]
    pool = rvq.ExpertPool(hc, hb, E_POOL, HIDDEN, INTER, 8)
    ws = rvq.make_moe_workspace(pool.bank, 1, k, "f32")
    wsr = rvq.make_moe_workspace(bank, 1, k, "f32")
    try:
        for t in range(4):
            x = torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT ^ 0x6, t, HIDDEN)).cuda()
            h, href = x.clone(), x.clone()
            for l in range(2):
                n = rvq.rmsnorm(h, 1e-6)
                ids, gates, _ = rvq.router_topk(routers[l], n, k)
                if l == 0:
                    pred, _, _ = rvq.router_topk(routers[1], n, k)
                    pred_h = pred[0].cpu().numpy() + E1
                slot = pool.acquire(ids[0].cpu().numpy() + l * E1)
                rvq.moe_layer_forward(pool.bank, n, torch.from_numpy(slot).cuda(), gates[0], residual=h, y=h,
                                      dtype="f32", workspace=ws)
                if l == 0:
                    pool.prefetch(pred_h)
                nr = rvq.rmsnorm(href, 1e-6)
                idr, gr, _ = rvq.router_topk(routers[l], nr, k)
                rvq.moe_layer_forward(bank, nr, idr[0] + l * E1, gr[0], residual=href, y=href, dtype="f32",
                                      workspace=wsr)
            assert torch.equal(h, href), t
        assert pool.stats()["prefetches"] > 0
    finally:
        pool.close()


def test_pool_evicts_slots_with_lookahead_copies_in_flight(store):
    """Look-ahead copies run on their own stream; an acquire that right away needs every slot evicts
    the slots being prefetched into, so its copies must queue behind theirs.  6 slots: acquire 4,
    prefetch 2 others, acquire 6 new ones at once; every decode equals the resident bank."""
    bank, hc, hb, w = store
    say("pool: eviction of slots with look-ahead copies in flight")
    pool = rvq.ExpertPool(hc, hb, E_POOL, HIDDEN, INTER, 6)
    ws = rvq.make_moe_workspace(pool.bank, 1, 6, "f32")
    wsr = rvq.make_moe_workspace(bank, 1, 6, "f32")
    rng = np.random.default_rng(9)
    x = torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT ^ 0x5, 77, HIDDEN)).cuda()

    def decode(ids):
        g = torch.from_numpy(rng.random(len(ids)).astype(np.float32)).cuda()
        slot = pool.acquire(ids)
        y = rvq.moe_layer_forward(pool.bank, x, torch.from_numpy(slot).cuda(), g, dtype="f32", workspace=ws)
        ref = rvq.moe_layer_forward(bank, x, torch.tensor(ids, dtype=torch.int32).cuda(), g, dtype="f32",
                                    workspace=wsr)
        assert torch.equal(y, ref), ids
    try:
        for r in range(4):
            perm = rng.permutation(E_POOL)
            decode(perm[:4])
            pool.prefetch(perm[4:6])
            decode(perm[6:12])
        assert pool.stats()["prefetches"] > 0
    finally:
        pool.close()


REC_LAYER = 17


@pytest.fixture(scope="module")
def records(store):
    """The 24 experts as records of layer 17, header CRCs computed by the oracle from the packed codes."""
    bank = store[0]
    say("write the pool's experts as records")
    codes = bank.codes.view(E_POOL, bank.stride)[:, :bank.record_bytes].cpu().numpy()
    crcs = [oracle.crc32(codes[e]) for e in range(E_POOL)]
    return rvq.write_records(bank, REC_LAYER, crcs), crcs


def _decode_both(pool, bank, ids, x, ws, wsr, rng, check_oracle=False):
    g = torch.from_numpy(rng.random(len(ids)).astype(np.float32)).cuda()
    slot = pool.acquire(ids)
    y = rvq.moe_layer_forward(pool.bank, x, torch.from_numpy(slot).cuda(), g, dtype="f32", workspace=ws)
    ref = rvq.moe_layer_forward(bank, x, torch.tensor(np.asarray(ids), dtype=torch.int32).cuda(), g, dtype="f32",
                                workspace=wsr)
    if check_oracle:
        assert_matches_oracle(y.cpu().numpy(), x.cpu().numpy(), ids, g.cpu().numpy())
    return y, ref


@pytest.mark.parametrize("verify", [False, True])
def test_record_pool_matches_resident_bank(store, records, verify):
    """Slots filled from records (header checked on every read; with verify, each payload's CRC-32 too)
    decode exactly as the resident bank, and the first and last decodes match the oracle's mix of
    the same experts and gates; clean records report no CRC failure."""
    bank = store[0]
    rec, _ = records
    say(f"record pool verify={verify}")
    pool = rvq.ExpertPool.from_records(rec, REC_LAYER, E_POOL, HIDDEN, INTER, 6, verify=verify)
    ws = rvq.make_moe_workspace(pool.bank, 1, 4, "f32")
    wsr = rvq.make_moe_workspace(bank, 1, 4, "f32")
    rng = np.random.default_rng(11)
    x = torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT ^ 0x5, 91, HIDDEN)).cuda()
    try:
        for r in range(5):
            perm = rng.permutation(E_POOL)
            y, ref = _decode_both(pool, bank, perm[:4], x, ws, wsr, rng, check_oracle=r in (0, 4))
            assert torch.equal(y, ref), r
            pool.prefetch(perm[4:6])
        assert pool.verify_status() == -1
        assert pool.stats()["misses"] > 0
    finally:
        pool.close()


def test_record_pool_refuses_bad_headers(store, records):
    """A record with a damaged magic, one carrying another expert's header (a wrongly joined store) and
    one whose code offset runs past its end are refused on read: the acquire that needs them copies
    nothing and changes no state; other records still load."""
    bank = store[0]
    rec, _ = records
    rb = rvq.record_bytes(HIDDEN, INTER)
    say("record pool: damaged headers")
    saved = {e: rec[e * rb:e * rb + 64].clone() for e in (3, 7, 9)}
    rec[3 * rb] ^= 0xFF                                                   # magic
    rec[7 * rb:7 * rb + 64] = rec[8 * rb:8 * rb + 64]                     # expert 8's header in record 7
    hdr = rvq.RecordHeader.from_buffer_copy(bytes(rec[9 * rb:9 * rb + 64].numpy()))
    hdr.codes_offset = rb - hdr.codes_bytes + 4096                        # past the record's end
    rec[9 * rb:9 * rb + 64] = torch.frombuffer(bytearray(bytes(hdr)), dtype=torch.uint8)
    pool = rvq.ExpertPool.from_records(rec, REC_LAYER, E_POOL, HIDDEN, INTER, 6)
    ws = rvq.make_moe_workspace(pool.bank, 1, 4, "f32")
    wsr = rvq.make_moe_workspace(bank, 1, 4, "f32")
    rng = np.random.default_rng(12)
    x = torch.from_numpy(synth.activation_f32(synth.SEED_EXPERT ^ 0x5, 92, HIDDEN)).cuda()
    try:
        for bad in (3, 7, 9):
            with pytest.raises(rvq.RvqError) as ei:
                pool.acquire([0, bad])
            assert ei.value.status == rvq._lib.RVQ_ERR_RECORD
        assert pool.stats() == {"hits": 0, "misses": 0, "prefetches": 0, "bytes_copied": 0}
        y, ref = _decode_both(pool, bank, [0, 1, 2, 8], x, ws, wsr, rng)
        assert torch.equal(y, ref)
        with pytest.raises(rvq.RvqError):
            pool.prefetch([4, 7, 5])   # copies 4, stops at 7
        assert pool.stats()["prefetches"] == 1
        y, ref = _decode_both(pool, bank, [4, 1, 10, 11], x, ws, wsr, rng)
        assert torch.equal(y, ref)
        assert pool.stats()["hits"] == 2
    finally:
        pool.close()
        for e, h in saved.items():
            rec[e * rb:e * rb + 64] = h


def test_record_pool_verify_reports_a_corrupt_payload(store, records):
    """One flipped byte in expert 5's codes (header intact, CRC of the clean payload): the header check
    passes, the device CRC check after the demand copy reports expert 5, once; loads of clean records
    report nothing; a flipped last byte of expert 9, copied by look-ahead, is reported by the other
    check stream; a pool without verify does not check."""
    bank = store[0]
    rec, crcs = records
    rb = rvq.record_bytes(HIDDEN, INTER)
    hdr = rvq.RecordHeader.from_buffer_copy(bytes(rec[5 * rb:5 * rb + 64].numpy()))
    pos = 5 * rb + hdr.codes_offset + 1_234_567
    pos9 = 9 * rb + hdr.codes_offset + hdr.codes_bytes - 1   # the last payload byte, copied ahead
    say("record pool: corrupt payload under verify")
    rec[pos] ^= 0x10
    rec[pos9] ^= 0x01
    try:
        pool = rvq.ExpertPool.from_records(rec, REC_LAYER, E_POOL, HIDDEN, INTER, 4, verify=True)
        try:
            pool.acquire([1, 2])
            assert pool.verify_status() == -1
            pool.acquire([5, 6])
            assert pool.verify_status() == 5
            assert pool.verify_status() == -1   # reported once, then cleared
            pool.prefetch([7])
            pool.acquire([7, 8])
            assert pool.verify_status() == -1
            pool.prefetch([9])                    # checked on the look-ahead side
            assert pool.verify_status() == 9
        finally:
            pool.close()
        plain = rvq.ExpertPool.from_records(rec, REC_LAYER, E_POOL, HIDDEN, INTER, 4, verify=False)
        try:
            plain.acquire([5])
            assert plain.verify_status() == -1
        finally:
            plain.close()
    finally:
        rec[pos] ^= 0x10
        rec[pos9] ^= 0x01
