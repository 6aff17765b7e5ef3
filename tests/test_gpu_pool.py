"""Expert pool (experts in pinned host memory, an LRU set of device slots): decoding through the
pool's slots gives the all-resident result bit for bit, and the hit/miss accounting follows the
LRU policy, computed independently here."""
import sys

import numpy as np
import pytest
import torch

import rvq_quantized_moe_amd as rvq
import synth
from workloads import HIDDEN, INTER, router, upload_bank

pytestmark = pytest.mark.gpu
E_POOL = 24


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
    bank = upload_bank(synth.SEED_EXPERT ^ 0x5, 0, E_POOL)
    hc = torch.empty(bank.codes.numel(), dtype=torch.uint8, pin_memory=True)
    hc.copy_(bank.codes)
    hb = torch.empty(bank.codebooks.shape, dtype=torch.float32, pin_memory=True)
    hb.copy_(bank.codebooks)
    bits, w = router(synth.SEED_EXPERT ^ 0x5, 0, E_POOL, HIDDEN)
    return bank, hc, hb, w


@pytest.mark.parametrize("slots,k,prefetch", [(10, 4, False), (4, 4, False), (12, 4, True)])
def test_pool_decode_matches_resident_bank(store, slots, k, prefetch):
    """slots = k evicts on almost every step (copies must wait for the previous step's kernels);
    with prefetch the next token's experts are copied while the current one decodes."""
    bank, hc, hb, w = store
    say(f"pool slots={slots} k={k} prefetch={prefetch}")
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
