"""GPU parity of the slot table's capacity and cold tier: the library, driven through the
C ABI, and the oracle's state machine (Shared KV Cache Serving, Cold-tier state
machine) take the same random sequence of stores, queries, lookups and drops; after
every step the statuses, every key's state and the telemetry must be identical. Slots
are small fp16 prefixes whose K + V bytes (4 H N D) are multiples of 256, the bytes
the library accounts per slot. Queries that succeed are also checked against the
attention oracle."""
import numpy as np
import pytest

import oracle
import synth
from oracle.cold_tier import ColdTier
from test_gpu_parity import check, dev, empty, host, query

pytestmark = pytest.mark.gpu

SID = "ct"
H, D = 2, 64
KEYS = 8


@pytest.fixture
def kp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_prefix_amd as kp
    kp.lib()
    s = kp.pion_prefix_stats()
    assert s["warm_slots"] == 0 and s["cold_slots"] == 0, "the slot table must start empty"
    saved = (s["max_slots"], s["max_bytes"], s["cold_capacity"])
    yield kp
    kp.pion_prefix_drop(SID, -1)
    kp.pion_prefix_set_capacity(*saved)


def slot_bytes(N):
    return 4 * H * N * D


def compare(kp, model, base):
    for i in range(KEYS):
        assert kp.pion_prefix_lookup(SID, i) == model.lookup((SID, i)), i
    s, m = kp.pion_prefix_stats(), model.stats()
    assert s["warm_slots"] == m["warm"] and s["cold_slots"] == m["cold"]
    assert s["demotions"] - base["demotions"] == m["demotions"]
    assert s["rehydrates"] - base["rehydrates"] == m["rehydrates"]
    assert s["resident_bytes"] == m["resident_bytes"]


def status_of(fn):
    import kv_cache_prefix_amd as k
    try:
        fn()
        return k.PION_OK
    except k.PionError as e:
        return e.status


@pytest.mark.parametrize("max_slots,max_bytes,cold", [(3, 0, 2), (5, 0, 1024), (8, 4 * H * 160 * D, 3)])
def test_state_machine_matches_oracle(kp, max_slots, max_bytes, cold):
    rng = np.random.default_rng(max_slots * 7 + cold)
    base = kp.pion_prefix_stats()
    kp.pion_prefix_set_capacity(max_slots, max_bytes, cold)
    model = ColdTier(max_slots, max_bytes, cold)
    data = {}
    for step in range(160):
        key = int(rng.integers(0, KEYS))
        r = rng.random()
        if r < 0.45:
            N = int(rng.choice([16, 32, 48, 64, 96]))
            inp = synth.generate(synth.DECODE, 40 + step, N=N, D=D, H_q=H, H_kv=H)
            want = model.store((SID, key), slot_bytes(N))
            got = status_of(lambda: kp.pion_prefix_store(SID, key, dev(inp.K), dev(inp.V)))
            assert got == want, (step, got, want)
            if got == 0:
                data[key] = inp
        elif r < 0.9:
            want = model.query((SID, key))
            inp = data.get(key)
            Q = inp.Q if inp is not None else np.zeros((H, 1, D), np.float16)
            res = {}
            got = status_of(lambda: res.setdefault("r", query(kp, SID, key, Q)))
            assert got == want, (step, got, want)
            if got == 0 and step % 10 == 0:
                check(*res["r"], *oracle.prefix_query(inp.Q, inp.K, inp.V))
        elif r < 0.95:
            assert kp.pion_prefix_drop(SID, key) == model.drop(SID, key)
        else:
            assert kp.pion_prefix_lookup(SID, key) == model.lookup((SID, key))
        compare(kp, model, base)
    # lowering the capacity demotes at once
    kp.pion_prefix_set_capacity(1, 0, cold)
    model.set_capacity(1, 0, cold)
    compare(kp, model, base)


def test_cold_key_answers_coldmiss_in_every_query_form(kp):
    import kv_cache_prefix_amd as k
    kp.pion_prefix_set_capacity(1, 0, 4)
    a = synth.generate(synth.DECODE, 60, N=64, D=D, H_q=H, H_kv=H, S_suf=8)
    b = synth.generate(synth.DECODE, 61, N=32, D=D, H_q=H, H_kv=H)
    kp.pion_prefix_store(SID, 0, dev(a.K), dev(a.V))
    kp.pion_prefix_store(SID, 1, dev(b.K), dev(b.V))          # demotes layer 0
    assert kp.pion_prefix_lookup(SID, 0) == 2
    with pytest.raises(k.PionError) as e:
        kp.pion_prefix_info(SID, 0)
    assert e.value.status == k.PION_ERR_COLDMISS
    calls = [
        lambda: query(kp, SID, 0, a.Q),
        lambda: kp.pion_prefix_query_layers(SID, 0, dev(a.Q[None]), empty((1, H, 1, D))),
        lambda: kp.pion_prefix_query_fused(SID, 0, dev(a.Q), dev(a.K_suf), dev(a.V_suf),
                                           empty((H, 1, D))),
        lambda: kp.pion_prefix_query_sparse_auto(SID, 0, dev(a.Q), 16, 2, empty((H, D)), H_kv=H),
        lambda: kp.pion_prefix_query_sparse(SID, 0, dev(a.Q), dev(np.zeros((H, 4), np.int32)),
                                            dev(np.ones(H, np.int32)), empty((H, D))),
    ]
    for c in calls:
        with pytest.raises(k.PionError) as e:
            c()
        assert e.value.status == k.PION_ERR_COLDMISS
    r0 = kp.pion_prefix_stats()["rehydrates"]
    kp.pion_prefix_store(SID, 0, dev(a.K), dev(a.V))          # rehydrate from the caller's copy
    assert kp.pion_prefix_stats()["rehydrates"] == r0 + 1
    assert kp.pion_prefix_lookup(SID, 0) == 1 and kp.pion_prefix_lookup(SID, 1) == 2
    check(*query(kp, SID, 0, a.Q), *oracle.prefix_query(a.Q, a.K, a.V))
