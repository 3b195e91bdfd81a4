"""Adapter slot cache (lora_cache_*): the library against the plain-Python
oracle of the pages' activate / evict / unload / pin rules, on the pages'
worked example, hand-derived LRU cases, error paths and long random
operation sequences (integer work: results must be identical)."""

import json
import os

import numpy as np
import pytest

import oracle
import segmented_rank_gemv_amd as srg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def both(n, policy=srg.CACHE_LRU):
    return srg.LoraSlotCache(n, policy), oracle.OracleSlotCache(n, policy)


def table(c):
    ids, pinned = c.slot_table()
    return [int(v) for v in ids], [int(v) for v in pinned]


def test_pages_slot_table_example():
    """vLLM §9: four slots; asr-v1 (id 1) then asr-v2 (id 2) give
    lora_index_to_id = [1, 2, None, None]; the first activation takes slot 0."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "vllm_slot_table_example.json")))["printed_by_page"]
    for c in both(g["max_loras"]):
        first = None
        for a in g["activated_in_order"]:
            slot, load, ev = c.activate(a)
            first = slot if first is None else first
            assert load and ev == -1
        assert first == g["first_activation_slot"]
        assert table(c)[0] == [-1 if v is None else v for v in g["lora_index_to_id"]]


def test_active_adapter_keeps_its_slot_and_no_evict_policy_fails_when_full():
    """vLLM §5.3: an active id is skipped (no reload); the base manager raises
    'No free lora slots' when every slot is taken."""
    lib, orc = both(3, srg.CACHE_NO_EVICT)
    for c in (lib, orc):
        assert [c.activate(a)[0] for a in (10, 11, 12)] == [0, 1, 2]
        assert c.activate(11) == (1, False, -1)
    with pytest.raises(srg.LoraError) as e:
        lib.activate(13)
    assert e.value.code == 7 and isinstance(e.value, ValueError)
    with pytest.raises(oracle.SlotCacheError) as e2:
        orc.activate(13)
    assert e2.value.code == 7
    assert table(lib) == table(orc)


def test_lru_evicts_least_recently_used_and_reuses_its_slot():
    """vLLM §7 (remove_oldest, activate into the first free slot, touch) and
    MAX-V3 activate_adapter, derived by hand: 1..4 fill four slots, touching 1
    makes 2 the oldest, so 5 evicts 2 and takes slot 1; then 6 evicts 3."""
    for c in both(4):
        for a in (1, 2, 3, 4):
            c.activate(a)
        assert c.activate(1) == (0, False, -1)
        assert c.activate(5) == (1, True, 2)
        assert c.activate(6) == (2, True, 3)
        assert table(c) == ([1, 5, 6, 4], [0, 0, 0, 0])
        assert c.lookup(2) == -1 and c.lookup(4) == 3


def test_pinned_adapters_are_never_evicted():
    for c in both(2):
        assert c.pin(7) == (0, True, -1)
        c.activate(8)
        assert c.activate(9) == (1, True, 8)   # 7 is older but pinned
        c.pin(9)
        with pytest.raises((srg.LoraError, oracle.SlotCacheError)) as e:
            c.activate(10)
        assert e.value.code == 7
        c.pin(7, False)
        assert c.activate(10) == (0, True, 7)


def test_unload_frees_the_slot():
    """MAX-V3 unload_adapter frees the adapter's LRU slot; unloading an
    adapter that holds none is UNLOAD_NAME_NONEXISTENT (NOT_ACTIVE)."""
    for c in both(3):
        for a in (4, 5, 6):
            c.activate(a)
        assert c.unload(5) == 1
        assert c.activate(7) == (1, True, -1)     # the freed slot, nothing evicted
        with pytest.raises((srg.LoraError, oracle.SlotCacheError)) as e:
            c.unload(5)
        assert e.value.code == 8


def test_batch_activation_never_evicts_its_own_adapters():
    """All adapters of a batch are active together (vLLM §3.6 / §4
    set_active_adapters before the forward): a batch evicts only adapters it
    does not use, fails if it needs more slots than exist, and leaves the cache
    unchanged when it fails."""
    for c in both(3):
        for a in (1, 2, 3):
            c.activate(a)
        slots, loads, ids = c.activate_batch([4, -1, 1, 4, 5])
        assert list(slots) == [1, -1, 0, 1, 2]   # 4 evicts 2, 5 evicts 3 (1 is in the batch)
        assert list(loads) == [1, 2] and list(ids) == [4, 5]
        before = table(c)
        with pytest.raises((srg.LoraError, oracle.SlotCacheError)) as e:
            c.activate_batch([6, 7, 8, 9])
        assert e.value.code == 7
        assert table(c) == before


@pytest.mark.parametrize("bad", [dict(n=0), dict(n=2, policy=5), dict(n=-3)])
def test_create_rejects_bad_arguments(bad):
    with pytest.raises(srg.LoraError) as e:
        srg.LoraSlotCache(bad["n"], bad.get("policy", srg.CACHE_LRU))
    assert e.value.code == 1


def test_bad_ids_rejected():
    c = srg.LoraSlotCache(2)
    for op in (lambda: c.activate(-1), lambda: c.unload(-4), lambda: c.pin(-1),
               lambda: c.activate_batch([0, -2])):
        with pytest.raises(srg.LoraError) as e:
            op()
        assert e.value.code == 1
    assert c.lookup(3) == -1


def run_op(c, op, arg):
    try:
        if op == "activate":
            r = c.activate(arg)
        elif op == "batch":
            s, l, i = c.activate_batch(arg)
            r = ([int(v) for v in s], [int(v) for v in l], [int(v) for v in i])
        elif op == "unload":
            r = c.unload(arg)
        elif op == "pin":
            r = c.pin(arg, True)
        elif op == "unpin":
            r = c.pin(arg, False)
        else:
            r = c.lookup(arg)
        return ("ok", r)
    except (srg.LoraError, oracle.SlotCacheError) as e:
        return ("err", e.code)


@pytest.mark.parametrize("policy", [srg.CACHE_LRU, srg.CACHE_NO_EVICT])
def test_random_operation_sequences_match_oracle(policy):
    rng = np.random.default_rng(1234 + policy)
    ops = ["activate", "activate", "activate", "batch", "unload", "pin", "unpin", "lookup"]
    for trial in range(300):
        n = int(rng.integers(1, 7))
        lib, orc = both(n, policy)
        for step in range(60):
            op = ops[int(rng.integers(len(ops)))]
            if op == "batch":
                arg = [int(v) for v in rng.integers(-1, 12, size=int(rng.integers(0, 9)))]
            else:
                arg = int(rng.integers(0, 12))
            a, b = run_op(lib, op, arg), run_op(orc, op, arg)
            assert a == b, (trial, step, op, arg, a, b)
            assert table(lib) == table(orc), (trial, step, op, arg)
