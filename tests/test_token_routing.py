"""Per-token routing on the host: lora_build_token_routing is bit-exact with
the oracle's routing of one request per token (the oracle's routing is
pinned on its own), on the pages' token_lora_mapping example, random
mappings, and the error paths."""

import ctypes

import numpy as np
import pytest

import oracle
import segmented_rank_gemv_amd as srg
from segmented_rank_gemv_amd import _lib


def oracle_tokens(token_slot, L):
    T = len(token_slot)
    return oracle.route(np.asarray(token_slot, np.int32), np.arange(T + 1, dtype=np.int64), L)


def same(got, want):
    assert np.array_equal(got["token_indices_sorted"], want["perm"])
    assert np.array_equal(got["lora_ids"], want["lora_ids"])
    assert np.array_equal(got["grouped_offsets"], want["grouped_offsets"])
    assert got["num_groups"] == want["num_groups"] and got["end"] == want["end"]


def test_pages_token_mapping_example():
    """[vLLM] §6 LoRAMapping: token_lora_mapping [slot 0, slot 0, slot 1, ...]
    holds a slot per token; here [0, 0, 1] plus a base token and another
    slot-0 token after it."""
    got = srg.lora_build_token_routing(np.array([0, 0, 1, -1, 0]), 2)
    assert got["token_indices_sorted"].tolist() == [0, 1, 4, 2, 3]
    assert got["lora_ids"].tolist() == [0, 1]
    assert got["grouped_offsets"].tolist() == [0, 3, 4]
    assert got["num_groups"] == 2 and got["end"] == 4
    same(got, oracle_tokens([0, 0, 1, -1, 0], 2))


@pytest.mark.parametrize("seed", range(40))
def test_random_mappings_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 33))
    T = int(rng.integers(0, 400))
    base = float(rng.uniform(0, 1))
    slots = np.where(rng.uniform(size=T) < base, -1, rng.integers(0, L, T)).astype(np.int32)
    same(srg.lora_build_token_routing(slots, L), oracle_tokens(slots, L))


def test_degenerate_mappings():
    for slots, L in (([], 4), ([-1, -1, -1], 4), ([3], 4), ([2] * 50, 3), (list(range(8))[::-1], 8)):
        same(srg.lora_build_token_routing(np.array(slots, np.int32), L), oracle_tokens(slots, L))


def test_errors():
    with pytest.raises(srg.LoraError) as e:
        srg.lora_build_token_routing(np.array([0, 4]), 4)
    assert e.value.code == 3
    with pytest.raises(srg.LoraError) as e:
        srg.lora_build_token_routing(np.array([-2]), 4)
    assert e.value.code == 3
    lib = _lib._load()
    out = np.zeros(8, np.int32)
    G = np.zeros(1, np.int32)
    end = np.zeros(1, np.int64)
    p = lambda a: a.ctypes.data
    assert lib.lora_build_token_routing(-1, None, 4, None, p(out), p(out), p(G), p(end)) == 1
    assert lib.lora_build_token_routing(2, None, 4, p(out), p(out), p(out), p(G), p(end)) == 1
    assert lib.lora_build_token_routing(0, None, 0, None, p(out), p(out), p(G), p(end)) == 1


def test_routing_struct_layout_carries_the_token_rows():
    """The binding's routing struct ends with token_rows and num_rows, as the
    header declares (ABI 7)."""
    names = [f[0] for f in _lib._LoraRouting._fields_]
    assert names[-2:] == ["token_rows", "num_rows"]
    assert ctypes.sizeof(_lib._LoraRouting) == 64
