"""Adapter activation on the GPU: a stream of batches whose requests name
more adapters than there are slots.  Each batch activates its adapters in
the library's slot cache, writes the adapters that need loading into the
device stacks with lora_write_slot, routes by slot and runs the delta; the
oracle keeps its own slot cache and packs each slot's adapter itself, and
the results are compared request by request.  Also: lora_reset_slot zeroes
exactly one slot."""

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg
from lora_case import TOL, GpuLayer, compare, dims_of, from_dev, log, oracle_layer

pytestmark = pytest.mark.gpu


def workload(L=4):
    base = synth.get_workload("decode")
    return synth.Workload(**{**base.__dict__, "hidden": 512, "n_heads": 4, "n_kv_heads": 2,
                             "head_dim": 128, "max_lora_rank": 16, "max_num_loras": L})


def adapter(w, adapter_id):
    rank = (8, 16, 4, 12)[adapter_id % 4]
    return rank, synth.draw_adapter(w, 0, 100 + adapter_id, rank)


def empty_stacks(w, d):
    """Device stacks of zeros, shaped as lora_pack_adapter lays one slot out."""
    import torch
    rank, wts = adapter(w, 0)
    pk = srg.lora_pack_adapter(d, rank, w.lora_alpha, w.use_rslora, True, "qkvo", wts)
    return {k: torch.zeros((w.max_num_loras,) + v.shape, dtype=torch.bfloat16, device="cuda")
            for k, v in pk.items()}


@pytest.mark.parametrize("fused", [False, True])
def test_activation_stream_matches_oracle(fused):
    import torch
    w = workload()
    d = dims_of(w)
    rng = np.random.default_rng(77)
    cache, ocache = srg.LoraSlotCache(w.max_num_loras), oracle.OracleSlotCache(w.max_num_loras)
    dev = empty_stacks(w, d)
    # the oracle's view of the stacks (logical layout, bf16 bit patterns)
    rank0, wts0 = adapter(w, 0)
    shapes = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.dtype,
                                 rank0, w.lora_alpha, w.use_rslora, True, "qkvo", wts0)
    ref = {k: np.zeros((w.max_num_loras,) + v.shape, v.dtype) for k, v in shapes.items()}
    total_loads = 0
    for b in range(8):
        n = int(rng.integers(3, 9))
        ids = rng.choice(np.array([-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9]), size=n)
        # at most max_num_loras distinct adapters per batch
        uniq = [a for a in dict.fromkeys(ids.tolist()) if a >= 0][:w.max_num_loras]
        ids = np.array([a if (a < 0 or a in uniq) else -1 for a in ids.tolist()], np.int64)
        lengths = rng.integers(0, 20, size=n).astype(np.int64)
        slots, load_slots, load_ids = cache.activate_batch(ids)
        o_slots, o_load_slots, o_load_ids = ocache.activate_batch(ids.tolist())
        assert list(slots) == o_slots and list(load_slots) == o_load_slots and list(load_ids) == o_load_ids
        for s, a in zip(load_slots.tolist(), load_ids.tolist()):
            rank, wts = adapter(w, a)
            pk = srg.lora_pack_adapter(d, rank, w.lora_alpha, w.use_rslora, True, "qkvo", wts)
            srg.lora_write_slot(d, s, pk, dev)
            po = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                                     w.dtype, rank, w.lora_alpha, w.use_rslora, True, "qkvo", wts)
            for k in ref:
                ref[k][s] = po[k]
        total_loads += len(load_slots)
        torch.cuda.synchronize()
        acts = synth.draw_activations(w, b, int(lengths.sum()))
        dummy = {k: np.zeros((1,), np.uint16) for k in ("A_qkv", "B_qkv", "A_o", "B_o")}
        gl = GpuLayer(w, dummy, lengths, slots.astype(np.int32), acts)
        gl.st = dev
        log(f"[slot-cache] batch {b} ids={ids.tolist()} slots={slots.tolist()} loads={load_ids.tolist()}")
        gl.run(srg.PATH_AUTO, fused=fused)
        ey, _ = compare(w, gl, oracle_layer(w, {"ref": ref}, lengths, slots.astype(np.int32), acts),
                        check_u=False)
        assert ey <= TOL["bf16"], (b, ey)
    assert total_loads > w.max_num_loras  # the stream evicted and reloaded


def test_reset_slot_zeroes_one_slot():
    import torch
    w = workload()
    d = dims_of(w)
    dev = empty_stacks(w, d)
    for k in dev:
        dev[k].fill_(1.5)
    srg.lora_reset_slot(d, 2, dev)
    torch.cuda.synchronize()
    for k, t in dev.items():
        h = from_dev(t)
        assert not np.any(h[2]), k
        assert np.all(h[[0, 1, 3]] == 1.5), k
    with pytest.raises(srg.LoraError) as e:
        srg.lora_reset_slot(d, w.max_num_loras, dev)
    assert e.value.code == 1
