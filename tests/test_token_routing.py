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
    header declares."""
    names = [f[0] for f in _lib._LoraRouting._fields_]
    assert names[-2:] == ["token_rows", "num_rows"]
    assert ctypes.sizeof(_lib._LoraRouting) == 64


# ------------------------------------------------------------------ C-ABI argument checks (no GPU)
# Device calls check every argument before any launch, so these calls return
# their error without touching the (fake, never dereferenced) device pointers.
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _llama_dims():
    return srg.LoraDims(4096, 32, 8, 128, 16, 8, "bf16").c()


def _token_routing_struct(num_rows, end=4):
    ids = np.array([0, 1], np.int32)
    offs = np.array([0, end - 1, end], np.int32)
    r = _lib._LoraRouting()
    r.lora_ids, r.grouped_offsets = FAKE, FAKE
    r.num_groups, r.end = 2, end
    r.host_lora_ids, r.host_grouped_offsets = ids.ctypes.data, offs.ctypes.data
    r.token_rows, r.num_rows = FAKE, num_rows
    return r, (ids, offs)


def _delta(lib, dims, fam, r, ldx, ldy, ws=FAKE, ws_bytes=1 << 30, path=srg.PATH_AUTO, opts=None):
    return lib.lora_sgmv_delta(ctypes.byref(dims), fam, FAKE, ldx, FAKE, FAKE, None, ctypes.byref(r), FAKE, ldy,
                               ws, ws_bytes, path, opts, None)


@pytest.mark.parametrize("gib", [2.0, 2.5, 3.0, 3.999])
def test_per_token_buffers_past_2gib_rejected_before_launch(gib):
    """Under per-token routing one buffer resource spans all num_rows rows of
    x or y, and masked lanes address offset 2^31: (num_rows + 1) x row bytes
    must stay within 2^31, or a masked lane would read and write back a real
    row.  Row counts whose y spans the 2-4 GiB band are rejected with
    LORA_ERR_INVALID_ARGUMENT on every device call."""
    lib = _lib._load()
    d = _llama_dims()
    for fam, width in ((srg.FAMILY_QKV, 6144), (srg.FAMILY_O, 4096)):
        row_bytes = width * 2
        num_rows = int(gib * 2 ** 30) // row_bytes
        r, keep = _token_routing_struct(num_rows)
        in_w = 4096
        assert _delta(lib, d, fam, r, in_w, width) == 1
        assert _delta(lib, d, fam, r, in_w, width, path=srg.PATH_FUSED) == 1
        assert lib.lora_sgmv_expand(ctypes.byref(d), fam, FAKE, FAKE, None, ctypes.byref(r), FAKE, width,
                                    srg.PATH_AUTO, None) == 1
        # the shrink's x (4096 wide) in the same band
        rx, keep2 = _token_routing_struct(int(gib * 2 ** 30) // (in_w * 2))
        assert lib.lora_sgmv_shrink(ctypes.byref(d), fam, FAKE, in_w, FAKE, ctypes.byref(rx), FAKE, FAKE,
                                    1 << 30, srg.PATH_AUTO, None) == 1


def test_per_token_bound_is_exactly_2gib():
    """The largest accepted y is (num_rows + 1) x row bytes = 2^31 exactly; one
    row more is rejected.  (Only the rejection is called here: an accepted
    call would launch.)"""
    lib = _lib._load()
    d = _llama_dims()
    row_bytes = 4096 * 2  # o_proj output rows
    ok_rows = 2 ** 31 // row_bytes - 1
    r, keep = _token_routing_struct(ok_rows + 1)
    assert lib.lora_sgmv_expand(ctypes.byref(d), srg.FAMILY_O, FAKE, FAKE, None, ctypes.byref(r), FAKE, 4096,
                                srg.PATH_AUTO, None) == 1


@pytest.mark.parametrize("tile", [16, 48, 96, 160, 1024, -32])
def test_bad_fused_feature_tile_option_rejected(tile):
    """fused_feature_tile must be 0 or a power of two in [32, 512]."""
    lib = _lib._load()
    d = _llama_dims()
    r, keep = _token_routing_struct(8)
    opts = srg.LoraOptions(fused_feature_tile=tile).c()
    assert _delta(lib, d, srg.FAMILY_QKV, r, 4096, 6144, path=srg.PATH_FUSED, opts=ctypes.byref(opts)) == 1


def test_two_kernel_delta_needs_a_workspace():
    """A NULL workspace is an argument error where the two-kernel path runs
    (here: a 300-token group, longer than the one-kernel path takes), and a
    short one is a capacity error."""
    lib = _lib._load()
    d = _llama_dims()
    ids = np.array([0], np.int32)
    offs = np.array([0, 300], np.int32)
    r = _lib._LoraRouting()
    r.lora_ids, r.grouped_offsets, r.num_groups, r.end = FAKE, FAKE, 1, 300
    r.host_lora_ids, r.host_grouped_offsets = ids.ctypes.data, offs.ctypes.data
    assert _delta(lib, d, srg.FAMILY_QKV, r, 4096, 6144, ws=None, ws_bytes=0) == 1
    assert _delta(lib, d, srg.FAMILY_QKV, r, 4096, 6144, ws=FAKE, ws_bytes=16) == 4
