"""Host-side checks of the C-ABI library (no GPU needed): the library loads and
exports every declared entry point, and its packing and routing match the
oracle bit for bit."""

import os
import re

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_sgmv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    import ctypes
    lib = ctypes.CDLL(srg.library_path())
    names = declared_functions()
    assert {"lora_pack_adapter", "lora_build_routing", "lora_sgmv_shrink", "lora_sgmv_expand"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    assert srg.lora_abi_version() == 9
    assert srg.lora_status_string(0) == "LORA_OK"
    assert srg.lora_status_string(3) == "LORA_ERR_SLOT_OUT_OF_RANGE"
    assert srg.lora_status_string(99) == "LORA_ERR_UNKNOWN"


def test_defaults_are_the_pages_lora_config_defaults():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "lora_config_defaults.json")))
    d = srg.LoraDims(hidden=128, n_heads=8, n_kv_heads=8, head_dim=16)
    assert d.max_lora_rank == g["printed_by_page"]["max_lora_rank"]
    assert d.max_num_loras == g["printed_by_page"]["max_num_loras"]


def dims_of(w):
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                        w.max_num_loras, w.dtype)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_family_shapes(name):
    w = synth.get_workload(name)
    d = dims_of(w)
    assert srg.lora_family_shape(d, srg.FAMILY_QKV) == (w.hidden, 3, (w.nq, w.nkv, w.nkv), w.n_qkv)
    assert srg.lora_family_shape(d, srg.FAMILY_O) == (w.nq, 1, (w.hidden,), w.hidden)


def logical_from_tiled(a, rows, K):
    """The device's A layout, read back by its index formula: element (r, k)
    sits at ((r // 16) * (K / 8) + k // 8) * 128 + (r % 16) * 8 + k % 8 and
    the rows added up to a multiple of 16 are zero."""
    flat = a.reshape(-1)
    nb = (rows + 15) // 16
    assert flat.size == nb * 16 * K
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    idx = ((r // 16) * (K // 8) + k // 8) * 128 + (r % 16) * 8 + k % 8
    rest = np.ones(flat.size, bool)
    rest[idx.reshape(-1)] = False
    assert not np.any(flat[rest]), "padding rows of the tiled A layout must be zero"
    return flat[idx]


def _pack_both(w, rank, weights, targets="qkvo", alpha=None, rs=None, bias_none=True, mask=None):
    """Library pack (A converted from the device layout to [rows, K]) and
    oracle pack of the same adapter."""
    alpha = w.lora_alpha if alpha is None else alpha
    rs = w.use_rslora if rs is None else rs
    got = srg.lora_pack_adapter(dims_of(w), rank, alpha, rs, bias_none, targets, weights, mask)
    want = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                               w.dtype, rank, alpha, rs, bias_none, targets, weights, mask)
    R = w.max_lora_rank
    got = dict(got)
    got["A_qkv"] = logical_from_tiled(got["A_qkv"], 3 * R, w.hidden)
    got["A_o"] = logical_from_tiled(got["A_o"], R, w.nq)
    return got, want


def test_tile_helpers_follow_the_layout_formula():
    rng = np.random.default_rng(3)
    for rows, K in ((48, 64), (24, 40), (16, 8), (8, 16), (96, 136)):
        a = rng.standard_normal((rows, K)).astype(np.float32)
        t = srg.tile_a(a)
        assert t.shape == srg.a_tiled_shape(rows, K)
        assert np.array_equal(logical_from_tiled(t, rows, K), a)
        assert np.array_equal(srg.untile_a(t, rows), a)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_pack_bit_exact_vs_oracle(name):
    w = synth.get_workload(name)
    ranks = synth.draw_ranks(w)
    slots = [0, w.max_num_loras - 1] if w.max_num_loras > 1 else [0]
    for layer in sorted({0, w.n_layers - 1}):
        for s in slots:
            weights = synth.draw_adapter(w, layer, s, int(ranks[s]))
            got, want = _pack_both(w, int(ranks[s]), weights)
            for k in want:
                assert got[k].dtype == want[k].dtype and got[k].shape == want[k].shape
                assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (name, layer, s, k)


@pytest.mark.parametrize("targets", ["qv", "o", "k", "qkvo", ""])
@pytest.mark.parametrize("rs", [False, True])
def test_pack_targets_and_scales_bit_exact(targets, rs):
    w = synth.get_workload("tiny")
    for dtype in ("f32", "bf16"):
        wd = synth.Workload(**{**w.__dict__, "dtype": dtype})
        weights = synth.draw_adapter(wd, 0, 1, 7 if not rs else 5)
        for alpha in (8.0, 3.0, 16.0):
            got, want = _pack_both(wd, 7 if not rs else 5, weights, targets, alpha, rs)
            for k in want:
                assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (targets, rs, dtype, k)


def test_pack_rounding_edge_values_bit_exact():
    w = synth.Workload(**{**synth.get_workload("tiny").__dict__, "dtype": "bf16"})
    rng = np.random.default_rng(1)
    r = 4
    # values near bf16 ties, subnormals and large magnitudes
    hi = rng.integers(0, 1 << 16, size=(r, w.hidden), dtype=np.uint32) << np.uint32(16)
    lo = rng.choice(np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32), size=hi.shape)
    A = (hi | lo).view(np.float32)
    A = np.where(np.isfinite(A), A, np.float32(1.0)).astype(np.float32)
    weights = synth.draw_adapter(w, 0, 0, r)
    weights["q"] = (A, weights["q"][1])
    weights["k"] = (weights["k"][0], weights["k"][1] * np.float32(3e37))
    got, want = _pack_both(w, r, weights, alpha=16.0, rs=True)
    for k in want:
        assert np.array_equal(got[k], want[k]), k


@pytest.mark.parametrize("kw,code", [
    (dict(bias_none=False), 2), (dict(rank=0), 2), (dict(rank=17), 2), (dict(mask=0x10 | 1), 2),
])
def test_pack_error_codes_match_oracle(kw, code):
    w = synth.get_workload("tiny")
    rank = kw.get("rank", 4)
    weights = synth.draw_adapter(w, 0, 0, max(rank, 1))
    with pytest.raises(srg.LoraError) as e1:
        srg.lora_pack_adapter(dims_of(w), rank, 8.0, False, kw.get("bias_none", True), "qkvo",
                              weights, kw.get("mask"))
    with pytest.raises(oracle.OracleError) as e2:
        oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.dtype,
                            rank, 8.0, False, kw.get("bias_none", True), "qkvo", weights, kw.get("mask"))
    assert e1.value.code == e2.value.code == code
    assert isinstance(e1.value, ValueError)


def test_pack_bad_dims_rejected():
    w = synth.get_workload("tiny")
    weights = synth.draw_adapter(w, 0, 0, 4)
    for bad in (dict(hidden=0), dict(n_heads=3, head_dim=3), dict(max_lora_rank=12), dict(dtype="f32", max_lora_rank=256)):
        d = srg.LoraDims(**{**dims_of(w).__dict__, **bad})
        with pytest.raises(srg.LoraError) as e:
            srg.lora_pack_adapter(d, 4, 8.0, False, True, "qkvo", weights)
        assert e.value.code == 1


def _route_both(slots, lengths, L):
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return srg.lora_build_routing(slots, offs, L), oracle.route(slots, offs, L)


def _same_routing(a, b):
    for k in ("perm", "sorted_offsets", "lora_ids", "grouped_offsets"):
        assert np.array_equal(a[k], b[k]), k
    assert a["num_groups"] == b["num_groups"] and a["end"] == b["end"]


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_routing_bit_exact_vs_oracle(name):
    w = synth.get_workload(name)
    lengths, slots = synth.draw_requests(w)
    got, want = _route_both(slots, lengths, w.max_num_loras)
    _same_routing(got, want)


def test_routing_random_bit_exact_vs_oracle():
    rng = np.random.default_rng(21)
    for _ in range(300):
        n = int(rng.integers(0, 200))
        L = int(rng.integers(1, 64))
        slots = rng.integers(-1, L, size=n).astype(np.int32)
        lengths = rng.integers(0, 30, size=n)
        got, want = _route_both(slots, lengths, L)
        _same_routing(got, want)


@pytest.mark.parametrize("slots,offsets,code", [
    ([0, 2], [0, 1, 2], 3), ([0, -2], [0, 1, 2], 3), ([0, 1], [0, 3, 2], 1), ([0, 1], [1, 3, 4], 1),
])
def test_routing_error_codes_match_oracle(slots, offsets, code):
    s = np.array(slots, np.int32)
    o = np.array(offsets, np.int64)
    with pytest.raises(srg.LoraError) as e1:
        srg.lora_build_routing(s, o, 2)
    with pytest.raises(oracle.OracleError) as e2:
        oracle.route(s, o, 2)
    assert e1.value.code == e2.value.code == code


def test_routing_token_count_must_fit_int32():
    s = np.array([0, 0], np.int32)
    o = np.array([0, 2 ** 30, 2 ** 31 + 5], np.int64)
    with pytest.raises(srg.LoraError) as e:
        srg.lora_build_routing(s, o, 1)
    assert e.value.code == 1


@pytest.mark.parametrize("name", ["decode", "prefill", "mixed", "stack"])
def test_workspace_bound_covers_every_batch_size(name):
    w = synth.get_workload(name)
    d = dims_of(w)
    for fam in (srg.FAMILY_QKV, srg.FAMILY_O):
        prev = 0
        for mt in (1, 63, 64, 65, 192, 1024, 4096):
            b = srg.lora_sgmv_workspace_bytes(d, fam, mt)
            assert b >= prev
            prev = b
    assert srg.lora_sgmv_workspace_bytes(d, srg.FAMILY_QKV, 0) == 0
