"""MLP targets (gate_proj, up_proj, down_proj): family shapes and the
family pack, bit-exact against the oracle; the oracle's family pack is
pinned to its attention pack (pinned on its own) and to closed forms."""

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg
from test_host_library import logical_from_tiled

MLP = synth.get_workload("mlp")


def mdims(w=MLP, dtype=None, R=None):
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, R or w.max_lora_rank,
                        w.max_num_loras, dtype or w.dtype, w.intermediate)


def small(dtype="bf16"):
    return synth.Workload(**{**MLP.__dict__, "name": "mlp", "hidden": 256, "n_heads": 4, "n_kv_heads": 2,
                             "head_dim": 64, "intermediate": 704, "dtype": dtype})


def test_mlp_family_shapes():
    d = mdims()
    assert srg.lora_family_shape(d, srg.FAMILY_GATE_UP) == (4096, 2, (14336, 14336), 28672)
    assert srg.lora_family_shape(d, srg.FAMILY_DOWN) == (14336, 1, (4096,), 4096)
    no_mlp = srg.LoraDims(4096, 32, 8, 128, 16, 8, "bf16")
    for fam in (srg.FAMILY_GATE_UP, srg.FAMILY_DOWN):
        with pytest.raises(srg.LoraError) as e:
            srg.lora_family_shape(no_mlp, fam)
        assert e.value.code == 1
    for bad in (-8, 12, 1 << 21):
        with pytest.raises(srg.LoraError):
            srg.lora_family_shape(srg.LoraDims(4096, 32, 8, 128, 16, 8, "bf16", bad), srg.FAMILY_QKV)


def slices_of(w, fam, weights, mask):
    names = ("gate", "up") if fam == srg.FAMILY_GATE_UP else ("down",)
    return [weights[p] if (mask >> i) & 1 else None for i, p in enumerate(names)]


def both(w, fam, rank, weights, mask, alpha=None, rs=None):
    alpha = w.lora_alpha if alpha is None else alpha
    rs = w.use_rslora if rs is None else rs
    d = mdims(w)
    in_f, n_s, widths, out_f = srg.lora_family_shape(d, fam)
    sl = slices_of(w, fam, weights, mask)
    got = srg.lora_pack_family(d, fam, rank, alpha, rs, True, sl)
    want = oracle.pack_family(in_f, widths, w.max_lora_rank, w.dtype, rank, alpha, rs, True, sl)
    got["A"] = logical_from_tiled(got["A"], n_s * w.max_lora_rank, in_f)
    return got, want


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_family_pack_bit_exact_vs_oracle(dtype, fam):
    w = small(dtype)
    for rank, mask, alpha, rs in ((16, 3, 16.0, False), (5, 1, 8.0, True), (9, 2, 3.0, False), (16, 0, 16.0, True)):
        mask &= 3 if fam == srg.FAMILY_GATE_UP else 1
        weights = synth.draw_mlp_adapter(w, 0, rank, rank)
        got, want = both(w, fam, rank, weights, mask, alpha, rs)
        for k in ("A", "B"):
            assert got[k].dtype == want[k].dtype and got[k].shape == want[k].shape
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (dtype, fam, rank, mask, k)


def test_full_size_mlp_pack_bit_exact():
    w = MLP
    ranks = synth.draw_ranks(w)
    weights = synth.draw_mlp_adapter(w, 0, 3, int(ranks[3]))
    for fam, mask in ((srg.FAMILY_GATE_UP, 3), (srg.FAMILY_DOWN, 1)):
        got, want = both(w, fam, int(ranks[3]), weights, mask)
        for k in ("A", "B"):
            assert np.array_equal(got[k], want[k]), (fam, k)


def test_family_pack_equals_attention_pack_for_qkv_and_o():
    """Both the library and the oracle: the family pack of QKV / O gives the
    bits of the attention pack (whose oracle side is pinned on its own)."""
    w = synth.get_workload("decode")
    d = srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.max_num_loras, w.dtype)
    weights = synth.draw_adapter(w, 0, 2, 8)
    att = srg.lora_pack_adapter(d, 8, w.lora_alpha, w.use_rslora, True, "qkvo", weights)
    oatt = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.dtype,
                               8, w.lora_alpha, w.use_rslora, True, "qkvo", weights)
    for fam, keys, names in ((srg.FAMILY_QKV, ("A_qkv", "B_qkv"), "qkv"), (srg.FAMILY_O, ("A_o", "B_o"), "o")):
        sl = [weights[p] for p in names]
        lib = srg.lora_pack_family(d, fam, 8, w.lora_alpha, w.use_rslora, True, sl)
        assert np.array_equal(lib["A"], att[keys[0]]) and np.array_equal(lib["B"], att[keys[1]])
        in_f, n_s, widths, _ = srg.lora_family_shape(d, fam)
        orc = oracle.pack_family(in_f, widths, w.max_lora_rank, w.dtype, 8, w.lora_alpha, w.use_rslora, True, sl)
        assert np.array_equal(orc["A"], oatt[keys[0]]) and np.array_equal(orc["B"], oatt[keys[1]])


def test_oracle_family_pack_closed_forms():
    """Power-of-two scale: packed B = bf16(B) * scale exactly; A rows past the
    rank and slices not targeted are zero; an untargeted slice leaves its
    neighbour's bits unchanged."""
    w = small()
    rank = 4
    weights = synth.draw_mlp_adapter(w, 1, 0, rank)
    in_f, widths = w.hidden, [w.intermediate, w.intermediate]
    full = oracle.pack_family(in_f, widths, 16, "bf16", rank, 8.0, False, True, [weights["gate"], weights["up"]])
    only_up = oracle.pack_family(in_f, widths, 16, "bf16", rank, 8.0, False, True, [None, weights["up"]])
    bf = lambda a: oracle.bf16_to_f64(a)
    # scale = 8 / 4 = 2 (exact): bf16 of (B * 2) equals 2 * bf16(B)
    gate_b = bf(full["B"][:w.intermediate, :rank])
    assert np.array_equal(gate_b, 2.0 * oracle.bf16_to_f64(oracle.bf16_round(weights["gate"][1])))
    assert not np.any(full["A"][rank:16]) and not np.any(full["B"][:, rank:])
    assert not np.any(only_up["A"][:16]) and not np.any(only_up["B"][:w.intermediate])
    assert np.array_equal(only_up["A"][16:], full["A"][16:]) and np.array_equal(only_up["B"][w.intermediate:],
                                                                              full["B"][w.intermediate:])


@pytest.mark.parametrize("kw,code", [(dict(bias_none=False), 2), (dict(rank=0), 2), (dict(rank=17), 2),
                                     (dict(mask_extra=True), 2)])
def test_family_pack_errors(kw, code):
    w = small()
    d = mdims(w)
    rank = kw.get("rank", 4)
    weights = synth.draw_mlp_adapter(w, 0, 0, max(rank, 1))
    sl = [weights["down"]]
    if kw.get("mask_extra"):
        sl = [weights["down"], weights["down"]]
        with pytest.raises(ValueError):
            srg.lora_pack_family(d, srg.FAMILY_DOWN, rank, 8.0, False, True, sl)
        return
    with pytest.raises(srg.LoraError) as e:
        srg.lora_pack_family(d, srg.FAMILY_DOWN, rank, 8.0, False, kw.get("bias_none", True), sl)
    assert e.value.code == code
    with pytest.raises(oracle.OracleError) as e2:
        oracle.pack_family(w.intermediate, [w.hidden], 16, "bf16", rank, 8.0, False, kw.get("bias_none", True), sl)
    assert e2.value.code == code
