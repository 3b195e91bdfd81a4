"""LoRA bias: the oracle's bias pack and bias term pinned to closed forms
and to a PEFT-style forward written with torch's linear layers; the
library's lora_pack_bias bit-exact against the oracle; argument errors."""

import ctypes

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg
from segmented_rank_gemv_amd import _lib

TINY = synth.get_workload("tiny")
MLP = synth.get_workload("mlp")


def tdims(w, dtype=None):
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                        w.max_num_loras, dtype or w.dtype, w.intermediate)


def small_mlp(dtype):
    return synth.Workload(**{**MLP.__dict__, "hidden": 256, "n_heads": 4, "n_kv_heads": 2,
                             "head_dim": 64, "intermediate": 704, "dtype": dtype})


# ----------------------------------------------------------------------------- oracle pins
def test_oracle_pack_bias_rounds_to_nearest_even():
    """bf16 keeps 8 significant bits: 1 + 2^-8 is halfway between 1 and
    1 + 2^-7 and goes to the even 1.0 (0x3F80); 1 + 3 2^-8 is halfway
    between 1 + 2^-7 (odd) and 1 + 2^-6 and goes to 0x3F82; -2.5 and 0 are
    exact (0xC020, 0)."""
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 0.0], np.float32)
    got = oracle.pack_bias([4], "bf16", [vals])
    assert got.dtype == np.uint16
    assert got.tolist() == [0x3F80, 0x3F82, 0xC020, 0x0000]
    f = oracle.pack_bias([4], "f32", [vals])
    assert f.dtype == np.float32 and np.array_equal(f, vals)


def test_oracle_pack_bias_slice_order_and_missing_slices():
    """Slices land at their offsets in the fused output (q, then k, then v);
    a slice without a bias is zero."""
    got = oracle.pack_bias([8, 4, 4], "f32", [np.full(8, 1.0), None, np.full(4, 3.0)])
    assert got.tolist() == [1.0] * 8 + [0.0] * 4 + [3.0] * 4
    assert oracle.pack_bias([2, 2], "bf16", [None, None]).tolist() == [0, 0, 0, 0]
    with pytest.raises(oracle.OracleError):
        oracle.pack_bias([4, 4], "f32", [np.zeros(4)])


def _peft_forward(x, y_in, A, B, b, scale):
    """y_in + scale * lora_B(lora_A(x)) + b, with lora_A and lora_B as
    torch linear layers (float64)."""
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    h = F.linear(t(x), t(A))
    return (t(y_in) + F.linear(h, t(B) * scale) + t(b)).numpy()


@pytest.mark.parametrize("alpha_is_rank", [True, False])
def test_oracle_bias_term_against_linear_layers(alpha_is_rank):
    """Per request, the oracle's y equals the adapter written as torch linear
    layers with the bias added after the scaled B (fp32 stacks, so the
    packing is exact when the scale is 1; otherwise to fp32 rounding of
    the scaled B).  Base requests keep y_in."""
    w = TINY
    lengths = np.array([3, 0, 5, 2, 4], np.int64)
    slots = np.array([1, 0, -1, 1, 0], np.int32)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    acts = synth.draw_activations(w, 0, T)
    rank = 4
    alpha = float(rank) if alpha_is_rank else 8.0
    R = w.max_lora_rank
    widths = [w.nq, w.nkv, w.nkv]
    A_st, B_st, b_st, raw = [], [], [], []
    for s in range(w.max_num_loras):
        ad = synth.draw_adapter(w, 0, s, rank)
        bias = synth.draw_bias(w, 0, s)
        pk = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, R, "f32", rank, alpha,
                                 False, True, "qkvo", ad)
        A_st.append(pk["A_qkv"])
        B_st.append(pk["B_qkv"])
        b_st.append(oracle.pack_bias(widths, "f32", [bias["q"], bias["k"], bias["v"]]))
        raw.append((ad, bias))
    A_st, B_st, b_st = np.stack(A_st), np.stack(B_st), np.stack(b_st)
    ref = oracle.reference_family(acts["x_qkv"], acts["y_qkv"], offs, slots, A_st, B_st, widths, R, "f32",
                                  bias_stack=b_st)
    scale = alpha / rank
    tol = 1e-12 if alpha_is_rank else 1e-6
    for i, (rows, y, u) in ref.items():
        a = int(offs[i])
        yin = acts["y_qkv"][a + rows]
        if slots[i] < 0:
            assert u is None and np.array_equal(y, yin.astype(np.float64))
            continue
        if len(rows) == 0:
            continue
        ad, bias = raw[slots[i]]
        parts = []
        for p in ("q", "k", "v"):
            parts.append(_peft_forward(acts["x_qkv"][a + rows], np.zeros((len(rows), len(bias[p]))),
                                       ad[p][0], ad[p][1], bias[p], scale))
        want = yin.astype(np.float64) + np.concatenate(parts, axis=1)
        assert np.max(np.abs(y - want)) <= tol * max(1.0, np.max(np.abs(want)))


def test_oracle_bias_with_zero_B_is_exactly_the_bias():
    """With B = 0 the delta of a LoRA request is its slot's bias, exactly."""
    w = TINY
    lengths = np.array([2, 3], np.int64)
    slots = np.array([1, 0], np.int32)
    offs = np.array([0, 2, 5], np.int64)
    acts = synth.draw_activations(w, 0, 5)
    R = w.max_lora_rank
    A = np.stack([oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, R, "f32", 4, 8.0, False,
                                      True, "o", synth.draw_adapter(w, 0, s, 4))["A_o"]
                  for s in range(w.max_num_loras)])
    B = np.zeros((w.max_num_loras, w.hidden, R), np.float32)
    bias = np.stack([oracle.pack_bias([w.hidden], "f32", [synth.draw_bias(w, 0, s)["o"]])
                     for s in range(w.max_num_loras)])
    ref = oracle.reference_family(acts["x_o"], acts["y_o"], offs, slots, A, B, [w.hidden], R, "f32",
                                  bias_stack=bias)
    for i, (rows, y, _) in ref.items():
        a = int(offs[i])
        assert np.array_equal(y - acts["y_o"][a + rows].astype(np.float64),
                              np.broadcast_to(bias[slots[i]].astype(np.float64), y.shape))


# ----------------------------------------------------------------------------- library vs oracle
CASES = [("qkv", srg.FAMILY_QKV, ("q", "k", "v")), ("o", srg.FAMILY_O, ("o",)),
         ("gate_up", srg.FAMILY_GATE_UP, ("gate", "up")), ("down", srg.FAMILY_DOWN, ("down",))]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_library_pack_bias_bit_exact_vs_oracle(case, dtype):
    _, fam, projs = case
    w = small_mlp(dtype)
    d = tdims(w)
    widths = srg.lora_family_shape(d, fam)[2]
    for slot in range(3):
        bias = synth.draw_bias(w, 0, slot, projs)
        for mask in range(1 << len(projs)):
            sl = [bias[p] if (mask >> i) & 1 else None for i, p in enumerate(projs)]
            got = srg.lora_pack_bias(d, fam, sl)
            want = oracle.pack_bias(widths, dtype, sl)
            assert got.dtype == want.dtype and np.array_equal(got.view(np.uint8), want.view(np.uint8)), \
                (case[0], dtype, slot, mask)


def test_library_pack_bias_errors():
    d = tdims(TINY, "bf16")
    lib = _lib._load()
    out = np.zeros(TINY.n_qkv, np.uint16)
    b = np.zeros(TINY.nq, np.float32)
    ptrs = (ctypes.c_void_p * 4)(b.ctypes.data, b.ctypes.data, b.ctypes.data, b.ctypes.data)
    dc = d.c()
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    # a mask bit past the family's three slices
    assert lib.lora_pack_bias(ctypes.byref(dc), srg.FAMILY_QKV, 0b1000, P(ptrs), out.ctypes.data) == 2
    # a set bit without a slice, a missing output, an unknown family
    assert lib.lora_pack_bias(ctypes.byref(dc), srg.FAMILY_QKV, 0b1, None, out.ctypes.data) == 1
    assert lib.lora_pack_bias(ctypes.byref(dc), srg.FAMILY_QKV, 0b1, P(ptrs), None) == 1
    assert lib.lora_pack_bias(ctypes.byref(dc), 9, 0b1, P(ptrs), out.ctypes.data) == 1
    # MLP families need an intermediate size
    assert lib.lora_pack_bias(ctypes.byref(dc), srg.FAMILY_DOWN, 0, None, out.ctypes.data) == 1
    with pytest.raises(ValueError):
        srg.lora_pack_bias(d, srg.FAMILY_QKV, [b, None])
    with pytest.raises(ValueError):
        srg.lora_pack_bias(d, srg.FAMILY_O, [np.zeros(3, np.float32)])
    # no slices set: zeros
    assert not srg.lora_pack_bias(d, srg.FAMILY_QKV, [None, None, None]).any()
