"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value a
page prints, a closed form, a library routine (numpy matmul, torch's bf16
cast), brute force on tiny inputs, or an invariant the method implies.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import OracleError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_adapter(rng, r, hidden, nq, nkv, dtype=np.float32):
    shapes = {"q": (hidden, nq), "k": (hidden, nkv), "v": (hidden, nkv), "o": (nq, hidden)}
    return {p: (rng.standard_normal((r, fi)).astype(dtype), rng.standard_normal((fo, r)).astype(dtype))
            for p, (fi, fo) in shapes.items()}


# --------------------------------------------------------------------------- scaling
def test_scaling_vllm_worked_example():
    g = golden("vllm_scaling_example.json")["printed_by_page"]
    assert oracle.scaling(g["lora_alpha"], g["r"], False) == g["q_proj"]["scaling"]


def test_scaling_max_docstring_example():
    g = golden("max_docstring_adapter.json")
    p = g["printed_by_page"]
    assert oracle.scaling(p["lora_alpha"], p["rank"], False) == g["derived_expectation"]["scaling"]


def test_scaling_rslora_closed_forms():
    # alpha / sqrt(r) at perfect squares, and 16/sqrt(32) = 2*sqrt(2)
    assert oracle.scaling(16, 64, True) == 2.0
    assert oracle.scaling(32, 16, True) == 8.0
    assert oracle.scaling(9, 9, True) == 3.0
    assert abs(oracle.scaling(16, 32, True) - 2.0 * math.sqrt(2.0)) <= 1e-15   # 2 ulp
    # the fp32 scale that packing multiplies by
    assert np.float32(oracle.scaling(16, 32, True)) == np.float32(2.8284271247461903)
    # plain alpha / r is not the rsLoRA value
    assert oracle.scaling(16, 32, False) == 0.5


# --------------------------------------------------------------------------- bf16 cast
def test_bf16_round_hand_cases():
    f = np.float32
    cases = [
        (f(1.0), 0x3F80),
        (f(-2.0), 0xC000),
        (f(0.0), 0x0000),
        (f(-0.0), 0x8000),
        (f(1.0 + 2.0 ** -8), 0x3F80),             # tie, even neighbour below
        (f(1.0 + 3 * 2.0 ** -8), 0x3F82),         # tie, even neighbour above
        (f(1.0 + 2.0 ** -8 + 2.0 ** -20), 0x3F81),  # just above the tie
        (f(np.inf), 0x7F80),
        (f(-np.inf), 0xFF80),
    ]
    for v, want in cases:
        got = int(oracle.bf16_round(np.array([v], dtype=np.float32))[0])
        assert got == want, (v, hex(got), hex(want))


def _special_f32():
    rng = np.random.default_rng(7)
    hi = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    f = bits.view(np.float32)
    return f[~np.isnan(f)]


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(20000) * 3e37).astype(np.float32),    # large magnitudes
        _special_f32(),
        np.array([3.3961e38, 3.3963e38, 3.4028e38, -3.4028e38, 1e-45, -1e-45], dtype=np.float32),
    ])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(vals)
    assert np.array_equal(got, want)


def test_bf16_decoder_fixed_values():
    """The oracle's bf16 decoder (the inverse of the pack's final cast,
    [MAX-lora] 加载时的处理管线) on patterns whose values follow from the
    bf16 format by hand: sign, 8 exponent bits (bias 127), 7 fraction bits."""
    pats = np.array([0x3F80, 0xC020, 0x8000, 0x0000, 0x0001, 0x8001, 0x0080, 0x7F7F, 0x7F80, 0xFF80,
                     0x4049, 0x3E80, 0x3F81], dtype=np.uint16)
    want = [1.0, -2.5, -0.0, 0.0, 2.0 ** -133, -(2.0 ** -133), 2.0 ** -126, (2 - 2 ** -7) * 2.0 ** 127,
            math.inf, -math.inf, 3.140625, 0.25, 1 + 2 ** -7]
    got = oracle.bf16_to_f64(pats)
    assert got.dtype == np.float64
    for g, w_, bits in zip(got, want, pats):
        assert g == w_, hex(bits)
        assert math.copysign(1.0, g) == math.copysign(1.0, w_), hex(bits)
    nan = oracle.bf16_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], np.uint16))
    assert np.all(np.isnan(nan))


def test_bf16_decoder_every_pattern_matches_torch():
    """All 65 536 bf16 patterns decode to the value torch's bfloat16 -> float64
    conversion gives (a library routine); NaN patterns stay NaN."""
    torch = pytest.importorskip("torch")
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(pats)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), want[~nan].view(np.uint64))


def test_bf16_decoder_inverts_the_rounding_on_random_values():
    """decode(round(v)) is the bf16 value nearest v: within half an ulp of
    v (2^-9 relative), and torch's cast of v to bfloat16 gives the same
    number, on 10^5 draws across magnitudes."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    dec = oracle.bf16_to_f64(oracle.bf16_round(v))
    assert np.all(np.abs(dec - v.astype(np.float64)) <= np.abs(v.astype(np.float64)) * 2.0 ** -8)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(dec, ref)


def test_stack_to_f64_by_dtype():
    """bf16 stacks decode their patterns; fp32 stacks widen exactly."""
    pats = np.array([[0x3F80, 0xC020]], np.uint16)
    assert oracle.stack_to_f64(pats, "bf16").tolist() == [[1.0, -2.5]]
    f = np.array([1.5, -3.0e-40, 3.4028235e38], np.float32)
    got = oracle.stack_to_f64(f, "f32")
    assert got.dtype == np.float64 and got.tolist() == [float(v) for v in f]


def test_bf16_round_nan_stays_nan():
    bits = np.array([0x7FC00000, 0x7F800001, 0xFFA00000], dtype=np.uint32)
    got = oracle.bf16_round(bits.view(np.float32))
    back = oracle.bf16_to_f64(got)
    assert np.all(np.isnan(back))


# --------------------------------------------------------------------------- pack
def test_pack_docstring_example_shapes_and_zeros():
    g = golden("max_docstring_adapter.json")
    p, d = g["printed_by_page"], g["derived_expectation"]
    H = p["n_heads"] * p["head_dim"]
    KV = p["n_kv_heads"] * p["head_dim"]
    r = p["rank"]
    weights = {
        "q": (np.zeros((r, H), np.float32), np.zeros((H, r), np.float32)),
        "k": (np.zeros((r, H), np.float32), np.zeros((KV, r), np.float32)),
        "v": (np.zeros((r, H), np.float32), np.zeros((KV, r), np.float32)),
        "o": (np.zeros((r, H), np.float32), np.zeros((H, r), np.float32)),
    }
    out = oracle.pack_adapter(H, p["n_heads"], p["n_kv_heads"], p["head_dim"], p["max_lora_rank"],
                              "bf16", r, p["lora_alpha"], False, True, "qkvo", weights)
    for key in ("A_qkv", "B_qkv", "A_o", "B_o"):
        assert list(out[key].shape) == d[key + "_shape"]
        assert not np.any(out[key])


def _dense_delta(weights, scale, x_qkv, x_o):
    """h - W0 x per projection from the unpacked PEFT matrices (numpy matmul)."""
    d = {}
    for p in "qkv":
        A, B = weights[p]
        d[p] = scale * (x_qkv.astype(np.float64) @ A.T.astype(np.float64)) @ B.T.astype(np.float64)
    A, B = weights["o"]
    d["o"] = scale * (x_o.astype(np.float64) @ A.T.astype(np.float64)) @ B.T.astype(np.float64)
    return d


@pytest.mark.parametrize("R", [4, 8, 16])
@pytest.mark.parametrize("alpha,rs", [(8.0, False), (16.0, False), (32.0, True)])
def test_pack_then_delta_equals_dense_lora(R, alpha, rs):
    """Per projection, the fused+padded+scaled slot gives exactly the LoRA
    forward h = W0 x + scaling * B A x of the raw PEFT matrices (fp32 stack,
    power-of-two scales so the packed B is exact)."""
    rng = np.random.default_rng(11 + R)
    r, H, nh, nkv_h, hd = 4, 24, 3, 1, 8
    nq, nkv = nh * hd, nkv_h * hd
    weights = rand_adapter(rng, r, H, nq, nkv)
    scale = oracle.scaling(alpha, r, rs)
    assert scale in (2.0, 4.0, 16.0)
    pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "f32", r, alpha, rs, True, "qkvo", weights)
    n = 5
    x_qkv = rng.standard_normal((n, H))
    x_o = rng.standard_normal((n, nq))
    y_qkv = rng.standard_normal((n, nq + 2 * nkv))
    y_o = rng.standard_normal((n, H))
    _, yq = oracle.delta(x_qkv, pk["A_qkv"], pk["B_qkv"], y_qkv, [nq, nkv, nkv], R)
    _, yo = oracle.delta(x_o, pk["A_o"], pk["B_o"], y_o, [H], R)
    dense = _dense_delta(weights, scale, x_qkv, x_o)
    want_qkv = y_qkv + np.concatenate([dense["q"], dense["k"], dense["v"]], axis=1)
    np.testing.assert_allclose(yq, want_qkv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(yo, y_o + dense["o"], rtol=1e-12, atol=1e-12)


def test_pack_bf16_cast_matches_torch_with_irrational_scale():
    """rsLoRA r=32, alpha=16: B is multiplied by fp32(16/sqrt(32)) in fp32 and
    then rounded to bf16; A is rounded to bf16.  torch performs the same two
    library operations."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    r, R, H, nh, nkv_h, hd = 32, 32, 64, 4, 2, 16
    nq, nkv = nh * hd, nkv_h * hd
    weights = rand_adapter(rng, r, H, nq, nkv)
    pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "bf16", r, 16.0, True, True, "qkvo", weights)
    s32 = torch.tensor(16.0 / math.sqrt(32.0), dtype=torch.float32)

    def tb(a):
        return a.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    A_want = np.concatenate([tb(torch.from_numpy(weights[p][0])) for p in "qkv"], axis=0)
    B_want = np.concatenate([tb(torch.from_numpy(weights[p][1]) * s32) for p in "qkv"], axis=0)
    assert np.array_equal(pk["A_qkv"], A_want)
    assert np.array_equal(pk["B_qkv"], B_want)
    assert np.array_equal(pk["A_o"], tb(torch.from_numpy(weights["o"][0])))
    assert np.array_equal(pk["B_o"], tb(torch.from_numpy(weights["o"][1]) * s32))


def test_pack_missing_projection_gives_zero_slice():
    rng = np.random.default_rng(6)
    r, R, H, nh, nkv_h, hd = 4, 8, 16, 2, 1, 8
    nq, nkv = nh * hd, nkv_h * hd
    weights = rand_adapter(rng, r, H, nq, nkv)
    pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "f32", r, 8.0, False, True, "qv", weights)
    x = rng.standard_normal((3, H))
    y = rng.standard_normal((3, nq + 2 * nkv))
    _, yo = oracle.delta(x, pk["A_qkv"], pk["B_qkv"], y, [nq, nkv, nkv], R)
    assert np.array_equal(yo[:, nq:nq + nkv], y[:, nq:nq + nkv])   # k untouched
    assert not np.array_equal(yo[:, :nq], y[:, :nq])                 # q moved
    assert not np.array_equal(yo[:, nq + nkv:], y[:, nq + nkv:])     # v moved
    assert not np.any(pk["A_o"]) and not np.any(pk["B_o"])


def test_pack_padding_invariance():
    rng = np.random.default_rng(8)
    r, H, nh, nkv_h, hd = 4, 32, 2, 1, 16
    nq, nkv = nh * hd, nkv_h * hd
    weights = rand_adapter(rng, r, H, nq, nkv)
    x = rng.standard_normal((4, H))
    y = rng.standard_normal((4, nq + 2 * nkv))
    outs = []
    for R in (4, 16, 64):
        pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "bf16", r, 16.0, False, True, "qkvo", weights)
        A = oracle.bf16_to_f64(pk["A_qkv"])
        B = oracle.bf16_to_f64(pk["B_qkv"])
        outs.append(oracle.delta(x, A, B, y, [nq, nkv, nkv], R)[1])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("kw,code", [
    (dict(bias_none=False), 2),
    (dict(rank=0), 2),
    (dict(rank=17), 2),
    (dict(target_mask=16 | 1), 2),
])
def test_pack_error_paths(kw, code):
    rng = np.random.default_rng(9)
    weights = rand_adapter(rng, 17, 16, 16, 8)
    args = dict(rank=4, bias_none=True, target_mask=None)
    args.update(kw)
    r = args["rank"]
    w = {p: (a[:max(r, 1)], b[:, :max(r, 1)]) for p, (a, b) in weights.items()}
    with pytest.raises(OracleError) as e:
        oracle.pack_adapter(16, 2, 1, 8, 16, "bf16", r, 8.0, False, args["bias_none"], "qkvo", w,
                            target_mask=args["target_mask"])
    assert e.value.code == code


def test_pack_rank_equal_to_max_is_accepted():
    rng = np.random.default_rng(10)
    weights = rand_adapter(rng, 16, 16, 16, 8)
    pk = oracle.pack_adapter(16, 2, 1, 8, 16, "bf16", 16, 8.0, False, True, "qkvo", weights)
    assert pk["A_qkv"].shape == (48, 16)


# --------------------------------------------------------------------------- routing
def naive_route(slots, lengths):
    """Second, independent statement of the routing: Python's stable sorted()
    with base last, itertools.groupby, truncation at the first base group."""
    order = sorted(range(len(slots)), key=lambda i: (slots[i] == -1, slots[i]))
    ids, offs, tok = [], [0], 0
    for s, grp in itertools.groupby(order, key=lambda i: slots[i]):
        if s == -1:
            break
        grp = list(grp)
        tok += sum(lengths[i] for i in grp)
        ids.append(s)
        offs.append(tok)
    return order, ids, offs, tok


def _check_route(slots, lengths, L):
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    got = oracle.route(np.array(slots, np.int32), offsets, L)
    order, ids, offs, end = naive_route(list(slots), list(lengths))
    assert list(got["perm"]) == order
    assert list(got["lora_ids"]) == ids
    assert list(got["grouped_offsets"]) == offs
    assert got["end"] == end and got["num_groups"] == len(ids)
    # properties
    assert all(a < b for a, b in zip(ids, ids[1:]))
    assert end == sum(l for s, l in zip(slots, lengths) if s != -1)
    srt = np.concatenate([[0], np.cumsum([lengths[i] for i in order])])
    assert np.array_equal(got["sorted_offsets"], srt)
    # tokens of group g come from requests with slot ids[g]
    tok_slot = np.concatenate([[slots[i]] * lengths[i] for i in order]) if sum(lengths) else np.array([])
    for g, s in enumerate(ids):
        assert np.all(tok_slot[offs[g]:offs[g + 1]] == s)
    assert np.all(tok_slot[end:] == -1)


def test_route_tiny_hand_example():
    got = oracle.route(np.array([0, 1, -1], np.int32), np.array([0, 5, 8, 12], np.int64), 2)
    assert list(got["lora_ids"]) == [0, 1]
    assert list(got["grouped_offsets"]) == [0, 5, 8]
    assert got["end"] == 8 and list(got["perm"]) == [0, 1, 2]


@pytest.mark.parametrize("n", range(0, 7))
def test_route_brute_force(n):
    rng = np.random.default_rng(100 + n)
    for slots in itertools.product([-1, 0, 1], repeat=n):
        lengths = list(rng.integers(0, 4, size=n))
        _check_route(list(slots), lengths, 2)


def test_route_random_large():
    rng = np.random.default_rng(12)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        L = int(rng.integers(1, 40))
        slots = list(rng.integers(-1, L, size=n))
        lengths = list(rng.integers(0, 50, size=n))
        _check_route(slots, lengths, L)


@pytest.mark.parametrize("slots,offsets,code", [
    ([0, 2], [0, 1, 2], 3),        # slot == L
    ([0, -2], [0, 1, 2], 3),       # below -1
    ([0, 1], [0, 3, 2], 1),        # decreasing offsets
    ([0, 1], [1, 3, 4], 1),        # offsets must start at 0
])
def test_route_error_paths(slots, offsets, code):
    with pytest.raises(OracleError) as e:
        oracle.route(np.array(slots, np.int32), np.array(offsets, np.int64), 2)
    assert e.value.code == code


def test_route_empty_and_base_only():
    got = oracle.route(np.zeros(0, np.int32), np.zeros(1, np.int64), 4)
    assert got["num_groups"] == 0 and got["end"] == 0
    got = oracle.route(np.array([-1, -1], np.int32), np.array([0, 3, 5], np.int64), 4)
    assert got["num_groups"] == 0 and got["end"] == 0 and list(got["grouped_offsets"]) == [0]


# --------------------------------------------------------------------------- forward
def test_delta_dense_special_case_matches_numpy():
    """One slice, any sizes: y + (x A^T) B^T by numpy matmul."""
    rng = np.random.default_rng(13)
    for n, fin, R, w in [(1, 7, 3, 5), (9, 40, 16, 33), (33, 128, 64, 100)]:
        x = rng.standard_normal((n, fin))
        A = rng.standard_normal((R, fin))
        B = rng.standard_normal((w, R))
        y = rng.standard_normal((n, w))
        u, yo = oracle.delta(x, A, B, y, [w], R)
        np.testing.assert_allclose(u, x @ A.T, rtol=1e-13, atol=1e-12)
        np.testing.assert_allclose(yo, y + (x @ A.T) @ B.T, rtol=1e-13, atol=1e-12)


def test_delta_fused_equals_unfused():
    """Three slices in one call equal three separate one-slice calls."""
    rng = np.random.default_rng(14)
    R, fin, widths, n = 8, 24, [16, 8, 8], 6
    A = rng.standard_normal((3 * R, fin))
    B = rng.standard_normal((sum(widths), R))
    x = rng.standard_normal((n, fin))
    y = rng.standard_normal((n, sum(widths)))
    u, yf = oracle.delta(x, A, B, y, widths, R)
    off = 0
    for s, w in enumerate(widths):
        us, ys = oracle.delta(x, A[s * R:(s + 1) * R], B[off:off + w], y[:, off:off + w], [w], R)
        assert np.array_equal(ys, yf[:, off:off + w])
        assert np.array_equal(us, u[:, s * R:(s + 1) * R])
        off += w


def test_delta_identity_with_base_weight():
    """W0 x + B (A x) == (W0 + B A) x."""
    rng = np.random.default_rng(15)
    n, fin, R, w = 4, 32, 8, 20
    W0 = rng.standard_normal((w, fin))
    A = rng.standard_normal((R, fin))
    B = rng.standard_normal((w, R))
    x = rng.standard_normal((n, fin))
    _, h = oracle.delta(x, A, B, x @ W0.T, [w], R)
    np.testing.assert_allclose(h, x @ (W0 + B @ A).T, rtol=1e-12, atol=1e-12)


def test_delta_zero_B_leaves_y_bitwise():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((5, 16))
    A = rng.standard_normal((8, 16))
    y = rng.standard_normal((5, 24))
    _, yo = oracle.delta(x, A, np.zeros((24, 8)), y, [24], 8)
    assert np.array_equal(yo, y)


def test_scaling_is_linear_in_the_delta():
    rng = np.random.default_rng(17)
    r, R, H, nh, nkv_h, hd = 8, 8, 16, 2, 1, 8
    nq, nkv = nh * hd, nkv_h * hd
    weights = rand_adapter(rng, r, H, nq, nkv)
    x = rng.standard_normal((3, H))
    y = np.zeros((3, nq + 2 * nkv))
    ds = []
    for alpha, rs in ((8.0, False), (32.0, False), (16.0, True)):
        pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "f32", r, alpha, rs, True, "qkvo", weights)
        ds.append(oracle.delta(x, pk["A_qkv"], pk["B_qkv"], y, [nq, nkv, nkv], R)[1])
    # scales 1, 4 and 16/sqrt(8) = 4 sqrt(2)
    np.testing.assert_allclose(ds[1], 4.0 * ds[0], rtol=1e-14, atol=1e-14)
    # fp32 scale and fp32 products: each term carries <= 2^-23 relative error
    want = 4.0 * math.sqrt(2.0) * ds[0]
    assert np.abs(ds[2] - want).max() <= 2.0 ** -20 * np.abs(want).max()


def test_reference_family_base_rows_untouched_and_lora_rows_moved():
    import synth
    w = synth.get_workload("tiny")
    lengths, slots = synth.draw_requests(w)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    ranks = synth.draw_ranks(w)
    A, B = [], []
    for s in range(w.max_num_loras):
        pk = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                                 w.dtype, int(ranks[s]), w.lora_alpha, w.use_rslora, True, "qkvo",
                                 synth.draw_adapter(w, 0, s, int(ranks[s])))
        A.append(pk["A_qkv"])
        B.append(pk["B_qkv"])
    act = synth.draw_activations(w, 0, int(offs[-1]))
    res = oracle.reference_family(act["x_qkv"], act["y_qkv"], offs, slots, np.stack(A), np.stack(B),
                                  [w.nq, w.nkv, w.nkv], w.max_lora_rank, w.dtype)
    for i, (rows, y, u) in res.items():
        yin = act["y_qkv"][offs[i]:offs[i + 1]].astype(np.float64)
        if slots[i] < 0:
            assert u is None and np.array_equal(y, yin)
        else:
            assert not np.allclose(y, yin)


def test_memory_formula_matches_stack_sizes():
    """The stacks hold exactly the page's per-layer memory formula summed over
    q/k/v/o; at the page's example factors that is 134217728 bytes."""
    g = golden("vllm_memory_example.json")
    p = g["printed_by_page"]
    formula = lambda layers, fin, fout, r, b, L: layers * (fin * r + fout * r) * b * L
    assert formula(p["num_lora_layers"], p["in_features"], p["out_features"], p["rank"],
                   p["dtype_bytes"], p["max_loras"]) == g["derived_expectation"]["formula_bytes"]
    # packed stacks of one adapter vs the formula over q, k, v, o
    H, nh, nkv_h, hd, R = 32, 4, 2, 8, 16
    nq, nkv = nh * hd, nkv_h * hd
    rng = np.random.default_rng(18)
    pk = oracle.pack_adapter(H, nh, nkv_h, hd, R, "bf16", 4, 8.0, False, True, "qkvo",
                             rand_adapter(rng, 4, H, nq, nkv))
    packed = sum(a.nbytes for a in pk.values())
    want = sum(formula(1, fi, fo, R, 2, 1) for fi, fo in ((H, nq), (H, nkv), (H, nkv), (nq, H)))
    assert packed == want


def test_delta_batch_composition_invariant_brute_force():
    """A request's result does not depend on the rest of its batch: on the
    tiny attention workload (5/3/4 tokens routed to slots 0, 1 and base) and on
    a five-request variant that repeats slots and adds an empty request, every
    non-empty subset of the requests, in every arrival order, gives each
    request bit-for-bit the y and u it gets in the whole batch (the routing
    sorts, groups and truncates per batch; the result must not see that)."""
    import synth
    w = synth.get_workload("tiny")
    ranks = synth.draw_ranks(w)
    A, B = [], []
    for s in range(w.max_num_loras):
        pk = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                                 w.dtype, int(ranks[s]), w.lora_alpha, w.use_rslora, True, "qkvo",
                                 synth.draw_adapter(w, 0, s, int(ranks[s])))
        A.append(pk["A_qkv"])
        B.append(pk["B_qkv"])
    A, B = np.stack(A), np.stack(B)
    widths = [w.nq, w.nkv, w.nkv]
    lengths0, slots0 = synth.draw_requests(w)
    cases = [(np.asarray(lengths0, np.int64), np.asarray(slots0, np.int32)),
             (np.array([2, 0, 3, 1, 4], np.int64), np.array([1, 0, -1, 1, 0], np.int32))]
    for lengths, slots in cases:
        offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        act = synth.draw_activations(w, 1, int(offs[-1]))
        full = oracle.reference_family(act["x_qkv"], act["y_qkv"], offs, slots, A, B, widths,
                                       w.max_lora_rank, w.dtype)
        n = len(lengths)
        for k in range(1, n + 1):
            for sub in itertools.permutations(range(n), k):
                sl = np.array([slots[i] for i in sub], np.int32)
                ln = np.array([lengths[i] for i in sub], np.int64)
                so = np.concatenate([[0], np.cumsum(ln)]).astype(np.int64)
                rows = np.concatenate([np.arange(offs[i], offs[i + 1]) for i in sub]).astype(np.int64)
                part = oracle.reference_family(act["x_qkv"][rows], act["y_qkv"][rows], so, sl, A, B,
                                               widths, w.max_lora_rank, w.dtype)
                for j, i in enumerate(sub):
                    r_sub, y_sub, u_sub = part[j]
                    r_all, y_all, u_all = full[i]
                    assert np.array_equal(r_sub, r_all)
                    assert np.array_equal(y_sub.view(np.int64), y_all.view(np.int64)), (sub, i)
                    if u_all is None:
                        assert u_sub is None
                    else:
                        assert np.array_equal(u_sub.view(np.int64), u_all.view(np.int64)), (sub, i)
