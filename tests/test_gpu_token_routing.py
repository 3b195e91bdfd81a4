"""GPU parity under per-token routing: x and y stay in the caller's token
order, a slot per token (lora_build_token_routing), and the kernels gather x
rows and scatter y rows through the sorted token indices.  Checked against
the oracle token by token (one request per token): LoRA tokens within the
bar, tokens without a slot and rows past the tokens bit-identical.

Cases: the decode batch (slots interleaved), the prefill and mixed batches
(token runs, and the same tokens shuffled so that every group is scattered
over the batch), the fp32 tiny case, ragged shuffled segments on every path
and rank, with a LoRA bias, with padded strided buffers, and with the
routing read from the device arrays only; argument errors."""

import numpy as np
import pytest

import synth
import segmented_rank_gemv_amd as srg
from lora_case import TOL, from_dev, log, oracle_layer, pack_bias_stacks, pack_stacks, rel_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PATHS = {"auto": srg.PATH_AUTO, "valu": srg.PATH_VALU, "mfma": srg.PATH_MFMA, "fused": srg.PATH_FUSED}
FAMS = ((srg.FAMILY_QKV, "x_qkv", "y_qkv", "A_qkv", "B_qkv", "bias_qkv"),
        (srg.FAMILY_O, "x_o", "y_o", "A_o", "B_o", "bias_o"))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dims_of(w):
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.max_num_loras, w.dtype)


def run_tokens(w, stacks, token_slot, acts, path, api, routing="host", bias=None, pad_rows=0, pad_cols=0,
               options=None):
    """Runs both families with per-token routing; returns y of both families
    in token order (with the padding rows) and the routing."""
    d = dims_of(w)
    T = len(token_slot)
    rt = srg.lora_build_token_routing(token_slot, w.max_num_loras)
    r = srg.LoraRouting.from_host(rt, host_copy=routing == "host")
    r.num_rows = T + pad_rows
    st = {k: to_dev(v, w.dtype) for k, v in stacks.items() if k != "ref"}
    bs = None if bias is None else {k: to_dev(v, w.dtype) for k, v in bias.items() if k != "ref"}
    out = {}
    for fam, xk, yk, ak, bk, bik in FAMS:
        fin, n_s, widths, fout = srg.lora_family_shape(d, fam)
        bufs = {}
        for key, width in ((xk, fin), (yk, fout)):
            host = np.full((T + pad_rows, width + pad_cols), 7.0, np.float32)
            host[:T, :width] = acts[key]
            full = to_dev(host, w.dtype)
            bufs[key] = (full[:, :width] if pad_cols else full, full)
        x, y = bufs[xk][0], bufs[yk][0]
        end = rt["end"]
        ws = torch.full((max(srg.lora_sgmv_workspace_bytes(d, fam, max(end, 1)), 16) // 4 + 4,), -1,
                        dtype=torch.int32, device="cuda")
        b = None if bs is None else bs[bik]
        log(f"  tokens family={fam} path={path} api={api} routing={routing} T={T} end={end} "
            f"G={rt['num_groups']} bias={b is not None} pad={pad_rows},{pad_cols}")
        if api == "delta":
            srg.lora_sgmv_delta(d, fam, x, st[ak], st[bk], r, y, ws, PATHS[path], bias=b, options=options)
        else:
            u = torch.full((max(end, 1), n_s * w.max_lora_rank), float("nan"), dtype=torch.float32,
                           device="cuda")
            srg.lora_sgmv_shrink(d, fam, x, st[ak], r, u, ws, PATHS[path])
            srg.lora_sgmv_expand(d, fam, u, st[bk], r, y, PATHS[path], bias=b)
        out[yk] = bufs[yk][1]
    torch.cuda.synchronize()
    return {k: from_dev(v) for k, v in out.items()}, rt


def check(w, stacks, token_slot, acts, ys, bias=None, pad_rows=0, pad_cols=0):
    T = len(token_slot)
    ref = oracle_layer(w, stacks, np.ones(T, np.int64), np.asarray(token_slot, np.int32), acts, bias=bias)
    worst = 0.0
    for fam, xk, yk, *_ in FAMS:
        y = ys[yk]
        width = acts[yk].shape[1]
        got, want = [], []
        for i, (rows, yref, uref) in ref[fam].items():
            g = y[i + rows, :width]
            if uref is None:
                assert np.array_equal(g.astype(np.float64), yref), f"token {i} without a slot changed"
                continue
            got.append(g)
            want.append(yref)
        if got:
            worst = max(worst, rel_err(np.concatenate(got), np.concatenate(want)))
        if pad_rows:
            assert np.all(y[T:] == 7.0), "rows past the tokens changed"
        if pad_cols:
            assert np.all(y[:, width:] == 7.0), "columns past the row changed"
    return worst


def token_case(name, shuffle):
    w = synth.get_workload(name)
    lengths, slots = synth.draw_requests(w)
    token_slot = np.repeat(slots, lengths).astype(np.int32)
    if shuffle:
        token_slot = token_slot[np.random.default_rng(11).permutation(len(token_slot))]
    stacks = pack_stacks(w, 0, synth.draw_ranks(w))
    acts = synth.draw_activations(w, 0, len(token_slot))
    return w, token_slot, stacks, acts


def fused_applies(w):
    return w.dtype == "bf16" and w.max_lora_rank in (16, 32)


@pytest.mark.parametrize("api", ["split", "delta"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name,shuffle", [("tiny", True), ("decode", False), ("prefill", False),
                                          ("prefill", True), ("mixed", True)])
def test_token_routing_full_workloads(name, shuffle, path, api):
    w, token_slot, stacks, acts = token_case(name, shuffle)
    if path == "mfma" and w.dtype != "bf16":
        pytest.skip("MFMA path is bf16 only")
    if path == "fused" and (api != "delta" or not fused_applies(w)):
        pytest.skip("the one-kernel path is lora_sgmv_delta's, for bf16 and rank 16 or 32")
    log(f"[tokens] workload={name} shuffle={shuffle} path={path} api={api} T={len(token_slot)}")
    ys, rt = run_tokens(w, stacks, token_slot, acts, path, api)
    ey = check(w, stacks, token_slot, acts, ys)
    log(f"[tokens] workload={name} shuffle={shuffle} path={path} api={api} y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]


def small_bf16(R, L=8):
    base = synth.get_workload("decode")
    return synth.Workload(**{**base.__dict__, "hidden": 512, "n_heads": 4, "n_kv_heads": 2,
                             "head_dim": 128, "max_lora_rank": R, "max_num_loras": L})


@pytest.mark.parametrize("routing", ["host", "device"])
@pytest.mark.parametrize("api", ["split", "delta"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("R", [8, 16, 32, 48, 64])
def test_token_routing_ragged_shuffled(R, path, api, routing):
    """Group sizes around the tile size, tokens shuffled, a LoRA bias, padded
    rows and columns (strided x and y); every path and rank."""
    w = small_bf16(R)
    if path == "mfma" and R % 16:
        pytest.skip("the MFMA path needs a rank that is a multiple of 16 (rejected otherwise)")
    if path == "fused" and (api != "delta" or not fused_applies(w)):
        pytest.skip("the one-kernel path is lora_sgmv_delta's, for bf16 and rank 16 or 32")
    lengths = ([1, 15, 16, 17, 32, 3, 20] if path == "fused"
               else [1, 15, 16, 17, 63, 64, 65, 127, 129, 3, 200])
    slots = [0, 1, 2, 3, 4, -1, 5, 6, 7, -1, 1][:len(lengths)]
    token_slot = np.repeat(np.array(slots, np.int32), lengths)
    token_slot = token_slot[np.random.default_rng(R).permutation(len(token_slot))]
    ranks = np.array([min(R, r) for r in (8, 8, 4, 8, 8, 2, 8, 8)], np.int32)
    stacks = pack_stacks(w, 0, ranks)
    bias = pack_bias_stacks(w, 0)
    acts = synth.draw_activations(w, 0, len(token_slot))
    log(f"[tokens-ragged] R={R} path={path} api={api} routing={routing}")
    ys, _ = run_tokens(w, stacks, token_slot, acts, path, api, routing, bias=bias, pad_rows=5, pad_cols=8)
    ey = check(w, stacks, token_slot, acts, ys, bias=bias, pad_rows=5, pad_cols=8)
    log(f"[tokens-ragged] R={R} path={path} api={api} routing={routing} y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]


def test_token_routing_equals_sorted_layout():
    """The same batch through per-token routing and through the sorted
    layout (the caller reorders x and y) gives bit-identical y: the gather
    changes where rows live, not the arithmetic."""
    w, token_slot, stacks, acts = token_case("decode", False)
    ys_tok, rt = run_tokens(w, stacks, token_slot, acts, "auto", "delta")
    order = rt["token_indices_sorted"]
    d = dims_of(w)
    r = srg.LoraRouting.from_host({k: rt[k] for k in ("lora_ids", "grouped_offsets", "num_groups", "end")})
    st = {k: to_dev(v, w.dtype) for k, v in stacks.items() if k != "ref"}
    for fam, xk, yk, ak, bk, _ in FAMS:
        x = to_dev(acts[xk][order], w.dtype)
        y = to_dev(acts[yk][order], w.dtype)
        ws = torch.zeros(max(srg.lora_sgmv_workspace_bytes(d, fam, rt["end"]), 16) // 4 + 4, dtype=torch.int32,
                         device="cuda")
        srg.lora_sgmv_delta(d, fam, x, st[ak], st[bk], r, y, ws, srg.PATH_AUTO)
        torch.cuda.synchronize()
        got = from_dev(y)
        back = np.empty_like(got)
        back[order] = got
        assert np.array_equal(back, ys_tok[yk]), fam


def test_token_routing_argument_errors():
    w = small_bf16(16)
    d = dims_of(w)
    token_slot = np.array([0, 1, -1, 0], np.int32)
    rt = srg.lora_build_token_routing(token_slot, w.max_num_loras)
    stacks = pack_stacks(w, 0, np.full(w.max_num_loras, 8, np.int32))
    st = {k: to_dev(v, w.dtype) for k, v in stacks.items() if k != "ref"}
    x = torch.zeros((4, w.hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((4, w.n_qkv), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    # fewer rows than LoRA tokens
    r = srg.LoraRouting.from_host(rt)
    r.num_rows = 2
    with pytest.raises(ValueError):
        srg.lora_sgmv_delta(d, srg.FAMILY_QKV, x, st["A_qkv"], st["B_qkv"], r, y, ws)
    # a row count whose byte offsets do not fit 32 bits (checked before any launch)
    r.num_rows = (1 << 31) - 1
    with pytest.raises(ValueError):
        srg.lora_sgmv_delta(d, srg.FAMILY_QKV, x, st["A_qkv"], st["B_qkv"], r, y, ws)
    torch.cuda.synchronize()
    assert not from_dev(y).any()
