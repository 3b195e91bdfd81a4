"""MLP targets on the GPU: the gate_up (two slices of the intermediate width)
and down families through the same kernels, against the oracle, request by
request: the Llama-3-8B MLP decode batch (hidden 4096, intermediate 14336)
and a small ragged case on every path."""

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg
from lora_case import TOL, from_dev, log, rel_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")

PATHS = {"auto": srg.PATH_AUTO, "valu": srg.PATH_VALU, "mfma": srg.PATH_MFMA, "fused": srg.PATH_FUSED}


def mdims(w):
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.max_num_loras,
                        w.dtype, w.intermediate)


def run_family(w, fam, lengths, slots, ranks, path, fused, layer=0, with_bias=False, options=None):
    import torch
    d = mdims(w)
    in_f, n_s, widths, out_f = srg.lora_family_shape(d, fam)
    names = ("gate", "up") if fam == srg.FAMILY_GATE_UP else ("down",)
    xk, yk = ("x_gu", "y_gu") if fam == srg.FAMILY_GATE_UP else ("x_down", "y_down")
    A, B, Ar, Br, bl, br = [], [], [], [], [], []
    for s in range(w.max_num_loras):
        weights = synth.draw_mlp_adapter(w, layer, s, int(ranks[s]))
        sl = [weights[p] for p in names]
        lib = srg.lora_pack_family(d, fam, int(ranks[s]), w.lora_alpha, w.use_rslora, True, sl)
        orc = oracle.pack_family(in_f, widths, w.max_lora_rank, w.dtype, int(ranks[s]), w.lora_alpha,
                                 w.use_rslora, True, sl)
        A.append(lib["A"]), B.append(lib["B"]), Ar.append(orc["A"]), Br.append(orc["B"])
        if with_bias:
            bias = synth.draw_bias(w, layer, s, names)
            bsl = [bias[p] for p in names]
            bl.append(srg.lora_pack_bias(d, fam, bsl))
            br.append(oracle.pack_bias(widths, w.dtype, bsl))
    lengths = np.asarray(lengths, np.int64)
    slots = np.asarray(slots, np.int32)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    acts = synth.draw_mlp_activations(w, layer, T)
    rt = srg.lora_build_routing(slots, offs, w.max_num_loras)
    order = (np.concatenate([np.arange(offs[p], offs[p + 1]) for p in rt["perm"]])
             if len(rt["perm"]) else np.zeros(0, np.int64)).astype(np.int64)
    x = to_dev(acts[xk][order], w.dtype)
    y = to_dev(acts[yk][order], w.dtype)
    end = rt["end"]
    ws = torch.full((max(srg.lora_sgmv_workspace_bytes(d, fam, max(end, 1)), 16) // 4 + 4,), -1,
                    dtype=torch.int32, device="cuda")
    routing = srg.LoraRouting.from_host(rt)
    As, Bs = to_dev(np.stack(A), w.dtype), to_dev(np.stack(B), w.dtype)
    bs = to_dev(np.stack(bl), w.dtype) if with_bias else None
    log(f"  mlp family={fam} path={path} fused={fused} T={T} end={end} G={rt['num_groups']} bias={with_bias}")
    if fused:
        srg.lora_sgmv_delta(d, fam, x, As, Bs, routing, y, ws, PATHS[path], bias=bs, options=options)
    else:
        u = torch.zeros((max(end, 1), n_s * w.max_lora_rank), dtype=torch.float32, device="cuda")
        srg.lora_sgmv_shrink(d, fam, x, As, routing, u, ws, PATHS[path])
        srg.lora_sgmv_expand(d, fam, u, Bs, routing, y, PATHS[path], bias=bs)
    torch.cuda.synchronize()
    ys = from_dev(y)
    got = np.empty_like(ys[:T])
    got[order] = ys[:T]
    ref = oracle.reference_family(acts[xk], acts[yk], offs, slots, np.stack(Ar), np.stack(Br), list(widths),
                                  w.max_lora_rank, w.dtype, bias_stack=np.stack(br) if with_bias else None)
    g_all, r_all = [], []
    for i, (rows, yref, uref) in ref.items():
        g = got[int(offs[i]) + rows]
        if uref is None:
            assert np.array_equal(g.astype(np.float64), yref), f"base request {i} changed"
            continue
        g_all.append(g)
        r_all.append(yref)
    return rel_err(np.concatenate(g_all), np.concatenate(r_all)) if g_all else 0.0


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_llama8b_mlp_decode_batch(fam, fused):
    w = synth.get_workload("mlp")
    lengths, slots = synth.draw_requests(w)
    ey = run_family(w, fam, lengths, slots, synth.draw_ranks(w), "auto", fused)
    log(f"[mlp] family={fam} fused={fused} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_small_mlp_ragged_every_path(fam, path):
    base = synth.get_workload("mlp")
    w = synth.Workload(**{**base.__dict__, "hidden": 256, "n_heads": 4, "n_kv_heads": 2, "head_dim": 64,
                          "intermediate": 704, "max_num_loras": 4})
    lengths = [1, 15, 16, 33, 64, 65, 3, 0, 20] if path != "fused" else [1, 15, 16, 17, 32, 3, 0, 20]
    slots = [0, 1, 2, 3, 0, 1, -1, 2, 3][:len(lengths)]
    ey = run_family(w, fam, lengths, slots, np.array([16, 8, 4, 12], np.int32), path, path == "fused")
    log(f"[mlp-small] family={fam} path={path} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("path", ["auto", "valu", "mfma"])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_mlp_with_lora_bias(fam, fused, path):
    """The MLP families with a LoRA bias per slot: the Llama-3-8B MLP decode
    batch (auto) and the small ragged case (VALU, MFMA)."""
    if path == "auto":
        w = synth.get_workload("mlp")
        lengths, slots = synth.draw_requests(w)
        ranks = synth.draw_ranks(w)
    else:
        base = synth.get_workload("mlp")
        w = synth.Workload(**{**base.__dict__, "hidden": 256, "n_heads": 4, "n_kv_heads": 2, "head_dim": 64,
                              "intermediate": 704, "max_num_loras": 4})
        lengths = [1, 15, 16, 33, 64, 65, 3, 0, 20]
        slots = [0, 1, 2, 3, 0, 1, -1, 2, 3]
        ranks = np.array([16, 8, 4, 12], np.int32)
    ey = run_family(w, fam, lengths, slots, ranks, path, fused, with_bias=True)
    log(f"[mlp-bias] family={fam} fused={fused} path={path} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_split_k_short_wide_and_long(fam):
    """The split-K delta for short groups at shapes past its tables: an
    intermediate width of 36 864 makes gate_up 73 728 features wide, more
    than 64 feature tiles of 1024, so its expand half falls back to the
    64-row expand kernel on the same slabs; down then has K = 36 864, split
    into at most 16 K ranges of 8 steps per wave."""
    base = synth.get_workload("mlp")
    w = synth.Workload(**{**base.__dict__, "intermediate": 36864, "max_num_loras": 4})
    # every group at most 32 tokens (slot 0: 1 + 30, slot 1: 24, slot 2: 16, slot 3: 0 + 3)
    lengths = np.array([1, 24, 16, 0, 9, 30, 3], np.int64)
    slots = np.array([0, 1, 2, 3, -1, 0, 3], np.int32)
    ey = run_family(w, fam, lengths, slots, np.full(w.max_num_loras, 16, np.int32), "auto", True,
                    options=srg.LoraOptions(splitk_short=1))
    log(f"[mlp] wide/long family={fam} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]
